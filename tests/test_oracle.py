"""Pins for the fp64 oracle: library routines, closed forms, finite differences
and structural invariants.  None of these retypes the oracle's own formulas."""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import (Params, backward, cap_derivative, cap_forward, dkv_keys, dq_rows, forward,
                    ranker_bounds_from_segments, sigmoid, unmasked_pairs, visible)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")

CAPS = [("none", 0.0, 0.0, 0.0), ("tanh", 3.0, 0.0, 0.0), ("soft_sign", 2.0, 0.0, 0.0),
        ("alsc", 3.0, 4.0, 0.5), ("alsc", 5.0, 2.0, 0.0)]


def rnd(rng, *shape):
    return rng.standard_normal(shape)


# ---------------------------------------------------------------------------
# Cap functions: closed forms, limits, symmetry, finite differences
# ---------------------------------------------------------------------------

def test_sigmoid_matches_library_logistic():
    x = np.linspace(-800, 800, 4001)
    ref = torch.sigmoid(torch.from_numpy(x)).numpy()
    assert np.allclose(sigmoid(x), ref, rtol=1e-15, atol=1e-300)


@pytest.mark.parametrize("method", ["none", "tanh", "soft_sign", "alsc"])
def test_cap_nonpositive_cap_is_identity(method):
    s = np.linspace(-40, 40, 81)
    for cap in (0.0, -1.0):
        assert np.array_equal(cap_forward(s, method, cap, 4.0, 0.5), s)
        assert np.array_equal(cap_derivative(s, method, cap, 4.0, 0.5), np.ones_like(s))


def test_cap_unknown_method_raises():
    with pytest.raises(ValueError):
        cap_forward(np.zeros(3), "hard", 1.0)
    with pytest.raises(ValueError):
        cap_derivative(np.zeros(3), "hard", 1.0)


def test_cap_closed_form_points():
    # tanh: value cap*tanh(1) at s = cap, limits +-cap, odd
    assert cap_forward(np.array([30.0]), "tanh", 30.0)[0] == pytest.approx(30 * 0.7615941559557649,
                                                                            rel=1e-15)
    assert cap_forward(np.array([1e9, -1e9]), "tanh", 30.0) == pytest.approx([30.0, -30.0])
    # soft-sign: s = cap gives cap/2; limits +-cap; s = -cap gives -cap/2
    assert cap_forward(np.array([20.0, -20.0]), "soft_sign", 20.0) == pytest.approx([10.0, -10.0],
                                                                                    rel=1e-15)
    assert cap_forward(np.array([1e12]), "soft_sign", 20.0)[0] == pytest.approx(20.0, rel=1e-9)


@pytest.mark.parametrize("cap,alpha,beta", [(30.0, 4.0, 0.5), (50.0, 2.0, 0.0), (20.0, 1.0, -1.0)])
def test_alsc_zero_limits_and_slope(cap, alpha, beta):
    sb = 1.0 / (1.0 + math.exp(-alpha * beta))
    denom = sb * (1 - sb) + 1e-12
    # zero at zero
    assert abs(cap_forward(np.array([0.0]), "alsc", cap, alpha, beta)[0]) < 1e-12
    # limits: sig -> 1 and sig -> 0
    hi = cap_forward(np.array([1e6]), "alsc", cap, alpha, beta)[0]
    lo = cap_forward(np.array([-1e6]), "alsc", cap, alpha, beta)[0]
    assert hi == pytest.approx(cap * (1 - sb) / denom, rel=1e-12)
    assert lo == pytest.approx(-cap * sb / denom, rel=1e-12)
    # slope at zero: alpha * sig'(alpha beta) / (sig'(alpha beta) + 1e-12) ~ alpha
    slope = cap_derivative(np.array([0.0]), "alsc", cap, alpha, beta)[0]
    assert slope == pytest.approx(alpha * (sb * (1 - sb)) / denom, rel=1e-12)


def test_alsc_limits_of_the_workloads():
    # (30, 4, 0.5): +34.06 / -251.67 ; (50, 2, 0): +-100
    assert cap_forward(np.array([1e6, -1e6]), "alsc", 30.0, 4.0, 0.5) == pytest.approx(
        [34.06006, -251.67168], abs=1e-4)
    assert cap_forward(np.array([1e6, -1e6]), "alsc", 50.0, 2.0, 0.0) == pytest.approx(
        [100.0, -100.0], rel=1e-9)


@pytest.mark.parametrize("method,cap,alpha,beta", [("tanh", 30.0, 0, 0), ("soft_sign", 20.0, 0, 0),
                                                   ("alsc", 50.0, 2.0, 0.0)])
def test_cap_odd_where_formula_implies(method, cap, alpha, beta):
    s = np.linspace(-200, 200, 801)
    assert np.allclose(cap_forward(s, method, cap, alpha, beta),
                       -cap_forward(-s, method, cap, alpha, beta), rtol=0, atol=1e-12)


def test_alsc_with_beta_is_not_odd():
    s = np.array([5.0])
    a = cap_forward(s, "alsc", 30.0, 4.0, 0.5)[0]
    b = cap_forward(-s, "alsc", 30.0, 4.0, 0.5)[0]
    assert abs(a + b) > 1e-3


@pytest.mark.parametrize("method,cap,alpha,beta", CAPS + [("tanh", 50.0, 0, 0),
                                                          ("alsc", 30.0, 4.0, 0.5)])
def test_cap_derivative_matches_central_differences(method, cap, alpha, beta):
    s = np.linspace(-60, 60, 241) + 0.013
    h = 1e-5   # roundoff ~ |f| 1e-16 / h with |f| up to ~250; truncation ~ f''' h^2 / 6
    fd = (cap_forward(s + h, method, cap, alpha, beta) - cap_forward(s - h, method, cap, alpha, beta)) / (2 * h)
    an = cap_derivative(s, method, cap, alpha, beta)
    assert np.allclose(an, fd, rtol=1e-7, atol=1e-8)


def test_cap_slope_at_zero_is_one_for_tanh_and_softsign():
    for m, c in (("tanh", 30.0), ("soft_sign", 20.0)):
        assert cap_derivative(np.array([0.0]), m, c)[0] == 1.0


# ---------------------------------------------------------------------------
# Visibility predicates: counts with closed forms
# ---------------------------------------------------------------------------

def test_pair_counts_closed_forms():
    L = 300
    assert unmasked_pairs(L, Params(1.0, causal=True)) == L * (L + 1) // 2
    W = 37
    assert unmasked_pairs(L, Params(1.0, causal=True, window_len=W)) == W * (W + 1) // 2 + (L - W) * W
    h = 170
    rb = np.array([[0, h, h, L]])
    assert unmasked_pairs(L, Params(1.0), ranker_bounds=rb) == L * h + (L - h)
    assert unmasked_pairs(L, Params(1.0)) == L * L


def test_window_rule_literal_noncausal():
    # without causality the literal rule j > i - W leaves every future key visible
    vis = visible(np.arange(10), 10, Params(1.0, window_len=3))
    assert vis[5].tolist() == [False] * 3 + [True] * 7


# ---------------------------------------------------------------------------
# Library routine: scaled_dot_product_attention in fp64 (cap none, w = 0)
# ---------------------------------------------------------------------------

def sdpa_reference(q, k, v, do, mask_bhll, sm_scale, temp=None):
    """O and grads via torch SDPA (fp64, CPU) with an explicit boolean mask.
    q (B,L,Hq,D); k, v (B,L,Hkv,D); mask (B, L, L) shared by heads."""
    B, L, Hq, D = q.shape
    G = Hq // k.shape[2]
    tq = torch.tensor(q, requires_grad=True)
    tk = torch.tensor(k, requires_grad=True)
    tv = torch.tensor(v, requires_grad=True)
    qq = tq if temp is None else tq * torch.tensor(temp)[:, :, None, None]
    qh = qq.permute(0, 2, 1, 3)
    kh = tk.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    vh = tv.repeat_interleave(G, dim=2).permute(0, 2, 1, 3)
    mask = torch.tensor(mask_bhll)[:, None, :, :]
    o = F.scaled_dot_product_attention(qh, kh, vh, attn_mask=mask, scale=sm_scale)
    o = o.permute(0, 2, 1, 3)
    (o * torch.tensor(do)).sum().backward()
    return o.detach().numpy(), tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def full_mask(B, L, p, seg=None, rb=None):
    return np.stack([visible(np.arange(L), L, p, None if seg is None else seg[b],
                             None if rb is None else rb[b]) for b in range(B)])


@pytest.mark.parametrize("case", ["dense", "causal", "window", "segments", "ranker", "gqa_causal",
                                  "temperature"])
def test_against_sdpa(case):
    rng = np.random.default_rng(7)
    B, L, Hq, Hkv, D = 2, 40, 4, 4, 16
    seg = rb = temp = None
    p = Params(0.3)
    if case == "causal":
        p = Params(0.3, causal=True)
    elif case == "window":
        p = Params(0.3, causal=True, window_len=7)
    elif case == "segments":
        p = Params(0.3, causal=True)
        seg = np.repeat(np.array([[0] * 13 + [1] * 20 + [2] * 7]), B, axis=0)
    elif case == "ranker":
        rb = np.array([[0, 25, 25, 40], [0, 17, 17, 40]])
    elif case == "gqa_causal":
        Hkv = 2
        p = Params(0.3, causal=True)
    elif case == "temperature":
        p = Params(0.3, causal=True)
        temp = rng.uniform(0.5, 1.5, size=(B, L))
    q, do = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    k, v = rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    o_ref, dq_ref, dk_ref, dv_ref = sdpa_reference(q, k, v, do, full_mask(B, L, p, seg, rb),
                                                   p.sm_scale, temp)
    res = backward(q, k, v, do, p, temp, seg, rb)
    assert np.allclose(res["o"], o_ref, atol=1e-12)
    assert np.allclose(res["dq"], dq_ref, atol=1e-11)
    assert np.allclose(res["dk"], dk_ref, atol=1e-11)
    assert np.allclose(res["dv"], dv_ref, atol=1e-11)
    # m and l against library max / logsumexp of the masked logits
    G = Hq // Hkv
    mask = full_mask(B, L, p, seg, rb)
    for b in range(B):
        for h in range(Hq):
            t = np.ones(L) if temp is None else temp[b]
            s = t[:, None] * p.sm_scale * (q[b, :, h] @ k[b, :, h // G].T)
            s = torch.tensor(np.where(mask[b], s, -np.inf))
            assert np.allclose(res["m"][b, h], torch.amax(s, dim=1).numpy(), atol=1e-13)
            lse = res["m"][b, h] + np.log(res["l"][b, h])
            assert np.allclose(lse, torch.logsumexp(s, dim=1).numpy(), atol=1e-12)


# ---------------------------------------------------------------------------
# Finite differences of the objective F = sum O*dO + (w/2) sum LSE^2
# ---------------------------------------------------------------------------

def objective(q, k, v, do, p, temp, seg, rb):
    o, m, l = forward(q, k, v, p, temp, seg, rb)
    ok = np.isfinite(m)
    lse = np.where(ok, m + np.log(np.where(ok, l, 1.0)), 0.0)
    return float(np.sum(o * do) + 0.5 * p.z_loss_weight * np.sum(lse * lse))


def fd_check(q, k, v, do, p, temp, seg, rb, n_samples=60, seed=0, rtol=2e-6, eps=1e-6):
    res = backward(q, k, v, do, p, temp, seg, rb)
    rng = np.random.default_rng(seed)
    scale = max(np.abs(res[n]).max() for n in ("dq", "dk", "dv"))
    pairs = [("dq", q), ("dk", k), ("dv", v)]
    if temp is not None:
        pairs.append(("dtemp", temp))
    for name, arr in pairs:
        flat = arr.reshape(-1)
        idx = rng.choice(flat.size, size=min(n_samples, flat.size), replace=False)
        for t in idx:
            old = flat[t]
            flat[t] = old + eps
            fp = objective(q, k, v, do, p, temp, seg, rb)
            flat[t] = old - eps
            fm = objective(q, k, v, do, p, temp, seg, rb)
            flat[t] = old
            fd = (fp - fm) / (2 * eps)
            an = res[name].reshape(-1)[t]
            sc = scale if name != "dtemp" else max(scale, np.abs(res["dtemp"]).max())
            assert abs(fd - an) <= rtol * sc + 1e-7 * abs(fd), (name, t, fd, an)


@pytest.mark.parametrize("cap", CAPS)
def test_backward_finite_differences_all_features(cap):
    method, c, a, bt = cap
    rng = np.random.default_rng(11)
    B, L, Hq, Hkv, D = 2, 12, 4, 2, 8
    q, do = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    k, v = rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    temp = rng.uniform(0.5, 1.5, size=(B, L))
    seg = rng.integers(0, 2, size=(B, L)).astype(np.int32)   # non-contiguous ids
    p = Params(0.7, causal=True, window_len=5, cap_method=method, cap=c, alpha=a, beta=bt,
               z_loss_weight=0.3)
    fd_check(q, k, v, do, p, temp, seg, None)


@pytest.mark.parametrize("cap", CAPS)
def test_backward_finite_differences_ranker_gqa(cap):
    method, c, a, bt = cap
    rng = np.random.default_rng(12)
    B, L, Hq, Hkv, D = 2, 12, 4, 1, 8
    q, do = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    k, v = rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    temp = rng.uniform(0.5, 1.5, size=(B, L))
    rb = np.array([[0, 7, 7, 12], [2, 5, 6, 11]])
    p = Params(0.5, cap_method=method, cap=c, alpha=a, beta=bt, z_loss_weight=0.2)
    fd_check(q, k, v, do, p, temp, None, rb)


def test_zloss_alone_finite_differences():
    rng = np.random.default_rng(13)
    B, L, Hq, Hkv, D = 1, 10, 2, 2, 8
    q, k, v = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    do = np.zeros((B, L, Hq, D))
    p = Params(0.9, causal=True, cap_method="alsc", cap=5.0, alpha=4.0, beta=0.5,
               z_loss_weight=0.5)
    res = backward(q, k, v, do, p)
    assert np.abs(res["dv"]).max() == 0.0            # dV only comes from dO
    assert np.abs(res["dq"]).max() > 1e-3            # z-loss alone moves dQ
    fd_check(q, k, v, do, p, None, None, None)
    # w = 0 with dO = 0 gives no gradient at all
    res0 = backward(q, k, v, do, Params(0.9, causal=True, cap_method="alsc", cap=5.0,
                                        alpha=4.0, beta=0.5))
    assert max(np.abs(res0[n]).max() for n in ("dq", "dk", "dv")) == 0.0


def test_page_test_pattern_sum_of_squares():
    # loss = sum O^2 (the Mosaic page's backward test), i.e. dO = 2 O; ALSC(30,4,0.5),
    # temperature U[0.8,1.2], half history / half candidates, GQA 4:2, D 64 (shrunk L)
    rng = np.random.default_rng(42)
    B, L, Hq, Hkv, D = 1, 16, 4, 2, 64
    q, k, v = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    temp = rng.uniform(0.8, 1.2, size=(B, L))
    rb = np.array([[0, L // 2, L // 2, L]])
    p = Params(1 / math.sqrt(D), cap_method="alsc", cap=30.0, alpha=4.0, beta=0.5)
    o, _, _ = forward(q, k, v, p, temp, None, rb)
    res = backward(q, k, v, 2 * o, p, temp, None, rb)

    def sumsq(qq, kk, vv):
        return float(np.sum(forward(qq, kk, vv, p, temp, None, rb)[0] ** 2))

    eps = 1e-6
    for name, arr in (("dq", q), ("dk", k), ("dv", v)):
        flat = arr.reshape(-1)
        for t in np.random.default_rng(1).choice(flat.size, 25, replace=False):
            old = flat[t]
            flat[t] = old + eps
            fp = sumsq(q, k, v)
            flat[t] = old - eps
            fm = sumsq(q, k, v)
            flat[t] = old
            an = res[name].reshape(-1)[t]
            assert abs((fp - fm) / (2 * eps) - an) < 1e-6 * max(1.0, abs(an))


# ---------------------------------------------------------------------------
# Structural invariants
# ---------------------------------------------------------------------------

def test_length_one():
    rng = np.random.default_rng(3)
    q, k, v, do = rnd(rng, 1, 1, 2, 8), rnd(rng, 1, 1, 1, 8), rnd(rng, 1, 1, 1, 8), rnd(rng, 1, 1, 2, 8)
    temp = np.array([[1.3]])
    p = Params(0.25, causal=True, cap_method="tanh", cap=2.0)
    res = backward(q, k, v, do, p, temp)
    assert np.allclose(res["o"][0, 0], np.repeat(v[0, 0], 2, axis=0))
    assert np.allclose(res["l"], 1.0)
    s00 = 1.3 * 2.0 * np.tanh(0.25 * (q[0, 0] @ k[0, 0, 0]) / 2.0)
    assert np.allclose(res["m"][0, :, 0], s00)
    assert np.abs(res["dq"]).max() < 1e-15 and np.abs(res["dk"]).max() < 1e-15
    assert np.allclose(res["dv"][0, 0, 0], do[0, 0].sum(axis=0))


def test_packed_segments_equal_separate_runs():
    rng = np.random.default_rng(4)
    L, H, D = 30, 2, 8
    q, k, v, do = (rnd(rng, 1, L, H, D) for _ in range(4))
    seg = np.array([[0] * 11 + [1] * 6 + [2] * 13])
    p = Params(0.4, causal=True, cap_method="soft_sign", cap=3.0, z_loss_weight=0.1)
    temp = rng.uniform(0.5, 1.5, size=(1, L))
    res = backward(q, k, v, do, p, temp, seg)
    for a, b in ((0, 11), (11, 17), (17, 30)):
        sub = backward(q[:, a:b], k[:, a:b], v[:, a:b], do[:, a:b], p, temp[:, a:b])
        for n in ("o", "dq", "dk", "dv"):
            assert np.allclose(res[n][:, a:b], sub[n], atol=1e-13)
        for n in ("m", "l"):
            assert np.allclose(res[n][:, :, a:b], sub[n], atol=1e-13)


def test_window_limits():
    rng = np.random.default_rng(5)
    L, D = 25, 8
    q, k, v, do = (rnd(rng, 1, L, 1, D) for _ in range(4))
    pc = Params(0.5, causal=True, cap_method="tanh", cap=4.0)
    big = backward(q, k, v, do, Params(0.5, causal=True, window_len=L, cap_method="tanh", cap=4.0))
    ref = backward(q, k, v, do, pc)
    for n in ("o", "dq", "dk", "dv", "m", "l"):
        assert np.allclose(big[n], ref[n], atol=1e-14)
    one = forward(q, k, v, Params(0.5, causal=True, window_len=1, cap_method="tanh", cap=4.0))[0]
    assert np.allclose(one, v, atol=1e-14)


def test_ranker_decomposes_into_plain_attention():
    # history rows attend to history keys (no causality); a candidate row attends to
    # history keys plus itself; checked row by row with SDPA on sub-sequences
    rng = np.random.default_rng(6)
    L, H, D, h = 20, 2, 8, 12
    q, k, v = rnd(rng, 1, L, H, D), rnd(rng, 1, L, H, D), rnd(rng, 1, L, H, D)
    rb = np.array([[0, h, h, L]])
    p = Params(0.5)
    o, _, _ = forward(q, k, v, p, None, None, rb)
    tq, tk, tv = (torch.tensor(x).permute(0, 2, 1, 3) for x in (q, k, v))
    hist = F.scaled_dot_product_attention(tq[:, :, :h], tk[:, :, :h], tv[:, :, :h], scale=0.5)
    assert np.allclose(o[0, :h], hist.permute(0, 2, 1, 3).numpy()[0], atol=1e-13)
    for i in range(h, L):
        idx = list(range(h)) + [i]
        ci = F.scaled_dot_product_attention(tq[:, :, i:i + 1], tk[:, :, idx], tv[:, :, idx], scale=0.5)
        assert np.allclose(o[0, i], ci.permute(0, 2, 1, 3).numpy()[0, 0], atol=1e-13)


def test_gqa_equals_repeated_heads():
    rng = np.random.default_rng(8)
    B, L, Hq, Hkv, D = 1, 18, 6, 2, 8
    q, do = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    k, v = rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    p = Params(0.4, causal=True, cap_method="alsc", cap=6.0, alpha=2.0, beta=0.3, z_loss_weight=0.2)
    g = backward(q, k, v, do, p)
    r = backward(q, np.repeat(k, 3, axis=2), np.repeat(v, 3, axis=2), do, p)
    for n in ("o", "dq", "m", "l"):
        assert np.allclose(g[n], r[n], atol=1e-14)
    assert np.allclose(g["dk"], r["dk"].reshape(B, L, Hkv, 3, D).sum(axis=3), atol=1e-13)
    assert np.allclose(g["dv"], r["dv"].reshape(B, L, Hkv, 3, D).sum(axis=3), atol=1e-13)


def test_fully_masked_row():
    rng = np.random.default_rng(9)
    L, D = 8, 4
    q, k, v, do = (rnd(rng, 1, L, 1, D) for _ in range(4))
    rb = np.array([[0, 3, 5, 7]])     # rows 3, 4 and 7 see nothing
    p = Params(0.5, cap_method="tanh", cap=3.0, z_loss_weight=0.5)
    res = backward(q, k, v, do, p, None, None, rb)
    for i in (3, 4, 7):
        assert np.all(res["o"][0, i] == 0) and res["l"][0, 0, i] == 0
        assert res["m"][0, 0, i] == -np.inf and np.all(res["dq"][0, i] == 0)
    assert np.all(np.isfinite(res["dk"])) and np.all(np.isfinite(res["dv"]))
    # keys 3, 4 are seen by nobody: no gradient reaches them
    assert np.all(res["dk"][0, 3:5] == 0) and np.all(res["dv"][0, 3:5] == 0)


def test_delta_identity_and_row_helpers():
    rng = np.random.default_rng(10)
    B, L, Hq, Hkv, D = 2, 16, 4, 2, 8
    q, do = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    k, v = rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    temp = rng.uniform(0.5, 1.5, size=(B, L))
    p = Params(0.4, causal=True, window_len=6, cap_method="tanh", cap=2.0, z_loss_weight=0.1)
    full = backward(q, k, v, do, p, temp)
    rows = np.array([0, 5, 15])
    r = dq_rows(q, k, v, do, p, 1, 3, rows, temp)
    assert np.allclose(r["dq"], full["dq"][1, rows, 3], atol=1e-14)
    assert np.allclose(r["delta"], full["delta"][1, 3, rows], atol=1e-14)
    # delta_i = sum_j P_ij dP_ij with P recovered from the oracle's m, l
    G = Hq // Hkv
    for b in range(B):
        for hq in range(Hq):
            s = p.sm_scale * q[b, :, hq] @ k[b, :, hq // G].T
            sp = temp[b][:, None] * 2.0 * np.tanh(s / 2.0)
            vis = visible(np.arange(L), L, p)
            P = np.where(vis, np.exp(sp - full["m"][b, hq][:, None]), 0) / full["l"][b, hq][:, None]
            dP = do[b, :, hq] @ v[b, :, hq // G].T
            assert np.allclose((P * dP).sum(1), full["delta"][b, hq], atol=1e-13)
    keys = np.array([0, 7, 15])
    kv = dkv_keys(q, k, v, do, p, 0, 1, keys, temp)
    assert np.allclose(kv["dk"], full["dk"][0, keys, 1], atol=1e-13)
    assert np.allclose(kv["dv"], full["dv"][0, keys, 1], atol=1e-13)


def test_preprocess_delta_identity_and_axis_order():
    """preprocess (delta = sum_d O dO, laid out (B, Hq, L)) against the identity
    delta_i = sum_j P_ij dP_ij with dP = dO V^T, where P and O come from torch's
    softmax on CPU, not from the oracle.  B, L, Hq and D all differ, so a
    reduction over the wrong axis or a transposed output fails."""
    rng = np.random.default_rng(12)
    B, L, Hq, Hkv, D = 2, 7, 3, 1, 5
    q, do = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    k, v = rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    o = np.zeros((B, L, Hq, D))
    ref = np.zeros((B, Hq, L))
    for b in range(B):
        for hq in range(Hq):
            s = torch.from_numpy(0.3 * q[b, :, hq] @ k[b, :, 0].T)
            P = torch.softmax(s, dim=-1).numpy()
            o[b, :, hq] = P @ v[b, :, 0]
            dP = do[b, :, hq] @ v[b, :, 0].T
            ref[b, hq] = (P * dP).sum(axis=1)
    from oracle import preprocess
    got = preprocess(o, do)
    assert got.shape == (B, Hq, L)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    # the planted mistake of an output in (B, L, Hq) order read as (B, Hq, L)
    wrong = np.einsum("blhd,blhd->blh", o, do).reshape(B, Hq, L)
    assert not np.allclose(wrong, ref, atol=1e-6)


def test_cap_golden_closed_forms():
    import json
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "cap_closed_forms.json")
    for c in json.load(open(path))["cases"]:
        s = np.array([c["s"]])
        args = (c["method"], c["cap"], c.get("alpha", 0.0), c.get("beta", 0.0))
        assert cap_forward(s, *args)[0] == pytest.approx(c["value"], rel=1e-11, abs=1e-12), c
        if "slope" in c:
            assert cap_derivative(s, *args)[0] == pytest.approx(c["slope"], rel=1e-11), c


# ---------------------------------------------------------------------------
# Temperature gradient and ranker bounds from segment ids
# ---------------------------------------------------------------------------

def test_dtemp_equals_dq_dot_q_without_cap():
    """Without a cap, temp_i scales row i of Q: t_i * dtemp_i = sum_h dQ_ih . Q_ih."""
    rng = np.random.default_rng(21)
    B, L, Hq, Hkv, D = 2, 16, 4, 2, 8
    q, do = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    k, v = rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    temp = rng.uniform(0.5, 1.5, size=(B, L))
    p = Params(0.6, causal=True, window_len=6, z_loss_weight=0.25)
    res = backward(q, k, v, do, p, temp)
    lhs = temp * res["dtemp"]
    rhs = np.einsum("blhd,blhd->bl", res["dq"], q)
    assert np.allclose(lhs, rhs, rtol=1e-12, atol=1e-13)
    assert np.abs(res["dtemp"]).max() > 1e-3


def test_dtemp_rows_helper_sums_to_backward():
    rng = np.random.default_rng(22)
    B, L, Hq, Hkv, D = 1, 12, 4, 2, 8
    q, do = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    k, v = rnd(rng, B, L, Hkv, D), rnd(rng, B, L, Hkv, D)
    temp = rng.uniform(0.5, 1.5, size=(B, L))
    p = Params(0.5, causal=True, cap_method="alsc", cap=6.0, alpha=3.0, beta=0.25,
               z_loss_weight=0.1)
    res = backward(q, k, v, do, p, temp)
    rows = np.array([0, 3, 7, 11])
    tot = sum(dq_rows(q, k, v, do, p, 0, h, rows, temp)["dtemp_h"] for h in range(Hq))
    assert np.allclose(tot, res["dtemp"][0, rows], rtol=1e-12, atol=1e-14)
    # a row restricted backward leaves dtemp undefined
    part = backward(q, k, v, do, p, temp, groups=[(0, 0)])
    assert np.all(np.isnan(part["dtemp"]))


def test_dtemp_of_fully_masked_row_is_zero():
    rng = np.random.default_rng(23)
    B, L, Hq, D = 1, 8, 2, 4
    q, do = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    k, v = rnd(rng, B, L, Hq, D), rnd(rng, B, L, Hq, D)
    rb = np.array([[2, 5, 5, 7]])        # rows 0, 1 and 7 see nothing
    res = backward(q, k, v, do, Params(0.5, z_loss_weight=0.2), rng.uniform(0.5, 1.5, (B, L)),
                   None, rb)
    assert np.all(res["dtemp"][0, [0, 1, 7]] == 0.0)
    assert np.all(res["dtemp"][0, 2:7] != 0.0)


def _bounds_by_loop(seg, hid, cid):
    out = []
    for row in seg:
        b = []
        for ident in (hid, cid):
            lo, hi = None, None
            for i, x in enumerate(row):
                if x == ident:
                    lo = i if lo is None else lo
                    hi = i + 1
            b += [0, 0] if lo is None else [lo, hi]
        out.append(b)
    return np.array(out, dtype=np.int32)


def test_ranker_bounds_page_test_pattern():
    """The page's test: the first half of each row is history, the rest candidates."""
    L, HID, CID = 128, 7, 9
    seg = np.zeros((2, L), dtype=np.int32)
    seg[:, :L // 2] = HID
    seg[:, L // 2:] = CID
    assert ranker_bounds_from_segments(seg, HID, CID).tolist() == [[0, 64, 64, 128]] * 2


def test_ranker_bounds_edge_cases_and_brute_force():
    HID, CID = 3, 5
    seg = np.array([[0, 0, 0, 0, 0, 0],      # neither id
                    [3, 3, 3, 3, 3, 3],      # history only
                    [5, 0, 0, 0, 0, 0],      # one candidate at the start
                    [0, 0, 0, 0, 0, 3],      # one history position at the end
                    [3, 0, 3, 5, 0, 5]],     # non-contiguous: the smallest covering interval
                   dtype=np.int32)
    got = ranker_bounds_from_segments(seg, HID, CID)
    assert got.tolist() == [[0, 0, 0, 0], [0, 6, 0, 0], [0, 0, 0, 1], [5, 6, 0, 0],
                            [0, 3, 3, 6]]
    rng = np.random.default_rng(24)
    for _ in range(20):
        s = rng.integers(0, 8, size=(3, int(rng.integers(1, 40)))).astype(np.int32)
        assert np.array_equal(ranker_bounds_from_segments(s, 2, 6), _bounds_by_loop(s, 2, 6))
