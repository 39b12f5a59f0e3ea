"""Plain fp64 CPU oracle for capped, masked, grouped-query softmax attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the CPU-baseline
leg of the benchmark may import this module.  It shares no code with the HIP
library and the library never calls it.

It computes the plain definition of the method, materialising whole score
rows: no online softmax, no tiles, no fused steps.  Query rows are independent
in every quantity below, so they are processed in chunks of ``row_chunk`` rows
purely to bound memory; key-side gradient sums simply accumulate over those
chunks.

Sources (web pages on unified blockwise attention):
  * triton_kernels.py page, ``make_triton_forward_kernel``: score
    s = sm_scale * q.k, the segment / causal / sliding-window predicates, the
    cap and temperature applied inside the online-softmax update, and the
    (l, m) residuals.
  * triton_kernels.py page, ``make_triton_backward_kernel_dq`` and
    ``..._dkv``: the backward chain dp = dO.V^T, ds = p*(dp - delta), the
    z-loss term, ds *= temp, ds *= cap_grad, ds *= sm_scale, dq = ds.K,
    dk = ds^T.Q, dv = p^T.dO.
  * mosaic_backward.py page, module docstring: the same chain, with
    delta = sum(p*dp) = sum(o*do)/l and the z-loss gradient
    ds += z_weight * p * (log l + m) / l.
  * mosaic_backward.py page, ``_apply_cap_mosaic``: the four cap functions.
  * mosaic_backward.py page, ``ranker_mask_mosaic_kv_q``: the history /
    candidate ranker mask.
  * mosaic_backward.py page, ``make_mosaic_backward_dq_kernel``: the
    grouped-query map kv_head = q_head // (Hq / Hkv).

Readings where the pages are silent or disagree (each one is listed in the
design notes with its reason):
  * Masked pairs get probability exactly 0; the cap and temperature act on
    unmasked logits only.
  * P is normalised over the whole row: P = exp(S' - LSE), LSE = m + ln l.
  * The ALSC derivative is the exact derivative of the ALSC forward,
    alpha * sig(z) * (1 - sig(z)) / denom (the Mosaic page prints a factor
    1/cap too small).
  * The z-loss objective is (w/2) * sum LSE^2 over post-temperature logits,
    natural-log LSE, so its gradient adds w * P * LSE to dS'.
  * A row with no visible key has O = 0, l = 0, m = -inf and contributes no
    gradient.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
from scipy.special import expit

CAP_METHODS = ("none", "tanh", "soft_sign", "alsc")


@dataclasses.dataclass(frozen=True)
class Params:
    sm_scale: float
    causal: bool = False
    window_len: int = 0          # 0: off; key j visible from row i iff j > i - window_len
    cap_method: str = "none"
    cap: float = 0.0
    alpha: float = 0.0
    beta: float = 0.0
    z_loss_weight: float = 0.0


# ---------------------------------------------------------------------------
# Elementwise pieces
# ---------------------------------------------------------------------------

def sigmoid(x):
    """Logistic function 1 / (1 + e^-x), evaluated without overflow.

    The Mosaic page imports ``_sigmoid`` without printing it; the standard
    logistic function is the plain reading.
    """
    return expit(np.asarray(x, dtype=np.float64))


def _alsc_consts(cap, alpha, beta):
    sb = float(sigmoid(np.array(alpha * beta)))
    denom = sb * (1.0 - sb) + 1e-12
    return sb, denom


def cap_forward(s, method: str, cap: float, alpha: float = 0.0, beta: float = 0.0):
    """Logit cap applied to s = sm_scale * q.k (mosaic_backward.py page,
    ``_apply_cap_mosaic``).

    none, or cap <= 0 : s
    tanh              : cap * tanh(s / cap)
    soft_sign         : s / (1 + |s| / cap)
    alsc              : cap * (sig(alpha (s/cap + beta)) - sig(alpha beta)) / denom,
                        denom = sig(alpha beta) (1 - sig(alpha beta)) + 1e-12
    """
    s = np.asarray(s, dtype=np.float64)
    if method not in CAP_METHODS:
        raise ValueError(f"unknown cap method {method!r}")
    if method == "none" or cap <= 0:
        return s.copy()
    if method == "tanh":
        return cap * np.tanh(s / cap)
    if method == "soft_sign":
        return s / (1.0 + np.abs(s) / cap)
    sb, denom = _alsc_consts(cap, alpha, beta)
    z = alpha * (s / cap + beta)
    return cap * (sigmoid(z) - sb) / denom


def cap_derivative(s, method: str, cap: float, alpha: float = 0.0, beta: float = 0.0):
    """d cap_forward / d s, the exact derivative of each cap.

    tanh and soft_sign agree with ``_apply_cap_grad_mosaic`` on the Mosaic page
    (1 - tanh^2 and (1/(1+|s|/cap))^2).  For ALSC the page prints
    (alpha/cap) sig'(z)/denom, which is 1/cap times the derivative of its own
    forward; the exact derivative alpha sig(z)(1 - sig(z)) / denom is used.
    """
    s = np.asarray(s, dtype=np.float64)
    if method not in CAP_METHODS:
        raise ValueError(f"unknown cap method {method!r}")
    if method == "none" or cap <= 0:
        return np.ones_like(s)
    if method == "tanh":
        t = np.tanh(s / cap)
        return 1.0 - t * t
    if method == "soft_sign":
        r = 1.0 / (1.0 + np.abs(s) / cap)
        return r * r
    _, denom = _alsc_consts(cap, alpha, beta)
    sz = sigmoid(alpha * (s / cap + beta))
    return alpha * sz * (1.0 - sz) / denom


def visible(rows, L: int, p: Params, seg_b=None, bounds_b=None):
    """Boolean visibility of keys 0..L-1 from query rows ``rows`` of one batch row.

    AND of every enabled predicate (triton_kernels.py page, forward kernel;
    mosaic_backward.py page, ``ranker_mask_mosaic_kv_q``):
      segment  : seg[i] == seg[j]
      causal   : i >= j
      window   : j > i - window_len
      ranker   : (j in [hl,hu) and (i in [hl,hu) or i in [cl,cu)))
                 or (i in [cl,cu) and j in [cl,cu) and i == j)
    """
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(L, dtype=np.int64)[None, :]
    vis = np.ones((i.shape[0], L), dtype=bool)
    if seg_b is not None:
        seg_b = np.asarray(seg_b)
        vis &= seg_b[i] == seg_b[j]
    if p.causal:
        vis &= i >= j
    if p.window_len > 0:
        vis &= j > i - p.window_len
    if bounds_b is not None:
        hl, hu, cl, cu = (int(x) for x in bounds_b)
        q_hist = (i >= hl) & (i < hu)
        q_cand = (i >= cl) & (i < cu)
        k_hist = (j >= hl) & (j < hu)
        k_cand = (j >= cl) & (j < cu)
        vis &= (k_hist & (q_hist | q_cand)) | (q_cand & k_cand & (i == j))
    return vis


# ---------------------------------------------------------------------------
# Row statistics (shared by forward and backward)
# ---------------------------------------------------------------------------

def _row_block(q, k, v, b, hq, rows, p: Params, G, temp, seg, bounds):
    """Scores, capped post-temperature logits, mask, m, l, LSE and P for the
    given query rows of (batch b, query head hq); full key range."""
    L = k.shape[1]
    g = hq // G
    qr = q[b, rows, hq, :]                        # (R, D)
    kg = k[b, :, g, :]                            # (L, D)
    s = p.sm_scale * (qr @ kg.T)                  # (R, L)
    c = cap_forward(s, p.cap_method, p.cap, p.alpha, p.beta)
    t = np.ones(len(rows)) if temp is None else temp[b, rows]
    sp = t[:, None] * c
    vis = visible(rows, L, p, None if seg is None else seg[b],
                  None if bounds is None else bounds[b])
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, np.max(np.where(vis, sp, -np.inf), axis=1), -np.inf)
    m_safe = np.where(any_vis, m, 0.0)
    e = np.where(vis, np.exp(np.where(vis, sp - m_safe[:, None], 0.0)), 0.0)
    l = e.sum(axis=1)
    lse = np.where(any_vis, m_safe + np.log(np.where(any_vis, l, 1.0)), -np.inf)
    P = np.where(any_vis[:, None], e / np.where(any_vis, l, 1.0)[:, None], 0.0)
    return dict(s=s, c=c, t=t, vis=vis, any=any_vis, m=m, l=l, lse=lse, P=P, g=g)


def _chunks(rows, n):
    for a in range(0, len(rows), n):
        yield rows[a:a + n]


def _check(q, k, v):
    B, L, Hq, D = q.shape
    Bk, Lk, Hkv, Dk = k.shape
    if (Bk, Lk, Dk) != (B, L, D) or v.shape != k.shape or Hq % Hkv != 0:
        raise ValueError("inconsistent shapes")
    return B, L, Hq, Hkv, D, Hq // Hkv


# ---------------------------------------------------------------------------
# Forward
# ---------------------------------------------------------------------------

def forward(q, k, v, p: Params, temperature=None, segment_ids=None, ranker_bounds=None,
            rows=None, heads=None, batches=None, row_chunk: int = 512):
    """O (B, L, Hq, D), m and l (B, Hq, L) by the plain definition.

    m_i = max over visible j of S'_ij, l_i = sum over visible j of
    exp(S'_ij - m_i), O_i = sum_j P_ij V_j with P_ij = exp(S'_ij - m_i) / l_i.
    ``rows``, ``heads``, ``batches`` restrict the computation (entries outside
    are left NaN).
    """
    B, L, Hq, Hkv, D, G = _check(q, k, v)
    rows = np.arange(L) if rows is None else np.asarray(rows)
    heads = range(Hq) if heads is None else heads
    batches = range(B) if batches is None else batches
    o = np.full((B, L, Hq, D), np.nan)
    m = np.full((B, Hq, L), np.nan)
    l = np.full((B, Hq, L), np.nan)
    for b in batches:
        for hq in heads:
            for rr in _chunks(rows, row_chunk):
                st = _row_block(q, k, v, b, hq, rr, p, G, temperature, segment_ids,
                                ranker_bounds)
                o[b, rr, hq, :] = st["P"] @ v[b, :, st["g"], :]
                m[b, hq, rr] = st["m"]
                l[b, hq, rr] = st["l"]
    return o, m, l


# ---------------------------------------------------------------------------
# Backward
# ---------------------------------------------------------------------------

def _dsp_block(st, v, do, b, hq, rr, p: Params, delta_rows):
    """dS' = dF/dS' for one row block: P (dP - delta) + w P LSE."""
    dP = do[b, rr, hq, :] @ v[b, :, st["g"], :].T
    lse = np.where(st["any"], st["lse"], 0.0)
    return st["P"] * (dP - delta_rows[:, None]) + p.z_loss_weight * st["P"] * lse[:, None]


def _ds_block(st, q, v, do, b, hq, rr, p: Params, delta_rows):
    """dS for one row block: dS = dS' * temp * cap'(s) * sm_scale."""
    dsp = _dsp_block(st, v, do, b, hq, rr, p, delta_rows)
    dcap = cap_derivative(st["s"], p.cap_method, p.cap, p.alpha, p.beta)
    return dsp * st["t"][:, None] * dcap * p.sm_scale


def _dtemp_block(st, v, do, b, hq, rr, p: Params, delta_rows):
    """One query head's share of the temperature gradient of the rows rr.
    S'_ij = temp_i c_ij, so dF/dtemp_i gets sum_j dS'_ij c_ij from every head."""
    dsp = _dsp_block(st, v, do, b, hq, rr, p, delta_rows)
    return np.sum(dsp * np.where(st["vis"], st["c"], 0.0), axis=1)


def backward(q, k, v, do, p: Params, temperature=None, segment_ids=None, ranker_bounds=None,
             row_chunk: int = 512, groups=None):
    """Gradients of F = sum(O * dO) + (w/2) * sum over rows of LSE^2.

    Returns dict(delta (B,Hq,L), dq (B,L,Hq,D), dk, dv (B,L,Hkv,D), dtemp (B,L),
    o, m, l).
    delta_i = sum_d O_id dO_id; dP = dO V^T; dS as in ``_ds_block``;
    dQ = dS K; dK = sum over the query heads of a group of dS^T Q;
    dV = likewise of P^T dO; dtemp_i = sum over the query heads of
    sum_j dS'_ij c_ij (the temperature multiplies the capped logits, and one
    temperature row serves every head).
    ``groups`` restricts the work to a list of (b, kv_head) pairs (every query
    head of each group); entries outside are left NaN, and so is dtemp unless
    every group is included.
    """
    B, L, Hq, Hkv, D, G = _check(q, k, v)
    if groups is None:
        groups = [(b, g) for b in range(B) for g in range(Hkv)]
    o = np.full((B, L, Hq, D), np.nan)
    m = np.full((B, Hq, L), np.nan)
    l = np.full((B, Hq, L), np.nan)
    for b, g in groups:
        o_, m_, l_ = forward(q, k, v, p, temperature, segment_ids, ranker_bounds,
                             heads=range(g * G, (g + 1) * G), batches=[b], row_chunk=row_chunk)
        hs = slice(g * G, (g + 1) * G)
        o[b, :, hs], m[b, hs], l[b, hs] = o_[b, :, hs], m_[b, hs], l_[b, hs]
    delta = preprocess(o, do)
    dq = np.full((B, L, Hq, D), np.nan)
    dk = np.full((B, L, Hkv, D), np.nan)
    dv = np.full((B, L, Hkv, D), np.nan)
    full = sorted(groups) == [(b, g) for b in range(B) for g in range(Hkv)]
    dtemp = np.zeros((B, L)) if full else np.full((B, L), np.nan)
    rows = np.arange(L)
    for b, g0 in groups:
        dk[b, :, g0] = 0.0
        dv[b, :, g0] = 0.0
        for hq in range(g0 * G, (g0 + 1) * G):
            for rr in _chunks(rows, row_chunk):
                st = _row_block(q, k, v, b, hq, rr, p, G, temperature, segment_ids,
                                ranker_bounds)
                ds = _ds_block(st, q, v, do, b, hq, rr, p, delta[b, hq, rr])
                g = st["g"]
                dq[b, rr, hq, :] = ds @ k[b, :, g, :]
                dk[b, :, g, :] += ds.T @ q[b, rr, hq, :]
                dv[b, :, g, :] += st["P"].T @ do[b, rr, hq, :]
                if full:
                    dtemp[b, rr] += _dtemp_block(st, v, do, b, hq, rr, p, delta[b, hq, rr])
    return dict(delta=delta, dq=dq, dk=dk, dv=dv, dtemp=dtemp, o=o, m=m, l=l)


def preprocess(o, do):
    """delta_i = sum_d O_id dO_id, (B, Hq, L) (mosaic_backward.py page,
    ``make_preprocess_backward_kernel``; with O normalised, the page's
    sum(o * do / l) over an unnormalised o is the same number)."""
    return np.einsum("blhd,blhd->bhl", np.asarray(o, np.float64), np.asarray(do, np.float64))


def dq_rows(q, k, v, do, p: Params, b, hq, rows, temperature=None, segment_ids=None,
            ranker_bounds=None):
    """dQ for selected rows of one (b, hq); also returns O, m, l, delta of those
    rows and this head's share of their temperature gradient (dtemp_h)."""
    B, L, Hq, Hkv, D, G = _check(q, k, v)
    rows = np.asarray(rows)
    st = _row_block(q, k, v, b, hq, rows, p, G, temperature, segment_ids, ranker_bounds)
    o_r = st["P"] @ v[b, :, st["g"], :]
    delta_r = np.sum(o_r * do[b, rows, hq, :], axis=1)
    ds = _ds_block(st, q, v, do, b, hq, rows, p, delta_r)
    return dict(dq=ds @ k[b, :, st["g"], :], o=o_r, m=st["m"], l=st["l"], delta=delta_r,
                dtemp_h=_dtemp_block(st, v, do, b, hq, rows, p, delta_r))


def dkv_keys(q, k, v, do, p: Params, b, g, keys, temperature=None, segment_ids=None,
             ranker_bounds=None, row_chunk: int = 512, rows=None):
    """dK, dV for selected keys of one (b, kv head g), summed over the group's
    query heads.  Needs the full-row statistics of every contributing query
    row, which are recomputed here by the plain definition.  ``rows`` may
    restrict the sum to the rows that can see the selected keys (a caller's
    statement about the mask; the omitted rows would add exact zeros)."""
    B, L, Hq, Hkv, D, G = _check(q, k, v)
    keys = np.asarray(keys)
    dk = np.zeros((len(keys), D))
    dv = np.zeros((len(keys), D))
    rows = np.arange(L) if rows is None else np.asarray(rows)
    for hq in range(g * G, (g + 1) * G):
        for rr in _chunks(rows, row_chunk):
            st = _row_block(q, k, v, b, hq, rr, p, G, temperature, segment_ids, ranker_bounds)
            o_r = st["P"] @ v[b, :, g, :]
            delta_r = np.sum(o_r * do[b, rr, hq, :], axis=1)
            ds = _ds_block(st, q, v, do, b, hq, rr, p, delta_r)
            dk += ds[:, keys].T @ q[b, rr, hq, :]
            dv += st["P"][:, keys].T @ do[b, rr, hq, :]
    return dict(dk=dk, dv=dv)


def unmasked_pairs(L: int, p: Params, segment_ids=None, ranker_bounds=None, B: int = 1,
                   row_chunk: int = 2048):
    """Number of visible (query, key) pairs summed over batch rows (one head)."""
    total = 0
    rows = np.arange(L)
    for b in range(B):
        for rr in _chunks(rows, row_chunk):
            total += int(visible(rr, L, p, None if segment_ids is None else segment_ids[b],
                                 None if ranker_bounds is None else ranker_bounds[b]).sum())
    return total


def ranker_bounds_from_segments(segment_ids, history_id: int, candidate_id: int):
    """Ranker bounds (B, 4) = [hl, hu, cl, cu] from segment ids (B, L).

    The mosaic_backward.py page's test marks history positions and candidate
    positions with two reserved segment ids and expects the kernels' ranker
    bounds to follow from them; the ids' values and the mapping are not
    printed.  Reading: [hl, hu) is the smallest interval holding every
    position whose id is ``history_id`` ([0, 0) if there is none), and the
    same for the candidates.  For contiguous runs that is the run itself."""
    seg = np.asarray(segment_ids)
    B = seg.shape[0]
    out = np.zeros((B, 4), dtype=np.int32)
    for b in range(B):
        for k, ident in enumerate((history_id, candidate_id)):
            pos = np.nonzero(seg[b] == ident)[0]
            if pos.size:
                out[b, 2 * k] = pos.min()
                out[b, 2 * k + 1] = pos.max() + 1
    return out
