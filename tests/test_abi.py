"""CPU tests of the C ABI: the library loads and exports every declared
symbol, host-side validation rejects bad arguments before any launch, and the
host planner's pair / tile counts agree with brute force over the oracle's
visibility predicate."""
import ctypes
import os
import re

import numpy as np
import pytest

import blockwise_softmax_attention_amd as ba
from oracle import Params, visible

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    src = open(os.path.join(ROOT, "include", "attn.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_0-9]+)\s*\(", src)))


def test_library_exports_every_declared_function():
    lib = ba.load_library()
    names = header_functions()
    assert {"attn_fwd", "attn_bwd_preprocess", "attn_bwd_dq", "attn_bwd_dkv",
            "attn_plan_count"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n
    assert b"gfx950" in lib.attn_build_info()


def base_params(**kw):
    d = dict(batch=1, seq_len=64, q_heads=2, kv_heads=1, head_dim=64, dtype=ba.ATTN_BF16,
             sm_scale=0.125, causal=True, cap_method=1, cap=30.0)
    d.update(kw)
    return ba.AttnParams(**d)


@pytest.mark.parametrize("kw,status", [
    (dict(batch=0), -2), (dict(seq_len=0), -2), (dict(seq_len=300000), -2), (dict(q_heads=0), -2),
    (dict(dtype=7), -3), (dict(head_dim=96), -4), (dict(q_heads=3, kv_heads=2), -4),
    (dict(cap_method=9), -6), (dict(window_len=-1), -6), (dict(z_loss_weight=-1.0), -6),
    (dict(sm_scale=0.0), -6), (dict(sm_scale=float("nan")), -6), (dict(cap=float("inf")), -6),
])
def test_params_validation(kw, status):
    with pytest.raises(ba.AttnError) as e:
        ba.attn_check_params(base_params(**kw))
    assert e.value.status == status


def test_valid_params_pass():
    ba.attn_check_params(base_params())
    ba.attn_check_params(base_params(cap=-1.0, cap_method=3))   # cap <= 0: no cap, still valid


def call_raw_fwd(p, ptrs):
    lib = ba.load_library()
    cp = p.to_c()
    return lib.attn_fwd(ctypes.byref(cp), *ptrs, None)


def test_null_and_misaligned_pointers_rejected_before_launch():
    lib = ba.load_library()
    p = base_params()
    good = 4096
    # q, k, v, temp, seg, bounds, o, m, l
    ptrs = [good, good, good, None, None, None, good, good, good]
    for idx, name in ((0, "q"), (1, "k"), (2, "v"), (6, "o"), (7, "m"), (8, "l")):
        bad = list(ptrs)
        bad[idx] = None
        assert call_raw_fwd(p, bad) == -1
        assert name in lib.attn_last_error().decode()
    bad = list(ptrs)
    bad[0] = good + 8
    assert call_raw_fwd(p, bad) == -5
    bad = list(ptrs)
    bad[3] = good + 2          # temperature must be 4-byte aligned
    assert call_raw_fwd(p, bad) == -5
    # segment ids beyond the segment-table limit
    p2 = base_params(seq_len=140000)
    bad = list(ptrs)
    bad[4] = good
    assert call_raw_fwd(p2, bad) == -4
    # backward entry points validate too
    cp = p.to_c()
    assert lib.attn_bwd_preprocess(ctypes.byref(cp), None, good, good, None) == -1
    assert lib.attn_bwd_dq(ctypes.byref(cp), good, good, good, None, None, None, good, good, good,
                           good, good + 4, None, None) == -5
    assert lib.attn_bwd_dq(ctypes.byref(cp), good, good, good, None, None, None, good, good, good,
                           good, good, good + 2, None) == -5     # dtemp_h 4-byte aligned
    assert "dtemp_h" in lib.attn_last_error().decode()
    assert lib.attn_reduce_heads(ctypes.byref(cp), None, good, None) == -1
    assert lib.attn_reduce_heads(ctypes.byref(cp), good, good + 1, None) == -5
    assert lib.attn_reduce_heads(None, good, good, None) == -1
    assert lib.attn_ranker_bounds(good, 2, 64, 3, 3, good, None) == -6   # ids must differ
    assert lib.attn_ranker_bounds(good, 0, 64, 3, 4, good, None) == -2
    assert lib.attn_ranker_bounds(good, 2, 0, 3, 4, good, None) == -2
    assert lib.attn_ranker_bounds(None, 2, 64, 3, 4, good, None) == -1
    assert lib.attn_ranker_bounds(good, 2, 64, 3, 4, good + 2, None) == -5
    assert lib.attn_bwd_dkv(ctypes.byref(cp), good, good, good, None, None, None, good, good, good,
                            good, good, None, None) == -1
    assert lib.attn_fwd(None, *ptrs, None) == -1
    # the stream probe: shape and pointer checks, before any launch
    assert lib.attn_probe_stream(good, 1 << 20, 0, good, None) == -2
    assert lib.attn_probe_stream(good, 1 << 20, 65537, good, None) == -2
    assert lib.attn_probe_stream(good, 1000 * 1024, 512, good, None) == -2   # not 1024 * blocks
    assert lib.attn_probe_stream(good, 0, 1, good, None) == -2
    assert lib.attn_probe_stream(None, 1 << 20, 4, good, None) == -1
    assert lib.attn_probe_stream(good + 8, 1 << 20, 4, good, None) == -5
    assert lib.attn_probe_stream(good, 1 << 20, 4, good + 2, None) == -5


def test_status_strings():
    lib = ba.load_library()
    for s, n in ba.STATUS_NAMES.items():
        assert lib.attn_status_str(s).decode() == n


# ---------------------------------------------------------------------------
# Host planner vs brute force
# ---------------------------------------------------------------------------

BM = 128   # query rows per forward workgroup


def brute(L, causal, window, seg, rb, B, bn):
    p = Params(1.0, causal=causal, window_len=window)
    pairs = 0
    tiles_with_pairs = 0
    for b in range(B):
        vis = visible(np.arange(L), L, p, None if seg is None else seg[b],
                      None if rb is None else rb[b])
        pairs += int(vis.sum())
        for q0 in range(0, L, BM):
            for k0 in range(0, L, bn):
                if vis[q0:q0 + BM, k0:k0 + bn].any():
                    tiles_with_pairs += 1
    return pairs, tiles_with_pairs


def fwd_bn(dtype, D):
    return 64 if (dtype == ba.ATTN_BF16 or D == 64) else 32


@pytest.mark.parametrize("seed", range(12))
def test_plan_count_matches_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    B = int(rng.integers(1, 3))
    L = int(rng.integers(1, 700))
    Hq = int(rng.integers(1, 4))
    causal = bool(rng.integers(0, 2))
    window = int(rng.choice([0, 0, 1, 7, 63, 64, 130, 1000]))
    use_seg = bool(rng.integers(0, 2))
    use_rk = bool(rng.integers(0, 2))
    dtype = int(rng.integers(0, 2))
    D = int(rng.choice([64, 128]))
    seg = rb = None
    if use_seg:
        if rng.integers(0, 2):
            seg = np.sort(rng.integers(0, 4, size=(B, L)), axis=1).astype(np.int32)   # packed
        else:
            seg = rng.integers(0, 3, size=(B, L)).astype(np.int32)                     # arbitrary
    if use_rk:
        rb = []
        for _ in range(B):
            h = int(rng.integers(0, L + 1))
            if rng.integers(0, 2):
                rb.append([0, h, h, L])
            else:
                a, b_, c, d = sorted(rng.integers(0, L + 1, size=4))
                rb.append([a, c, b_, d])        # general (possibly overlapping) bounds
        rb = np.array(rb, dtype=np.int32)
    p = ba.AttnParams(batch=B, seq_len=L, q_heads=Hq, kv_heads=1, head_dim=D, dtype=dtype,
                      sm_scale=1.0, causal=causal, window_len=window)
    pairs, tiles = ba.attn_plan_count(p, seg, rb)
    bp, bt = brute(L, causal, window, seg, rb, B, fwd_bn(dtype, D))
    assert pairs == bp * Hq
    # sound: every tile holding a visible pair is visited; never more than all tiles
    n_all = B * ((L + BM - 1) // BM) * ((L + fwd_bn(dtype, D) - 1) // fwd_bn(dtype, D))
    assert bt * Hq <= tiles <= n_all * Hq
    if seg is None and not (use_rk and (causal or window)):
        assert tiles == bt * Hq       # exact for causal/window alone and for the ranker alone


def test_plan_count_closed_forms_of_workloads():
    # causal, L = 32768, 8 heads: 8 L (L + 1) / 2 pairs; W = 512 window on L = 4096
    p = ba.AttnParams(batch=1, seq_len=32768, q_heads=8, kv_heads=8, head_dim=128, causal=True)
    assert ba.attn_plan_count(p)[0] == 8 * 32768 * 32769 // 2
    p = ba.AttnParams(batch=1, seq_len=4096, q_heads=16, kv_heads=16, head_dim=128, causal=True,
                      window_len=512)
    assert ba.attn_plan_count(p)[0] == 16 * (512 * 513 // 2 + (4096 - 512) * 512)
    rb = np.array([[0, 5000, 5000, 8192], [0, 4096, 4096, 8192]], dtype=np.int32)
    p = ba.AttnParams(batch=2, seq_len=8192, q_heads=16, kv_heads=4, head_dim=128)
    assert ba.attn_plan_count(p, None, rb)[0] == 16 * sum(8192 * h + 8192 - h for h in (5000, 4096))


# ---------------------------------------------------------------------------
# Stored-dS workspace: size and requirements (host only)
# ---------------------------------------------------------------------------

def brute_ds_tiles(L, causal, window, T=128):
    """Per (batch row, head): sum over query tiles of the width of the key-tile
    band between the first and last key any of its rows may see under the
    causal and window predicates (segments and ranker bounds left aside)."""
    nt = (L + T - 1) // T
    total = 0
    for qt in range(nt):
        rows = np.arange(qt * T, min(qt * T + T, L))
        keys = np.arange(L)
        vis = np.ones((rows.size, L), dtype=bool)
        if causal:
            vis &= keys[None, :] <= rows[:, None]
        if window > 0:
            vis &= keys[None, :] > rows[:, None] - window
        ks = np.nonzero(vis.any(axis=0))[0]
        assert ks.size > 0
        total += ks.max() // T - ks.min() // T + 1
    return total


@pytest.mark.parametrize("L", [1, 127, 128, 129, 300, 1000, 2048])
@pytest.mark.parametrize("causal,window", [(True, 0), (False, 0), (True, 1), (True, 37),
                                           (True, 128), (True, 129), (True, 257), (False, 200),
                                           (True, 5000)])
def test_ds_workspace_size_matches_band(L, causal, window):
    p = base_params(batch=3, q_heads=4, kv_heads=2, seq_len=L, causal=causal, window_len=window,
                    precise_ds=False)
    assert ba.attn_bwd_ds_workspace_size(p) == 3 * 4 * brute_ds_tiles(L, causal, window) * 128 * 128 * 2


def test_ds_workspace_closed_forms():
    # long-context workload: causal, 256 tiles -> 256 * 257 / 2 per head
    p = base_params(batch=1, q_heads=8, kv_heads=8, seq_len=32768, head_dim=128, precise_ds=False)
    assert ba.attn_bwd_ds_workspace_size(p) == 8 * (256 * 257 // 2) * 32768
    # ranker workload: no causal mask -> the full 64 x 64 tiles per head
    p = base_params(batch=4, q_heads=16, kv_heads=4, seq_len=8192, head_dim=128, causal=False,
                    precise_ds=False)
    assert ba.attn_bwd_ds_workspace_size(p) == 64 * 64 * 64 * 32768


@pytest.mark.parametrize("kw,status", [(dict(dtype=ba.ATTN_F32), -3), (dict(precise_ds=True), -4)])
def test_ds_path_requirements(kw, status):
    d = dict(precise_ds=False)
    d.update(kw)
    with pytest.raises(ba.AttnError) as e:
        ba.attn_bwd_ds_workspace_size(base_params(**d))
    assert e.value.status == status


def test_ds_calls_reject_null_workspace_before_launch():
    lib = ba.load_library()
    p = base_params(precise_ds=False)
    cp = p.to_c()
    buf = ctypes.create_string_buffer(1 << 16)
    a = ctypes.addressof(buf)
    a16 = a + (-a) % 16
    need = ba.attn_bwd_ds_workspace_size(p)
    st = lib.attn_bwd_dq_ds(ctypes.byref(cp), a16, None, None, None, need, a16, None)
    assert st == -1 and b"ds" in lib.attn_last_error()
    st = lib.attn_bwd_dq_ds(ctypes.byref(cp), a16, None, None, a16 + 4, need, a16, None)
    assert st == -5
    # a workspace smaller than the layout needs is refused before any launch
    st = lib.attn_bwd_dq_ds(ctypes.byref(cp), a16, None, None, a16, need - 1, a16, None)
    assert st == -2 and b"needed" in lib.attn_last_error()
    st = lib.attn_bwd_dkv_ds(ctypes.byref(cp), a16, a16, a16, None, None, None, a16, a16, a16, a16,
                             a16, a16, a16, need - 1, None)
    assert st == -2 and b"needed" in lib.attn_last_error()


def test_stored_ds_auto_selection_cap():
    """attention_forward_backward takes the stored-dS backward on its own only
    when it applies and its workspace fits STORED_DS_AUTO_MAX_BYTES."""
    cap = ba.STORED_DS_AUTO_MAX_BYTES
    assert cap == 16 << 30
    long_ctx = base_params(batch=1, seq_len=32768, q_heads=8, kv_heads=8, head_dim=128,
                           causal=True, precise_ds=False)
    need = ba.attn_bwd_ds_workspace_size(long_ctx)
    assert need == 8 * (256 * 257 // 2) * 32768 and need <= cap
    assert ba.stored_ds_auto(long_ctx)
    # four times the length: ~16x the workspace, past the cap -> recomputing dQ
    longer = base_params(batch=1, seq_len=131072, q_heads=8, kv_heads=8, head_dim=128,
                         causal=True, precise_ds=False)
    assert ba.attn_bwd_ds_workspace_size(longer) > cap
    assert not ba.stored_ds_auto(longer)
    # a caller's own cap
    assert not ba.stored_ds_auto(long_ctx, max_bytes=need - 1)
    assert ba.stored_ds_auto(long_ctx, max_bytes=need)
    # not eligible: hi+lo operands, float inputs, temperature gradient
    assert not ba.stored_ds_auto(base_params(precise_ds=True))
    assert not ba.stored_ds_auto(base_params(dtype=ba.ATTN_F32, precise_ds=False))
    assert not ba.stored_ds_auto(base_params(precise_ds=False), dtemp=True)
    assert ba.stored_ds_auto(base_params(precise_ds=False))


def test_static_ds_entry_point_rejects_shapes_beyond_its_array_before_launch():
    """attn_bwd_ds_static refuses a shape whose stored-dS workspace exceeds the
    library's fixed array, on the host, before touching the GPU."""
    lib = ba.load_library()
    good = 4096
    big = base_params(batch=1, seq_len=32768, q_heads=8, kv_heads=8, head_dim=128, causal=True,
                      precise_ds=False)
    assert ba.attn_bwd_ds_workspace_size(big) > ba.ATTN_STATIC_DS_BYTES
    cp = big.to_c()
    # q, k, v, temp, seg, bounds, d_o, m, l, delta, dq, dk, dv, stream
    st = lib.attn_bwd_ds_static(ctypes.byref(cp), good, good, good, None, None, None, good, good, good,
                                good, good, good, good, None)
    assert st == -2
    assert "fixed array" in lib.attn_last_error().decode()
    # the requirements of the stored-dS backward hold here too
    cp = base_params(precise_ds=True).to_c()
    assert lib.attn_bwd_ds_static(ctypes.byref(cp), good, good, good, None, None, None, good, good,
                                  good, good, good, good, good, None) == -4
    cp = base_params(precise_ds=False).to_c()
    assert lib.attn_bwd_ds_static(ctypes.byref(cp), good, good, good, None, None, None, good, good,
                                  good, good, None, good, good, None) == -1
    assert "dq" in lib.attn_last_error().decode()
    # the two sizes the header quotes as fitting
    packed = base_params(batch=2, seq_len=2048, q_heads=8, kv_heads=8, head_dim=128, causal=True,
                         precise_ds=False)
    window = base_params(batch=1, seq_len=4096, q_heads=16, kv_heads=16, head_dim=128, causal=True,
                         window_len=512, precise_ds=False)
    for p, mib in ((packed, 68), (window, 75)):
        n = ba.attn_bwd_ds_workspace_size(p)
        assert n <= ba.ATTN_STATIC_DS_BYTES and abs(n / 2**20 - mib) < 1, (n, mib)
