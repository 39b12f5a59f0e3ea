"""GPU parity at the sequence-length limits of the API, in both operand modes.

* L = ATTN_MAX_SEQ_LEN (262144) without segment ids: GQA (two query heads on
  one KV head), D 64, causal with a 300-key sliding window, tanh cap,
  per-query temperature.
* L = ATTN_MAX_SEQ_LEN_SEGMENTS (131072) with segment ids: 512 packed causal
  segments, D 128, ALSC cap (the long-context workload's parameters), z-loss;
  the stored-dS backward is requested explicitly
  (its workspace, sized for the whole causal band, is above the binding's
  automatic limit here).

The short window and the short segments keep the work, and the oracle's
share of it, small at these lengths.  Compared: sampled rows (O, m, l, dQ) and
sampled keys (dK, dV), among them the first and last positions, tile
boundaries and, for the packed case, the keys on either side of segment
boundaries.  Each key's dK / dV is summed by the oracle over exactly the rows
that can see it (the window or the key's segment), which is the definition
with the exact zeros of the other rows left out.

Bars: bf16 rel-L2 <= 8e-3 and max-abs <= 3e-2 on O, dQ, dK, dV;
|dm| <= 1e-3, |dl|/l <= 1e-3.
"""
import math

import numpy as np
import pytest

from oracle_pool import dkv_keys_pooled, dq_rows_pooled
from test_gpu_parity import check_ml, check_tensor, run_gpu, say
from workloads import Workload, make_inputs

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning"),
              pytest.mark.timeout(900)]

MAX_SEQ_LEN = 262144            # ATTN_MAX_SEQ_LEN in include/attn.h
MAX_SEQ_LEN_SEGMENTS = 131072   # ATTN_MAX_SEQ_LEN_SEGMENTS

WINDOW = Workload("max_len_window_tanh_gqa_bf16", 41, B=1, Hq=2, Hkv=1, L=MAX_SEQ_LEN, D=64,
                  dtype="bf16", sm_scale=1.0 / 8.0, causal=True, window_len=300,
                  cap_method="tanh", cap=30.0, temperature=(0.5, 1.5))
SEGMENTS = Workload("max_len_segments_alsc_bf16", 42, B=1, Hq=1, Hkv=1, L=MAX_SEQ_LEN_SEGMENTS,
                    D=128, dtype="bf16", sm_scale=1.0 / math.sqrt(128), causal=True, window_len=0,
                    cap_method="alsc", cap=50.0, alpha=2.0, beta=0.0, z_loss_weight=1e-4,
                    temperature=(0.8, 1.2), n_segments=512, input_scale=0.5)

# (precise_ds, stored_ds): hi+lo operands with the recomputing dQ; single bf16
# with the stored-dS backward
MODES = ((True, False), (False, True))


def run_modes(w, inp, pick):
    out = {}
    for precise, stored in MODES:
        say(f"[limits] {w.name}: GPU run precise={precise} stored_ds={stored}")
        got = run_gpu(w, inp, precise=precise, stored_ds=stored)
        out[precise] = pick(got)
        del got
    return out


def compare(w, gpu, rows_by_head, keys, rref, kref, precise):
    g = gpu[precise]
    heads = sorted(rows_by_head)
    check_ml(np.concatenate([g["m"][hq] for hq in heads]), np.concatenate([g["l"][hq] for hq in heads]),
             np.concatenate([r["m"] for r in rref]), np.concatenate([r["l"] for r in rref]), "bf16")
    check_tensor("O rows", np.concatenate([g["o"][hq] for hq in heads]),
                 np.concatenate([r["o"] for r in rref]), "bf16")
    check_tensor("dQ rows", np.concatenate([g["dq"][hq] for hq in heads]),
                 np.concatenate([r["dq"] for r in rref]), "bf16")
    check_tensor("dK keys", g["dk"], kref[0]["dk"], "bf16")
    check_tensor("dV keys", g["dv"], kref[0]["dv"], "bf16")


def picker(rows_by_head, keys):
    def pick(got):
        keep = {n: {hq: got[n][0, hq, r] for hq, r in rows_by_head.items()} for n in ("m", "l")}
        for n in ("o", "dq"):
            keep[n] = {hq: got[n][0, r, hq] for hq, r in rows_by_head.items()}
        for n in ("dk", "dv"):
            keep[n] = got[n][0, keys, 0]
        return keep
    return pick


# ---------------------------------------------------------------------------
# L = ATTN_MAX_SEQ_LEN, sliding window
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def window_case():
    w = WINDOW
    L, W = w.L, w.window_len
    rng = np.random.default_rng(51)
    keys = np.unique(np.concatenate([
        [0, 1, 127, 128, 129], L // 2 + np.arange(-2, 3), rng.choice(L, 6, replace=False),
        [L - 129, L - 128, L - 2, L - 1]]))
    rows = np.unique(np.concatenate([[0, 1, 299, 300, 127, 128, L - 1], rng.choice(L, 24, replace=False)]))
    rows_by_head = {0: rows, 1: rows}
    # the rows that see key k: [k, k + W - 1]
    krows = np.unique(np.concatenate([np.arange(k, min(L, k + W)) for k in keys]))
    gpu = run_modes(w, make_inputs(w), picker(rows_by_head, keys))
    say(f"[limits] {w.name}: oracle on {len(rows)} rows x 2 heads, {len(keys)} keys "
        f"({len(krows)} rows see them)")
    rref = dq_rows_pooled(w, [(0, hq, rows) for hq in (0, 1)], say)
    kref = dkv_keys_pooled(w, [(0, 0, keys, krows)], say, part_rows=512)
    return dict(gpu=gpu, rows_by_head=rows_by_head, keys=keys, rref=rref, kref=kref)


@pytest.mark.parametrize("precise", [m[0] for m in MODES])
def test_max_seq_len_window(window_case, precise):
    say(f"[limits] L={MAX_SEQ_LEN} window, precise={precise}")
    c = window_case
    compare(WINDOW, c["gpu"], c["rows_by_head"], c["keys"], c["rref"], c["kref"], precise)


# ---------------------------------------------------------------------------
# L = ATTN_MAX_SEQ_LEN_SEGMENTS, packed segments
# ---------------------------------------------------------------------------
@pytest.fixture(scope="module")
def segments_case():
    w = SEGMENTS
    L = w.L
    inp = make_inputs(w)
    seg = inp["segment_ids"].numpy()[0]
    starts = np.flatnonzero(np.diff(seg)) + 1          # first position of each later segment
    ends = np.append(starts, L)
    begins = np.insert(starts, 0, 0)
    rng = np.random.default_rng(52)
    picks = rng.choice(len(starts), 5, replace=False)
    keys = np.unique(np.concatenate([
        [0, 1, L - 1], starts[picks] - 1, starts[picks], starts[:2], rng.choice(L, 5, replace=False)]))
    rows = np.unique(np.concatenate([[0, L - 1], starts[picks], starts[picks] - 1,
                                     rng.choice(L, 20, replace=False)]))
    rows_by_head = {0: rows}
    # the rows that see key k (causal, same segment): [k, end of k's segment)
    sid = seg[keys]
    krows = np.unique(np.concatenate([np.arange(k, ends[s]) for k, s in zip(keys, sid)]))
    assert np.all(begins[sid] <= keys)
    gpu = run_modes(w, inp, picker(rows_by_head, keys))
    say(f"[limits] {w.name}: oracle on {len(rows)} rows, {len(keys)} keys ({len(krows)} rows see them)")
    rref = dq_rows_pooled(w, [(0, 0, rows)], say)
    kref = dkv_keys_pooled(w, [(0, 0, keys, krows)], say, part_rows=512)
    return dict(gpu=gpu, rows_by_head=rows_by_head, keys=keys, rref=rref, kref=kref)


@pytest.mark.parametrize("precise", [m[0] for m in MODES])
def test_max_seq_len_segments(segments_case, precise):
    say(f"[limits] L={MAX_SEQ_LEN_SEGMENTS} segments, precise={precise}")
    c = segments_case
    compare(SEGMENTS, c["gpu"], c["rows_by_head"], c["keys"], c["rref"], c["kref"], precise)
