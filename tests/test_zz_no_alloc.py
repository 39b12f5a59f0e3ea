"""The allocation-free stored-dS backward (attn_bwd_ds_static) against the
stored-dS pair with a caller workspace (attn_bwd_dkv_ds + attn_bwd_dq_ds):
the same kernels, so dQ, dK and dV must agree bit for bit, on two calls in a
row (the second smaller, over the first call's leftover array contents), and
both meet the oracle's bf16 bars."""
import numpy as np
import pytest
import torch

import blockwise_softmax_attention_amd as ba
from oracle import backward
from workloads import WORKLOADS, make_inputs

from test_gpu_parity import check_tensor, host_inputs, oracle_params, say

pytestmark = [pytest.mark.gpu, pytest.mark.filterwarnings("ignore::RuntimeWarning")]


def one_call(w):
    p = ba.params_for(w, precise_ds=False)
    assert ba.attn_bwd_ds_workspace_size(p) <= ba.ATTN_STATIC_DS_BYTES
    inp = make_inputs(w)
    d = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
    o, m, l = ba.attn_fwd(p, d["q"], d["k"], d["v"], d["temperature"], d["segment_ids"],
                          d["ranker_bounds"])
    delta = ba.attn_bwd_preprocess(p, o, d["do"])
    dq, dk, dv = ba.attn_bwd_ds_static(p, d["q"], d["k"], d["v"], d["do"], m, l, delta,
                                       d["temperature"], d["segment_ids"], d["ranker_bounds"])
    ws = ba.ds_workspace(p, "cuda")
    rk, rv = ba.attn_bwd_dkv_ds(p, d["q"], d["k"], d["v"], d["do"], m, l, delta, ws, d["temperature"],
                                d["segment_ids"], d["ranker_bounds"])
    rq = ba.attn_bwd_dq_ds(p, d["k"], ws, d["segment_ids"], d["ranker_bounds"])
    torch.cuda.synchronize()
    for name, a, b in (("dq", dq, rq), ("dk", dk, rk), ("dv", dv, rv)):
        assert torch.equal(a, b), name
    say(f"[no-alloc] {w.name} B{w.B} Hq{w.Hq} L{w.L}: dq, dk, dv bit-identical to the pair")
    return inp, {"dq": dq, "dk": dk, "dv": dv}


def test_static_matches_caller_workspace_two_calls():
    big = WORKLOADS[2]                         # B2 Hq8 L2048, 68 MiB of the array
    small = WORKLOADS[2].scaled(L=900, B=1, Hq=4, Hkv=4)
    for w in (big, small):
        inp, got = one_call(w)
        h = host_inputs(inp)
        ref = backward(h["q"], h["k"], h["v"], h["do"], oracle_params(w), h["temp"], h["seg"],
                       h["rb"])
        for n in ("dq", "dk", "dv"):
            check_tensor(n, got[n].cpu().double().numpy(), ref[n], "bf16")


def test_static_rejects_beyond_its_array():
    w = WORKLOADS[5].scaled(L=8192, Hq=2, Hkv=2)
    p = ba.params_for(w, precise_ds=False)
    assert ba.attn_bwd_ds_workspace_size(p) > ba.ATTN_STATIC_DS_BYTES
    x = torch.zeros(16, dtype=torch.bfloat16, device="cuda")
    f = torch.zeros(16, dtype=torch.float32, device="cuda")
    with pytest.raises(ba.AttnError) as e:
        ba.attn_bwd_ds_static(p, x, x, x, x, f, f, f, dq=f, dk=f, dv=f)
    assert e.value.status == -2
