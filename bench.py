"""Benchmark: attention forward + backward TFLOP/s (unmasked FLOPs) on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
attn_fwd, attn_bwd_preprocess, then the stored-dS backward (attn_bwd_dkv_ds,
attn_bwd_dq_ds) where it applies, else attn_bwd_dq + attn_bwd_dkv.  FLOPs
count only visible (query, key) pairs (exact count from attn_plan_count):
forward 4 D per pair per query head, backward 10 D.

The headline line is the long-context workload (B1 Hq8 L32768 D128, causal,
ALSC cap) through the stored-dS backward.  The same run then times, after
the headline's timed region, the recomputing backward (preprocess +
attn_bwd_dq + attn_bwd_dkv: O(L) memory, no stored dS) on the same inputs
("recompute_bwd") and the ranker GQA workload (B4 Hq16 Hkv4 L8192, soft-sign
cap) in both backward modes ("ranker_gqa").

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload 5]
                    [--no-cpu-baseline] [--headline-only] [--precise-ds 0|1]

Prints one JSON line.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd+bwd TFLOP/s (unmasked FLOPs) and % bf16 MFMA peak, 1 GPU"
PEAK_BF16_TFLOPS = 2516.6      # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 flop/clk/CU)
PEAK_F32_TFLOPS = 157.3        # fp32 (matrix and vector)
HBM_GBPS = 8000.0

# HBM bytes per launch measured with rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE on the
# long-context and ranker workloads (default mode: single-bf16 dS, stored-dS
# backward), scaled by what the same counters read for a plain 1 GiB device
# copy (FETCH_SIZE x2.0, WRITE_SIZE x1.0); keyed by a hash of the kernel
# sources they were taken on, so a changed kernel reports null (the key was
# moved once for an edit that left the device assembly byte-identical).  Summary and
# commands: profiles/counters_long_context_causal_alsc_L32768.md and
# profiles/kernel_trace_ranker_gqa_softsign_L8192.md.
KERNEL_SOURCES = ["attn_bf16.hip", "attn_bf16.h", "attn_device.h", "attn_tiles.h",
                  "attn_internal.h", "attn_bwd_common.h", "attn_preprocess.hip"]
MEASURED_TRAFFIC = {
    ("be66c260ca48d300", 5, 0): {"attn_fwd": (237641 * 2.0 + 133989) * 1024,
                                 "attn_bwd_preprocess": (98333 * 2.0 + 4097) * 1024,
                                 "attn_bwd_dkv_ds": (362220 * 2.0 + 8683520) * 1024,
                                 "attn_bwd_dq_ds": (4353492 * 2.0 + 131273) * 1024},
    ("be66c260ca48d300", 4, 0): {"attn_fwd": (171941 * 2.0 + 270478) * 1024,
                                 "attn_bwd_preprocess": (196638 * 2.0 + 16402) * 1024,
                                 "attn_bwd_dkv_ds": (1036320 * 2.0 + 6423051) * 1024,
                                 "attn_bwd_dq_ds": (3207965 * 2.0 + 262161) * 1024},
}


def kernel_source_hash() -> str:
    """Hash of the kernel sources' code and their per-source compiler flags:
    comments and whitespace are dropped, so an edited comment keeps the
    measured traffic, a changed kernel not."""
    import hashlib
    import re
    from blockwise_softmax_attention_amd.build import SOURCE_FLAGS
    h = hashlib.sha256()
    h.update(repr(sorted(SOURCE_FLAGS.items())).encode())
    for f in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "blockwise_softmax_attention_amd", "csrc", f)) as fh:
            src = fh.read()
        src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
        src = re.sub(r"//[^\n]*", " ", src)
        h.update(" ".join(src.split()).encode())
    return h.hexdigest()[:16]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5, help="workload number 1..5")
    ap.add_argument("--precise-ds", type=int, default=-1,
                    help="1: hi+lo bf16 P and dS; 0: single bf16; -1 (default): 0 for the "
                         "workloads whose full-size parity tests run in that mode (4, 5), else 1")
    ap.add_argument("--stored-ds", type=int, default=-1,
                    help="1: stored-dS backward (dK/dV stores dS, dQ = dS K); 0: recomputing dQ; "
                         "-1 (default): 1 wherever it applies (bf16, single-bf16 dS)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline path (no recomputing-backward or ranker lines)")
    ap.add_argument("--cpu-sample-len", type=int, default=16384,
                    help="prefix length of the oracle's bounded sample")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (HBM counter "
                         "calibration) and exit")
    ap.add_argument("--hbm-probe", type=int, default=0, metavar="MIB",
                    help="only time torch's own streaming kernels (sum, copy, fill) on MIB MiB "
                         "as a reference for the HBM rate this chip sustains, and exit")
    ap.add_argument("--stream-probe", type=int, default=0, metavar="MIB",
                    help="only time attn_probe_stream (the kernels' direct-to-LDS loads "
                         "streaming MIB MiB from HBM) as a reference for the read rate "
                         "those loads reach, and exit")
    ap.add_argument("--gemm-probe", type=int, default=0, metavar="N",
                    help="only time the vendor bf16 GEMM (torch.matmul, N x N x N) as a "
                         "reference for the MFMA rate this chip sustains, and exit")
    return ap.parse_args()


def cpu_threads() -> tuple:
    """(threads the oracle's BLAS may use, cores in this process's affinity
    set): the affinity count, capped by OMP_NUM_THREADS where that is set."""
    aff = len(os.sched_getaffinity(0))
    env = os.environ.get("OMP_NUM_THREADS", "")
    n = min(aff, int(env)) if env.isdigit() and int(env) > 0 else aff
    return n, aff


def cpu_baseline(w, sample_len: int):
    """The fp64 oracle, as is, on a bounded sample of the workload: batch 0,
    query head 0 (its KV head), the first `sample_len` positions.  The forward
    alone, then the backward (which recomputes the forward it needs); rate =
    counted FLOPs (4 D + 10 D per visible pair) / the backward call's wall time."""
    from oracle import Params, backward, forward, unmasked_pairs
    from workloads import make_inputs, to_f64, to_i32
    threads, aff = cpu_threads()
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=threads)
    except Exception:  # pragma: no cover
        limiter = None
    ws = w.scaled(L=min(sample_len, w.L), B=1, Hq=1, Hkv=1)
    inp = make_inputs(ws)
    q, k, v, do = (to_f64(inp[n]) for n in ("q", "k", "v", "do"))
    temp, seg, rb = to_f64(inp["temperature"]), to_i32(inp["segment_ids"]), to_i32(inp["ranker_bounds"])
    p = Params(w.sm_scale, w.causal, w.window_len, w.cap_method, w.cap, w.alpha, w.beta,
               w.z_loss_weight)
    t0 = time.perf_counter()
    forward(q, k, v, p, temp, seg, rb)
    t_fwd = time.perf_counter() - t0
    t0 = time.perf_counter()
    backward(q, k, v, do, p, temp, seg, rb)
    t_all = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    pairs = unmasked_pairs(ws.L, p, seg, rb, B=1)
    flops = 14.0 * w.D * pairs
    return {"value": flops / t_all / 1e12, "unit": "TFLOP/s", "cores": int(threads), "kind": "oracle",
            "sample": f"batch 0, head 0, first {ws.L} positions of the workload in fp64 "
                      f"({pairs} visible pairs): forward {t_fwd:.1f} s alone; backward call "
                      f"(forward + gradients) {t_all:.1f} s",
            "fwd_seconds": round(t_fwd, 3), "bwd_seconds": round(max(t_all - t_fwd, 0.0), 3),
            "seconds": round(t_all, 3), "affinity_cores": aff}


class Path:
    """Device buffers and the launch sequence of one workload: forward,
    preprocess, then either the stored-dS pair or the recomputing dQ + dK/dV."""

    def __init__(self, w, precise: bool):
        import torch
        import blockwise_softmax_attention_amd as ba
        from workloads import make_inputs
        self.ba, self.torch, self.w = ba, torch, w
        inp = make_inputs(w)
        dev = {k: (v.cuda() if v is not None else None) for k, v in inp.items()}
        self.p = ba.params_for(w, precise_ds=precise)
        self.pairs, _ = ba.attn_plan_count(self.p, inp["segment_ids"], inp["ranker_bounds"])
        B, L, Hq, Hkv, D = w.B, w.L, w.Hq, w.Hkv, w.D
        f32 = dict(dtype=torch.float32, device="cuda")
        self.o = torch.empty((B, L, Hq, D), **f32)
        self.m = torch.empty((B, Hq, L), **f32)
        self.l = torch.empty((B, Hq, L), **f32)
        self.delta = torch.empty((B, Hq, L), **f32)
        self.dq = torch.empty((B, L, Hq, D), **f32)
        self.dk = torch.empty((B, L, Hkv, D), **f32)
        self.dv = torch.empty((B, L, Hkv, D), **f32)
        self.q, self.k, self.v, self.do = dev["q"], dev["k"], dev["v"], dev["do"]
        self.temp, self.seg, self.rb = dev["temperature"], dev["segment_ids"], dev["ranker_bounds"]
        self.ws = None
        self.stream = torch.cuda.current_stream()

    def names(self, stored: bool):
        return (["attn_fwd", "attn_bwd_preprocess", "attn_bwd_dkv_ds", "attn_bwd_dq_ds"] if stored else
                ["attn_fwd", "attn_bwd_preprocess", "attn_bwd_dq", "attn_bwd_dkv"])

    def step(self, stored: bool, ev=None):
        ba, p, s = self.ba, self.p, self.stream
        if stored and self.ws is None:
            self.ws = ba.ds_workspace(p, "cuda")
        rec = (lambda i: ev[i].record(s)) if ev is not None else (lambda i: None)
        rec(0)
        ba.attn_fwd(p, self.q, self.k, self.v, self.temp, self.seg, self.rb, self.o, self.m, self.l,
                    stream=s)
        rec(1)
        ba.attn_bwd_preprocess(p, self.o, self.do, self.delta, stream=s)
        rec(2)
        if stored:
            ba.attn_bwd_dkv_ds(p, self.q, self.k, self.v, self.do, self.m, self.l, self.delta, self.ws,
                               self.temp, self.seg, self.rb, self.dk, self.dv, stream=s)
            rec(3)
            ba.attn_bwd_dq_ds(p, self.k, self.ws, self.seg, self.rb, self.dq, stream=s)
        else:
            ba.attn_bwd_dq(p, self.q, self.k, self.v, self.do, self.m, self.l, self.delta, self.temp,
                           self.seg, self.rb, self.dq, stream=s)
            rec(3)
            ba.attn_bwd_dkv(p, self.q, self.k, self.v, self.do, self.m, self.l, self.delta, self.temp,
                            self.seg, self.rb, self.dk, self.dv, stream=s)
        rec(4)

    def measure(self, stored: bool, steps: int, warmup: int):
        """Per-kernel average ms (HIP events on the launch stream) and the wall
        time of `steps` steps bracketed by synchronisation."""
        torch = self.torch
        for _ in range(warmup):
            self.step(stored)
        torch.cuda.synchronize()
        evs = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            self.step(stored, evs[i])
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        names = self.names(stored)
        avg = {n: sum(e[j].elapsed_time(e[j + 1]) for e in evs) / steps for j, n in enumerate(names)}
        return avg, wall * 1e3 / steps

    def summary(self, avg, peak):
        D = self.w.D
        fwd_flop, bwd_flop = 4.0 * D * self.pairs, 10.0 * D * self.pairs
        names = list(avg)
        fwd_ms = avg["attn_fwd"]
        bwd_ms = sum(avg[n] for n in names[1:])
        return {
            "fwd": {"ms": round(fwd_ms, 4), "tflops": round(fwd_flop / (fwd_ms * 1e-3) / 1e12, 2),
                    "pct_peak": round(100.0 * fwd_flop / (fwd_ms * 1e-3) / 1e12 / peak, 2)},
            "bwd": {"ms": round(bwd_ms, 4), "tflops": round(bwd_flop / (bwd_ms * 1e-3) / 1e12, 2),
                    "pct_peak": round(100.0 * bwd_flop / (bwd_ms * 1e-3) / 1e12 / peak, 2)},
            "kernels_ms": {n: round(avg[n], 4) for n in names},
        }


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the benchmark runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch
    import blockwise_softmax_attention_amd as ba
    from workloads import WORKLOADS

    torch.cuda.set_device(0)
    if args.copy_probe:
        n = args.copy_probe * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_probe_bytes": n * 4}), flush=True)
        return
    if args.hbm_probe:
        n = args.hbm_probe * (1 << 20) // 4
        x = torch.ones(n, dtype=torch.float32, device="cuda")
        y = torch.empty_like(x)

        def rate(fn, nbytes, reps=10):
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                fn()
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            return {"ms": round(ms, 4), "tb_per_s": round(nbytes / (ms * 1e-3) / 1e12, 2)}

        print(json.dumps({"hbm_probe_bytes": n * 4,
                          "sum_read": rate(lambda: x.sum(), n * 4),
                          "copy_read_write": rate(lambda: y.copy_(x), 2 * n * 4),
                          "fill_write": rate(lambda: y.fill_(1.0), n * 4)}), flush=True)
        return
    if args.stream_probe:
        nbytes = args.stream_probe * (1 << 20)
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        res = {"stream_probe_bytes": nbytes}
        for blocks in (512, 1024, 2048, 4096):
            if nbytes % (1024 * blocks):
                continue
            out = torch.empty(blocks, dtype=torch.float32, device="cuda")
            for _ in range(3):
                ba.attn_probe_stream(src, blocks, out)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            reps = 10
            e0.record()
            for _ in range(reps):
                ba.attn_probe_stream(src, blocks, out)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1) / reps
            res[f"blocks_{blocks}"] = {"ms": round(ms, 4), "tb_per_s": round(nbytes / (ms * 1e-3) / 1e12, 2)}
        print(json.dumps(res), flush=True)
        return
    if args.gemm_probe:
        n = args.gemm_probe
        g = torch.Generator(device="cuda").manual_seed(0)
        a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
        b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16, generator=g)
        for _ in range(5):
            c = a @ b
        torch.cuda.synchronize()
        ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        reps = 20
        ev0.record()
        for _ in range(reps):
            c = a @ b
        ev1.record()
        torch.cuda.synchronize()
        ms = ev0.elapsed_time(ev1) / reps
        tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
        print(json.dumps({"gemm_probe_n": n, "ms": round(ms, 4), "tflops": round(tf, 1),
                          "pct_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2)}), flush=True)
        del c
        return
    w = WORKLOADS[args.workload]
    precise = args.precise_ds if args.precise_ds >= 0 else (0 if args.workload in (4, 5) else 1)
    path = Path(w, bool(precise))
    p, pairs = path.p, path.pairs
    stored = ba.stored_ds_eligible(p) if args.stored_ds < 0 else bool(args.stored_ds)
    names = path.names(stored)
    B, L, Hq, Hkv, D = w.B, w.L, w.Hq, w.Hkv, w.D
    fwd_flop = 4.0 * D * pairs
    bwd_flop = 10.0 * D * pairs
    avg, step_ms = path.measure(stored, args.steps, args.warmup)
    value = (fwd_flop + bwd_flop) / (step_ms * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS

    # Roofline of the dominant kernel: algorithmic MFMA FLOPs per launch over its
    # average duration (HIP events on the launch stream, timed region only).
    # Per visible pair and query head: fwd 4 D (QK^T, PV); dq 6 D (QK^T, dO V^T,
    # dS K); dkv 8 D (QK^T, dO V^T, P^T dO, dS^T Q).  Preprocess is HBM-bound:
    # reads O (f32) and dO, writes delta.
    # With the stored-dS backward the dK/dV kernel does the same MFMA work and
    # dQ = dS K (2 D per pair) streams the stored dS from HBM.
    alg = {"attn_fwd": 4.0 * D * pairs, "attn_bwd_dq": 6.0 * D * pairs,
           "attn_bwd_dkv": 8.0 * D * pairs, "attn_bwd_dkv_ds": 8.0 * D * pairs,
           "attn_bwd_dq_ds": 2.0 * D * pairs}
    dom = max((n for n in names if n in alg), key=lambda n: avg[n])
    achieved = alg[dom] / (avg[dom] * 1e-3) / 1e12
    pre_bytes = B * L * Hq * D * (4 + (2 if w.dtype == "bf16" else 4)) + B * Hq * L * 4
    measured = MEASURED_TRAFFIC.get((kernel_source_hash(), args.workload, precise))
    traffic = None if measured is None else int(measured[dom])
    roofline = {"bound": "mfma", "kernel": dom, "achieved": round(achieved, 2),
                "peak": peak, "unit": "TFLOP/s", "frac": round(achieved / peak, 4),
                "traffic": traffic, "traffic_unit": "bytes per launch (HBM, calibrated)"}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(step_ms, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": w.dtype, "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "seq_len": L, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": D, "cap": w.cap_method, "causal": w.causal, "window": w.window_len,
                   "precise_ds": bool(precise), "stored_ds": stored, "visible_pairs": pairs},
        "pct_peak": round(100.0 * value / peak, 2),
    }
    out.update(path.summary(avg, peak))
    out["preprocess_gbps"] = round(pre_bytes / (avg["attn_bwd_preprocess"] * 1e-3) / 1e9, 1)
    # stored-dS dQ: workspace bytes (every band tile; tiles skipped by a mask
    # are not read, so this bounds the dS bytes streamed) per launch time
    out["dq_ds_gbps"] = (round(path.ws.numel() / (avg["attn_bwd_dq_ds"] * 1e-3) / 1e9, 1)
                         if stored else None)
    out["roofline"] = roofline

    if not args.headline_only:
        # The O(L)-memory backward of the pages (preprocess + recomputing dQ +
        # dK/dV, no stored dS) on the same inputs, timed after the headline.
        if stored:
            ravg, _ = path.measure(False, args.steps, args.warmup)
            r = path.summary(ravg, peak)
            out["recompute_bwd"] = {"workload": w.name, "precise_ds": bool(precise), **r["bwd"],
                                    "kernels_ms": {k: v for k, v in r["kernels_ms"].items()
                                                   if k != "attn_fwd"}}
        if args.workload == 5:
            # the second workload at L >= 8192: ranker mask, GQA, soft-sign cap
            path.ws = None
            del path
            torch.cuda.empty_cache()
            w4 = WORKLOADS[4]
            p4 = Path(w4, False)
            st4 = ba.stored_ds_eligible(p4.p)
            a4, s4 = p4.measure(st4, args.steps, args.warmup)
            r4 = p4.summary(a4, peak)
            ra4, _ = p4.measure(False, args.steps, args.warmup)
            rr4 = p4.summary(ra4, peak)
            alg4 = {"attn_fwd": 4.0 * w4.D * p4.pairs, "attn_bwd_dkv_ds": 8.0 * w4.D * p4.pairs,
                    "attn_bwd_dq_ds": 2.0 * w4.D * p4.pairs, "attn_bwd_dkv": 8.0 * w4.D * p4.pairs,
                    "attn_bwd_dq": 6.0 * w4.D * p4.pairs}
            dom4 = max((n for n in a4 if n in alg4), key=lambda n: a4[n])
            ach4 = alg4[dom4] / (a4[dom4] * 1e-3) / 1e12
            meas4 = MEASURED_TRAFFIC.get((kernel_source_hash(), 4, 0))
            out["ranker_gqa"] = {
                "workload": w4.name, "batch": w4.B, "seq_len": w4.L, "q_heads": w4.Hq,
                "kv_heads": w4.Hkv, "visible_pairs": p4.pairs, "precise_ds": False,
                "stored_ds": st4, "ms_per_step": round(s4, 4),
                "tflops": round(14.0 * w4.D * p4.pairs / (s4 * 1e-3) / 1e12, 2),
                "fwd": r4["fwd"], "bwd": r4["bwd"], "kernels_ms": r4["kernels_ms"],
                "roofline": {"bound": "mfma", "kernel": dom4, "achieved": round(ach4, 2), "peak": peak,
                             "unit": "TFLOP/s", "frac": round(ach4 / peak, 4),
                             "traffic": None if meas4 is None else int(meas4[dom4]),
                             "traffic_unit": "bytes per launch (HBM, calibrated)"},
                "recompute_bwd": {**rr4["bwd"], "kernels_ms": {k: v for k, v in rr4["kernels_ms"].items()
                                                               if k != "attn_fwd"}},
            }
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_sample_len)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
