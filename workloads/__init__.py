"""Seeded synthetic workloads for capped, masked, grouped-query attention.

This module only draws random inputs and describes the five workload shapes.
It contains none of the attention arithmetic: both the fp64 oracle (through the
tests) and the HIP path consume the exact tensors produced here, so the two
sides always see identical fp32/bf16 bits.

Draw order for a workload with seed ``s`` (``numpy.random.default_rng(s)``):
  1. Q (B, L, Hq, D), K (B, L, Hkv, D), V (B, L, Hkv, D), dO (B, L, Hq, D),
     each ``standard_normal(dtype=float32)``, times ``input_scale``;
  2. bf16 workloads round all four once to bf16 (round-to-nearest-even);
  3. per-query temperature (B, L) ``uniform(lo, hi)`` as float32, if any;
  4. segment cut points, per batch row, if the workload packs segments;
  5. ranker history length h per batch row, if the workload uses the ranker
     mask; bounds are then ``[0, h, h, L]`` (history [0, h), candidates [h, L)).
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np
import torch

CAP_CODES = {"none": 0, "tanh": 1, "soft_sign": 2, "alsc": 3}


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    B: int
    Hq: int
    Hkv: int
    L: int
    D: int
    dtype: str                      # "f32" or "bf16": storage type of Q, K, V, dO
    sm_scale: float
    causal: bool
    window_len: int                 # 0: no sliding window
    cap_method: str                 # none | tanh | soft_sign | alsc
    cap: float
    alpha: float = 0.0
    beta: float = 0.0
    z_loss_weight: float = 0.0
    temperature: Optional[tuple] = None   # (lo, hi) for U[lo, hi], None: temperature 1
    n_segments: int = 1             # >1: contiguous packed segments per row
    ranker: Optional[tuple] = None  # (h_lo, h_hi) inclusive range of the history length
    input_scale: float = 1.0

    def scaled(self, **kw) -> "Workload":
        """Same structure at another size (ranker history range scales with L)."""
        w = dataclasses.replace(self, **kw)
        if self.ranker is not None and "L" in kw and "ranker" not in kw:
            lo = self.ranker[0] * w.L // self.L
            hi = self.ranker[1] * w.L // self.L
            w = dataclasses.replace(w, ranker=(lo, hi))
        return w


# The five workloads.  sm_scale for the last three is 1/sqrt(D) (not stated
# with them; 1/sqrt(D) is the scale the backward test on the Mosaic page uses).
WORKLOADS = {
    1: Workload("tiny_causal_tanh_f32", 1, B=1, Hq=1, Hkv=1, L=256, D=64, dtype="f32",
                sm_scale=1.0 / 8.0, causal=True, window_len=0, cap_method="tanh", cap=30.0),
    2: Workload("packed_causal_tanh_bf16", 2, B=2, Hq=8, Hkv=8, L=2048, D=128, dtype="bf16",
                sm_scale=1.0 / math.sqrt(128), causal=True, window_len=0, cap_method="tanh",
                cap=50.0, temperature=(0.5, 1.5), n_segments=4),
    3: Workload("alsc_window512_bf16", 3, B=1, Hq=16, Hkv=16, L=4096, D=128, dtype="bf16",
                sm_scale=1.0 / math.sqrt(128), causal=True, window_len=512, cap_method="alsc",
                cap=30.0, alpha=4.0, beta=0.5, z_loss_weight=1e-4),
    4: Workload("ranker_gqa_softsign_bf16", 4, B=4, Hq=16, Hkv=4, L=8192, D=128, dtype="bf16",
                sm_scale=1.0 / math.sqrt(128), causal=False, window_len=0,
                cap_method="soft_sign", cap=20.0, ranker=(4096, 7168)),
    5: Workload("long_context_causal_alsc_bf16", 5, B=1, Hq=8, Hkv=8, L=32768, D=128,
                dtype="bf16", sm_scale=1.0 / math.sqrt(128), causal=True, window_len=0,
                cap_method="alsc", cap=50.0, alpha=2.0, beta=0.0, z_loss_weight=1e-4,
                temperature=(0.8, 1.2), input_scale=0.5),
}


def make_inputs(w: Workload) -> dict:
    """Draw the seeded inputs of workload ``w`` as CPU torch tensors.

    Returns q, k, v, do in the storage dtype (float32 or bfloat16), temperature
    (B, L) float32 or None, segment_ids (B, L) int32 or None, ranker_bounds
    (B, 4) int32 or None.
    """
    rng = np.random.default_rng(w.seed)
    shapes = [(w.B, w.L, w.Hq, w.D), (w.B, w.L, w.Hkv, w.D), (w.B, w.L, w.Hkv, w.D),
              (w.B, w.L, w.Hq, w.D)]
    arrs = []
    for shp in shapes:
        a = rng.standard_normal(size=shp, dtype=np.float32)
        if w.input_scale != 1.0:
            a = a * np.float32(w.input_scale)
        arrs.append(torch.from_numpy(a))
    if w.dtype == "bf16":
        arrs = [a.to(torch.bfloat16) for a in arrs]
    elif w.dtype != "f32":
        raise ValueError(f"unknown dtype {w.dtype}")
    q, k, v, do = arrs

    temperature = None
    if w.temperature is not None:
        lo, hi = w.temperature
        temperature = torch.from_numpy(
            rng.uniform(lo, hi, size=(w.B, w.L)).astype(np.float32))

    segment_ids = None
    if w.n_segments > 1:
        seg = np.zeros((w.B, w.L), dtype=np.int32)
        for b in range(w.B):
            cuts = np.sort(rng.choice(np.arange(1, w.L), w.n_segments - 1, replace=False))
            for c in cuts:
                seg[b, c:] += 1
        segment_ids = torch.from_numpy(seg)

    ranker_bounds = None
    if w.ranker is not None:
        lo, hi = w.ranker
        rb = np.zeros((w.B, 4), dtype=np.int32)
        for b in range(w.B):
            h = int(rng.integers(lo, hi, endpoint=True))
            rb[b] = (0, h, h, w.L)
        ranker_bounds = torch.from_numpy(rb)

    return dict(q=q, k=k, v=v, do=do, temperature=temperature,
                segment_ids=segment_ids, ranker_bounds=ranker_bounds)


def to_f64(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    """Exact widening of a float32/bfloat16 tensor to a float64 numpy array."""
    if t is None:
        return None
    return t.to(torch.float64).numpy()


def to_i32(t: Optional[torch.Tensor]) -> Optional[np.ndarray]:
    if t is None:
        return None
    return t.numpy().astype(np.int32)
