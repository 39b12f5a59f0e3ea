"""Thin Python binding of libattn.so (blockwise online-softmax attention, gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/attn.h.  PyTorch provides device
memory and the current HIP stream.  There is no fallback: if the library is
missing or the tensors are not on the GPU, the calls raise.

Names mirror the C ABI: attn_fwd, attn_bwd_preprocess, attn_bwd_dq,
attn_bwd_dkv, attn_bwd_ds_workspace_size, attn_bwd_dkv_ds, attn_bwd_dq_ds,
attn_bwd_ds_static, attn_reduce_heads, attn_ranker_bounds, attn_plan_count,
attn_check_params, and the measurement helper attn_probe_stream.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")

ATTN_F32, ATTN_BF16 = 0, 1
CAP_CODES = {"none": 0, "tanh": 1, "soft_sign": 2, "alsc": 3}
STATUS_NAMES = {0: "ATTN_OK", -1: "ATTN_ERR_NULL_PTR", -2: "ATTN_ERR_SHAPE", -3: "ATTN_ERR_DTYPE",
                -4: "ATTN_ERR_UNSUPPORTED", -5: "ATTN_ERR_ALIGN", -6: "ATTN_ERR_PARAM",
                -7: "ATTN_ERR_HIP"}


class AttnError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {detail}")


class _CParams(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("seq_len", ctypes.c_int32),
                ("q_heads", ctypes.c_int32), ("kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("sm_scale", ctypes.c_float), ("causal", ctypes.c_int32),
                ("window_len", ctypes.c_int32), ("cap_method", ctypes.c_int32),
                ("cap", ctypes.c_float), ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("z_loss_weight", ctypes.c_float), ("precise_ds", ctypes.c_int32)]


@dataclasses.dataclass
class AttnParams:
    batch: int
    seq_len: int
    q_heads: int
    kv_heads: int
    head_dim: int
    dtype: int = ATTN_BF16
    sm_scale: float = 1.0
    causal: bool = False
    window_len: int = 0
    cap_method: int = 0
    cap: float = 0.0
    alpha: float = 0.0
    beta: float = 0.0
    z_loss_weight: float = 0.0
    precise_ds: bool = True

    def to_c(self) -> _CParams:
        return _CParams(int(self.batch), int(self.seq_len), int(self.q_heads), int(self.kv_heads),
                        int(self.head_dim), int(self.dtype), float(self.sm_scale),
                        int(bool(self.causal)), int(self.window_len), int(self.cap_method),
                        float(self.cap), float(self.alpha), float(self.beta),
                        float(self.z_loss_weight), int(bool(self.precise_ds)))


_lib = None
_P = ctypes.c_void_p
_FN_SIGS = {
    "attn_fwd": [ctypes.POINTER(_CParams), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "attn_bwd_preprocess": [ctypes.POINTER(_CParams), _P, _P, _P, _P],
    "attn_bwd_dq": [ctypes.POINTER(_CParams), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "attn_reduce_heads": [ctypes.POINTER(_CParams), _P, _P, _P],
    "attn_ranker_bounds": [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P, _P],
    "attn_probe_stream": [_P, ctypes.c_int64, ctypes.c_int32, _P, _P],
    "attn_bwd_dkv": [ctypes.POINTER(_CParams), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P],
    "attn_plan_count": [ctypes.POINTER(_CParams), _P, _P, ctypes.POINTER(ctypes.c_int64),
                        ctypes.POINTER(ctypes.c_int64)],
    "attn_check_params": [ctypes.POINTER(_CParams)],
    "attn_bwd_ds_workspace_size": [ctypes.POINTER(_CParams), ctypes.POINTER(ctypes.c_uint64)],
    "attn_bwd_dkv_ds": [ctypes.POINTER(_CParams), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                        ctypes.c_uint64, _P],
    "attn_bwd_dq_ds": [ctypes.POINTER(_CParams), _P, _P, _P, _P, ctypes.c_uint64, _P, _P],
    "attn_bwd_ds_static": [ctypes.POINTER(_CParams), _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P,
                           _P, _P],
}

# Size of the library's fixed stored-dS array (include/attn.h, ATTN_STATIC_DS_BYTES).
ATTN_STATIC_DS_BYTES = 128 << 20


def load_library(path: str = LIB_PATH):
    """Load libattn.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} not found: build it with "
                           "`python -m blockwise_softmax_attention_amd.build`")
    lib = ctypes.CDLL(path)
    for name, args in _FN_SIGS.items():
        fn = getattr(lib, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    for name in ("attn_status_str", "attn_last_error", "attn_build_info"):
        getattr(lib, name).restype = ctypes.c_char_p
    lib.attn_status_str.argtypes = [ctypes.c_int]
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise AttnError(status, load_library().attn_last_error().decode())


def _ptr(t: Optional[torch.Tensor], name: str, dtype=None, device_required=True):
    if t is None:
        return None
    if device_required and t.device.type != "cuda":
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> int:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


def _in_dtype(p: AttnParams):
    return torch.bfloat16 if p.dtype == ATTN_BF16 else torch.float32


def attn_check_params(p: AttnParams) -> None:
    cp = p.to_c()
    _check(load_library().attn_check_params(ctypes.byref(cp)))


def attn_fwd(p: AttnParams, q, k, v, temperature=None, segment_ids=None, ranker_bounds=None,
             o=None, m=None, l=None, stream=None):
    """Returns (o, m, l); allocates the outputs it is not given."""
    B, L, Hq, D = p.batch, p.seq_len, p.q_heads, p.head_dim
    dev = q.device
    o = torch.empty((B, L, Hq, D), dtype=torch.float32, device=dev) if o is None else o
    m = torch.empty((B, Hq, L), dtype=torch.float32, device=dev) if m is None else m
    l = torch.empty((B, Hq, L), dtype=torch.float32, device=dev) if l is None else l
    dt = _in_dtype(p)
    cp = p.to_c()
    _check(load_library().attn_fwd(
        ctypes.byref(cp), _ptr(q, "q", dt), _ptr(k, "k", dt), _ptr(v, "v", dt),
        _ptr(temperature, "temperature", torch.float32), _ptr(segment_ids, "segment_ids", torch.int32),
        _ptr(ranker_bounds, "ranker_bounds", torch.int32), _ptr(o, "o", torch.float32),
        _ptr(m, "m", torch.float32), _ptr(l, "l", torch.float32), _stream(stream)))
    return o, m, l


def attn_bwd_preprocess(p: AttnParams, o, d_o, delta=None, stream=None):
    delta = torch.empty((p.batch, p.q_heads, p.seq_len), dtype=torch.float32,
                        device=o.device) if delta is None else delta
    cp = p.to_c()
    _check(load_library().attn_bwd_preprocess(
        ctypes.byref(cp), _ptr(o, "o", torch.float32), _ptr(d_o, "d_o", _in_dtype(p)),
        _ptr(delta, "delta", torch.float32), _stream(stream)))
    return delta


def attn_bwd_dq(p: AttnParams, q, k, v, d_o, m, l, delta, temperature=None, segment_ids=None,
                ranker_bounds=None, dq=None, dtemp_h=None, stream=None):
    """Returns dq; with a (B, Hq, L) float tensor dtemp_h (or dtemp_h=True to
    allocate one) also fills each head's share of the temperature gradient
    and returns (dq, dtemp_h)."""
    dq = torch.empty((p.batch, p.seq_len, p.q_heads, p.head_dim), dtype=torch.float32,
                     device=q.device) if dq is None else dq
    want = dtemp_h is not None and dtemp_h is not False
    if dtemp_h is True:
        dtemp_h = torch.empty((p.batch, p.q_heads, p.seq_len), dtype=torch.float32, device=q.device)
    dt = _in_dtype(p)
    cp = p.to_c()
    _check(load_library().attn_bwd_dq(
        ctypes.byref(cp), _ptr(q, "q", dt), _ptr(k, "k", dt), _ptr(v, "v", dt),
        _ptr(temperature, "temperature", torch.float32), _ptr(segment_ids, "segment_ids", torch.int32),
        _ptr(ranker_bounds, "ranker_bounds", torch.int32), _ptr(d_o, "d_o", dt),
        _ptr(m, "m", torch.float32), _ptr(l, "l", torch.float32), _ptr(delta, "delta", torch.float32),
        _ptr(dq, "dq", torch.float32), _ptr(dtemp_h if want else None, "dtemp_h", torch.float32),
        _stream(stream)))
    return (dq, dtemp_h) if want else dq


def attn_reduce_heads(p: AttnParams, x, out=None, stream=None):
    """out (B, L) = sum over the Hq heads of x (B, Hq, L), in head order."""
    out = torch.empty((p.batch, p.seq_len), dtype=torch.float32, device=x.device) if out is None else out
    cp = p.to_c()
    _check(load_library().attn_reduce_heads(ctypes.byref(cp), _ptr(x, "x", torch.float32),
                                            _ptr(out, "out", torch.float32), _stream(stream)))
    return out


def attn_ranker_bounds(segment_ids, history_id: int, candidate_id: int, out=None, stream=None):
    """Ranker bounds (B, 4) int32 from segment ids (B, L) int32 on the GPU."""
    B, L = segment_ids.shape
    out = torch.empty((B, 4), dtype=torch.int32, device=segment_ids.device) if out is None else out
    _check(load_library().attn_ranker_bounds(
        _ptr(segment_ids, "segment_ids", torch.int32), int(B), int(L), int(history_id),
        int(candidate_id), _ptr(out, "ranker_bounds", torch.int32), _stream(stream)))
    return out


def attn_probe_stream(src, blocks: int, out=None, stream=None):
    """Measurement helper: blocks work-groups stream src (a contiguous device
    tensor, nbytes a multiple of 1024 * blocks) into LDS with the kernels'
    direct-to-LDS loads; out (blocks,) float32 gets the first float of each
    slice's last 1 KB."""
    if not src.is_contiguous():
        raise ValueError("src must be contiguous")
    out = torch.empty((blocks,), dtype=torch.float32, device=src.device) if out is None else out
    _check(load_library().attn_probe_stream(_ptr(src, "src"), int(src.numel() * src.element_size()),
                                            int(blocks), _ptr(out, "out", torch.float32), _stream(stream)))
    return out


def attn_bwd_dkv(p: AttnParams, q, k, v, d_o, m, l, delta, temperature=None, segment_ids=None,
                 ranker_bounds=None, dk=None, dv=None, stream=None):
    shape = (p.batch, p.seq_len, p.kv_heads, p.head_dim)
    dk = torch.empty(shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(shape, dtype=torch.float32, device=q.device) if dv is None else dv
    dt = _in_dtype(p)
    cp = p.to_c()
    _check(load_library().attn_bwd_dkv(
        ctypes.byref(cp), _ptr(q, "q", dt), _ptr(k, "k", dt), _ptr(v, "v", dt),
        _ptr(temperature, "temperature", torch.float32), _ptr(segment_ids, "segment_ids", torch.int32),
        _ptr(ranker_bounds, "ranker_bounds", torch.int32), _ptr(d_o, "d_o", dt),
        _ptr(m, "m", torch.float32), _ptr(l, "l", torch.float32), _ptr(delta, "delta", torch.float32),
        _ptr(dk, "dk", torch.float32), _ptr(dv, "dv", torch.float32), _stream(stream)))
    return dk, dv


def attn_bwd_ds_workspace_size(p: AttnParams) -> int:
    """Bytes of the stored-dS workspace (bf16 inputs, precise_ds off)."""
    n = ctypes.c_uint64(0)
    cp = p.to_c()
    _check(load_library().attn_bwd_ds_workspace_size(ctypes.byref(cp), ctypes.byref(n)))
    return int(n.value)


def ds_workspace(p: AttnParams, device) -> torch.Tensor:
    """A workspace tensor for attn_bwd_dkv_ds / attn_bwd_dq_ds."""
    return torch.empty(attn_bwd_ds_workspace_size(p), dtype=torch.uint8, device=device)


def attn_bwd_dkv_ds(p: AttnParams, q, k, v, d_o, m, l, delta, ds, temperature=None, segment_ids=None,
                    ranker_bounds=None, dk=None, dv=None, stream=None):
    """dK, dV as attn_bwd_dkv, and dS stored into the workspace ds."""
    shape = (p.batch, p.seq_len, p.kv_heads, p.head_dim)
    dk = torch.empty(shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(shape, dtype=torch.float32, device=q.device) if dv is None else dv
    dt = _in_dtype(p)
    cp = p.to_c()
    _check(load_library().attn_bwd_dkv_ds(
        ctypes.byref(cp), _ptr(q, "q", dt), _ptr(k, "k", dt), _ptr(v, "v", dt),
        _ptr(temperature, "temperature", torch.float32), _ptr(segment_ids, "segment_ids", torch.int32),
        _ptr(ranker_bounds, "ranker_bounds", torch.int32), _ptr(d_o, "d_o", dt),
        _ptr(m, "m", torch.float32), _ptr(l, "l", torch.float32), _ptr(delta, "delta", torch.float32),
        _ptr(dk, "dk", torch.float32), _ptr(dv, "dv", torch.float32), _ptr(ds, "ds", torch.uint8),
        int(ds.numel()), _stream(stream)))
    return dk, dv


def attn_bwd_dq_ds(p: AttnParams, k, ds, segment_ids=None, ranker_bounds=None, dq=None, stream=None):
    """dQ = dS K from the workspace written by attn_bwd_dkv_ds."""
    dq = torch.empty((p.batch, p.seq_len, p.q_heads, p.head_dim), dtype=torch.float32,
                     device=k.device) if dq is None else dq
    cp = p.to_c()
    _check(load_library().attn_bwd_dq_ds(
        ctypes.byref(cp), _ptr(k, "k", _in_dtype(p)), _ptr(segment_ids, "segment_ids", torch.int32),
        _ptr(ranker_bounds, "ranker_bounds", torch.int32), _ptr(ds, "ds", torch.uint8),
        int(ds.numel()), _ptr(dq, "dq", torch.float32), _stream(stream)))
    return dq


def attn_bwd_ds_static(p: AttnParams, q, k, v, d_o, m, l, delta, temperature=None, segment_ids=None,
                       ranker_bounds=None, dq=None, dk=None, dv=None, stream=None):
    """The stored-dS backward with the library's fixed dS array as its
    workspace (the C entry point allocates nothing; outputs not given are
    allocated here by torch).  Returns (dq, dk, dv)."""
    dq = torch.empty((p.batch, p.seq_len, p.q_heads, p.head_dim), dtype=torch.float32,
                     device=q.device) if dq is None else dq
    shape = (p.batch, p.seq_len, p.kv_heads, p.head_dim)
    dk = torch.empty(shape, dtype=torch.float32, device=q.device) if dk is None else dk
    dv = torch.empty(shape, dtype=torch.float32, device=q.device) if dv is None else dv
    dt = _in_dtype(p)
    cp = p.to_c()
    _check(load_library().attn_bwd_ds_static(
        ctypes.byref(cp), _ptr(q, "q", dt), _ptr(k, "k", dt), _ptr(v, "v", dt),
        _ptr(temperature, "temperature", torch.float32), _ptr(segment_ids, "segment_ids", torch.int32),
        _ptr(ranker_bounds, "ranker_bounds", torch.int32), _ptr(d_o, "d_o", dt),
        _ptr(m, "m", torch.float32), _ptr(l, "l", torch.float32), _ptr(delta, "delta", torch.float32),
        _ptr(dq, "dq", torch.float32), _ptr(dk, "dk", torch.float32), _ptr(dv, "dv", torch.float32),
        _stream(stream)))
    return dq, dk, dv


def stored_ds_eligible(p: AttnParams, dtemp: bool = False) -> bool:
    """The stored-dS backward applies: bf16 inputs, single-bf16 dS, no
    temperature gradient (which the recomputing dQ kernel forms)."""
    return p.dtype == ATTN_BF16 and not p.precise_ds and not dtemp


# Largest stored-dS workspace attention_forward_backward allocates on its own
# (16 GiB, about 6% of one GPU's 288 GB).  The workspace grows with the number
# of visited 128 x 128 blocks, i.e. with L^2 (8.6 GB for 8 causal heads at
# L = 32768, ~137 GB at L = 131072); beyond this cap the recomputing dQ
# (O(L) memory, as the pages' backward) is taken unless the caller asks for
# the stored-dS path or hands in a workspace.
STORED_DS_AUTO_MAX_BYTES = 16 << 30


def stored_ds_auto(p: AttnParams, dtemp: bool = False,
                   max_bytes: int = STORED_DS_AUTO_MAX_BYTES) -> bool:
    """Whether attention_forward_backward takes the stored-dS backward when the
    caller leaves the choice to it: eligible, and its workspace fits max_bytes."""
    return stored_ds_eligible(p, dtemp) and attn_bwd_ds_workspace_size(p) <= max_bytes


def attn_plan_count(p: AttnParams, segment_ids=None, ranker_bounds=None):
    """(unmasked pairs, visited forward tiles), both summed over batch and heads.
    Host-side; segment_ids / ranker_bounds are CPU int32 tensors or None."""
    import numpy as np

    def host(t):
        if t is None:
            return None, None
        a = np.ascontiguousarray(t.cpu().numpy() if isinstance(t, torch.Tensor) else t, dtype=np.int32)
        return a, a.ctypes.data

    seg, seg_p = host(segment_ids)
    rb, rb_p = host(ranker_bounds)
    pairs, tiles = ctypes.c_int64(0), ctypes.c_int64(0)
    cp = p.to_c()
    _check(load_library().attn_plan_count(ctypes.byref(cp), seg_p, rb_p, ctypes.byref(pairs),
                                          ctypes.byref(tiles)))
    del seg, rb
    return pairs.value, tiles.value


def attention_forward_backward(p: AttnParams, q, k, v, d_o, temperature=None, segment_ids=None,
                               ranker_bounds=None, dtemp: bool = False, stream=None,
                               stored_ds: Optional[bool] = None, ds=None):
    """One pass of the whole path: forward, then preprocess, dQ and dK/dV
    (and, with dtemp=True, the temperature gradient (B, L)).  stored_ds: use
    the stored-dS backward (dK/dV, then dQ from the stored dS); None picks it
    when it applies and either a workspace ds is given or the one it would
    allocate fits STORED_DS_AUTO_MAX_BYTES (stored_ds_auto), else the
    recomputing dQ.  ds: a workspace to reuse (uint8, at least
    attn_bwd_ds_workspace_size bytes); one is allocated if not given."""
    if stored_ds is None:
        stored_ds = stored_ds_eligible(p, dtemp) if ds is not None else stored_ds_auto(p, dtemp)
    o, m, l = attn_fwd(p, q, k, v, temperature, segment_ids, ranker_bounds, stream=stream)
    delta = attn_bwd_preprocess(p, o, d_o, stream=stream)
    if stored_ds:
        if dtemp:
            raise ValueError("the temperature gradient needs the recomputing dQ (stored_ds=False)")
        if ds is None:
            ds = ds_workspace(p, q.device)
        dk, dv = attn_bwd_dkv_ds(p, q, k, v, d_o, m, l, delta, ds, temperature, segment_ids,
                                 ranker_bounds, stream=stream)
        dq = attn_bwd_dq_ds(p, k, ds, segment_ids, ranker_bounds, stream=stream)
        dtemp_h = None
    else:
        res = attn_bwd_dq(p, q, k, v, d_o, m, l, delta, temperature, segment_ids, ranker_bounds,
                          dtemp_h=True if dtemp else None, stream=stream)
        dq, dtemp_h = res if dtemp else (res, None)
        dk, dv = attn_bwd_dkv(p, q, k, v, d_o, m, l, delta, temperature, segment_ids, ranker_bounds,
                              stream=stream)
    out = dict(o=o, m=m, l=l, delta=delta, dq=dq, dk=dk, dv=dv)
    if dtemp:
        out["dtemp_h"] = dtemp_h
        out["dtemp"] = attn_reduce_heads(p, dtemp_h, stream=stream)
    return out


def params_for(w, precise_ds: bool = True) -> AttnParams:
    """AttnParams of a workloads.Workload description."""
    return AttnParams(batch=w.B, seq_len=w.L, q_heads=w.Hq, kv_heads=w.Hkv, head_dim=w.D,
                      dtype=ATTN_BF16 if w.dtype == "bf16" else ATTN_F32, sm_scale=w.sm_scale,
                      causal=w.causal, window_len=w.window_len,
                      cap_method=CAP_CODES[w.cap_method], cap=w.cap, alpha=w.alpha, beta=w.beta,
                      z_loss_weight=w.z_loss_weight, precise_ds=precise_ds)
