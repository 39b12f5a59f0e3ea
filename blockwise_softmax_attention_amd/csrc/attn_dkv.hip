// Backward kernels: preprocess (delta), dQ, and dK/dV.
//
// Chain (triton_kernels.py page, make_triton_backward_kernel_dq / _dkv; the
// module docstring of the mosaic_backward.py page): with P recomputed from the
// forward's m and l as P = exp(S' - LSE),
//   dP = dO V^T,  dS' = P (dP - delta) + w P LSE,  dS = dS' temp cap'(s) sm_scale,
//   dQ = dS K,  dK = dS^T Q,  dV = P^T dO,
// where delta = rowsum(O * dO) (mosaic_backward.py page,
// make_preprocess_backward_kernel) and the z-loss term is folded into
// delta' = delta - w LSE, so dS' = P (dP - delta').
//
// dQ kernel: like the forward, a workgroup owns 128 query rows of one query
// head (lane = query): S^T = K Q^T and dP^T = V dO^T (K, V from LDS, Q^T and
// dO^T in registers), then dQ^T += K^T dS^T with K^T from a transposed LDS
// copy of the same tile.
//
// dK/dV kernel: a workgroup owns 128 keys of one KV head (lane = key) and
// loops over every query head of the group and every query tile that can see
// those keys: S = Q K^T and dP = dO V^T (Q, dO from LDS, K^T, V^T in
// registers), then dV^T += dO^T P and dK^T += Q^T dS with transposed LDS
// copies of the Q and dO tiles.  Each output row has exactly one owner, so
// there are no atomics and the result is deterministic.
//
// dS enters the two dS products as bfloat16; with precise_ds it is split
// into hi + lo bfloat16 parts (two MFMAs) so that its rounding error does not
// reach dQ and dK.
#include "attn_bwd_common.h"

namespace attn {

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
template <typename T, int D> struct DkvCfg {
  static constexpr int BQ = 32;   // query rows per streamed tile
};

template <typename T, int D, int CAP, bool PRECISE>
__global__ __launch_bounds__(NTHREADS, 1) void dkv_kernel(KArgs a) {
  constexpr int BQ = DkvCfg<T, D>::BQ;
  constexpr bool ACC = sizeof(T) == 4;
  using E = Elem<T>;
  using frag = typename E::frag;
  using QIO = TileIO<T, BQ, D, NTHREADS>;
  using CapF = Cap<CAP, ACC>;
  constexpr int NQB = BQ / 32;
  constexpr int NDB = D / 32;
  constexpr int NT16 = D / 16;

  __shared__ __attribute__((aligned(16))) T sQ[2][QIO::ROW_ELEMS];
  __shared__ __attribute__((aligned(16))) T sdO[2][QIO::ROW_ELEMS];
  __shared__ __attribute__((aligned(16))) T sQt[2][QIO::T_ELEMS];
  __shared__ __attribute__((aligned(16))) T sdOt[2][QIO::T_ELEMS];
  __shared__ __attribute__((aligned(16))) float sKf[2][BQ];
  __shared__ __attribute__((aligned(16))) float sC2[2][BQ];
  __shared__ __attribute__((aligned(16))) float sR[2][BQ];
  __shared__ __attribute__((aligned(16))) float sDl[2][BQ];
  __shared__ int sSeg[2][BQ];
  __shared__ unsigned char sFlag[MAX_TILES];
  __shared__ int sRange[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= a.n_items) return;

  const int L = a.L, G = a.G;
  const int kt = item % a.n_kv_tiles;
  const int rest = item / a.n_kv_tiles;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int k0 = kt * BKV, k1 = imin(k0 + BKV, L);
  const int kw0 = k0 + wave * 32;
  const int krow = kw0 + l32;
  const bool key_ok = krow < L;

  const long q_rs = (long)a.Hq * D, kv_rs = (long)a.Hkv * D;
  const T* Kb = (const T*)a.k + ((long)b * L * a.Hkv + hkv) * D;
  const T* Vb = (const T*)a.v + ((long)b * L * a.Hkv + hkv) * D;

  MaskSpec ms;
  ms.L = L;
  ms.causal = a.causal;
  ms.window = a.window;
  ms.ranker = a.bounds != nullptr;
  ms.hl = ms.hu = ms.cl = ms.cu = 0;
  if (ms.ranker) {
    ms.hl = a.bounds[4 * b + 0];
    ms.hu = a.bounds[4 * b + 1];
    ms.cl = a.bounds[4 * b + 2];
    ms.cu = a.bounds[4 * b + 3];
  }
  const bool has_seg = a.seg != nullptr;
  ms.has_seg = has_seg;
  const int* segb = has_seg ? a.seg + (long)b * L : nullptr;

  // K^T and V^T fragments (B operands), one per 16-wide step over D.
  frag kf[NT16], vf[NT16];
#pragma unroll
  for (int t = 0; t < NT16; ++t) {
    kf[t] = global_frag<T>(Kb + (long)krow * kv_rs + 16 * t + 8 * hh, key_ok);
    vf[t] = global_frag<T>(Vb + (long)krow * kv_rs + 16 * t + 8 * hh, key_ok);
  }
  const int seg_k = (has_seg && key_ok) ? segb[krow] : 0;

  // Query tiles that can see keys [k0, k1) (causal / window), then per-tile
  // ranker and segment skips.
  int t_lo = 0, t_hi = 0;
  const bool any = query_tile_range(k0, k1, BQ, ms, &t_lo, &t_hi);
  if (has_seg && any) {
    if (tid == 0) { sRange[0] = 0x7fffffff; sRange[1] = (int)0x80000000; }
    __syncthreads();
    if (tid < k1 - k0) {
      const int s = segb[k0 + tid];
      atomicMin(&sRange[0], s);
      atomicMax(&sRange[1], s);
    }
    for (int t = t_lo + tid; t < t_hi; t += NTHREADS) sFlag[t - t_lo] = 0;
    __syncthreads();
    const int smin = sRange[0], smax = sRange[1];
    const int q_end = imin(t_hi * BQ, L);
    for (int qq = t_lo * BQ + tid; qq < q_end; qq += NTHREADS) {
      const int s = segb[qq];
      if (s >= smin && s <= smax) sFlag[qq / BQ - t_lo] = 1;
    }
    __syncthreads();
  }
  auto needed = [&](int t) -> bool {
    if (tile_class(t * BQ, t * BQ + BQ, k0, k1, ms) == TILE_EMPTY) return false;
    if (has_seg && !sFlag[t - t_lo]) return false;
    return true;
  };
  auto next_needed = [&](int t) -> int {
    for (; t < t_hi; ++t)
      if (needed(t)) return t;
    return -1;
  };
  // The step sequence is (query head g, query tile t) for g over the group.
  auto next_step = [&](int g, int t, int& gn, int& tn) -> bool {
    int x = next_needed(t + 1);
    if (x >= 0) { gn = g; tn = x; return true; }
    if (g + 1 < G) {
      x = next_needed(t_lo);
      if (x >= 0) { gn = g + 1; tn = x; return true; }
    }
    return false;
  };

  QIO qio, dio;
  auto load_step = [&](int g, int t) {
    const int hq = hkv * G + g;
    const int qb0 = t * BQ;
    qio.load((const T*)a.q + (((long)b * L + qb0) * a.Hq + hq) * D, q_rs, L - qb0, tid);
    dio.load((const T*)a.dout + (((long)b * L + qb0) * a.Hq + hq) * D, q_rs, L - qb0, tid);
  };
  auto store_step = [&](int g, int t, int bf) {
    qio.store_rows(sQ[bf], tid);
    qio.store_T(sQt[bf], tid);
    dio.store_rows(sdO[bf], tid);
    dio.store_T(sdOt[bf], tid);
    if (tid < BQ) {
      const int hq = hkv * G + g;
      const int qq = t * BQ + tid;
      float lse2 = ATTN_POS_INF, dlt = 0.f, tmp = 1.f;
      int sg = -1;
      if (qq < L) {
        row_residuals(a, ((long)b * a.Hq + hq) * L + qq, lse2, dlt);
        if (a.temp != nullptr) tmp = a.temp[(long)b * L + qq];
        if (has_seg) sg = segb[qq];
      }
      const RowC rc = row_consts(a, tmp, lse2);
      sKf[bf][tid] = rc.Kf;
      sC2[bf][tid] = rc.C2;
      sR[bf][tid] = rc.R;
      sDl[bf][tid] = dlt;
      sSeg[bf][tid] = sg;
    }
  };

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dkacc[i] = dvacc[i] = f32x16{};

  int gc = 0, tc = any ? next_needed(t_lo) : -1;
  bool have = tc >= 0;
  if (have) {
    load_step(gc, tc);
    store_step(gc, tc, 0);
  }
  __syncthreads();
  int buf = 0;
  while (have) {
    int gn = 0, tn = 0;
    const bool more = next_step(gc, tc, gn, tn);
    if (more) load_step(gn, tn);

    const int qb0 = tc * BQ;
    const bool full = tile_class(qb0, qb0 + BQ, kw0, kw0 + 32, ms) == TILE_FULL;

    // S = Q K^T, dP = dO V^T  (rows = queries in pi order, lane = key)
    f32x16 sacc[NQB], pacc[NQB];
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) sacc[qb] = pacc[qb] = f32x16{};
#pragma unroll
    for (int t = 0; t < NT16; ++t) {
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        sacc[qb] = E::mfma(QIO::row_frag(sQ[buf], qb, t, lane), kf[t], sacc[qb]);
        pacc[qb] = E::mfma(QIO::row_frag(sdO[buf], qb, t, lane), vf[t], pacc[qb]);
      }
    }
    // P into sacc, dS into pacc
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int qoff = qb * 32 + prow(r, hh);
        const float Kf = sKf[buf][qoff], C2 = sC2[buf][qoff];
        const float R = sR[buf][qoff], dl = sDl[buf][qoff];
        float aux;
        const float x = sacc[qb][r];
        float p = fast_exp2(__builtin_fmaf(CapF::f(x, a, aux), Kf, C2));
        if (!full) {
          bool vis = pair_visible(qb0 + qoff, krow, ms);
          if (has_seg) vis = vis && (sSeg[buf][qoff] == seg_k);
          p = vis ? p : 0.f;
        }
        pacc[qb][r] = p * (pacc[qb][r] - dl) * R * CapF::g(aux, a);
        sacc[qb][r] = p;
      }
    }
    // dV^T += dO^T P ; dK^T += Q^T dS
#pragma unroll
    for (int t = 0; t < BQ / 16; ++t) {
      const frag pb = E::from_acc(sacc[t / 2], 8 * (t % 2));
      frag hi, lo;
      if (PRECISE) {
        E::split_acc(pacc[t / 2], 8 * (t % 2), hi, lo);
      } else {
        hi = E::from_acc(pacc[t / 2], 8 * (t % 2));
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        dvacc[db] = E::mfma(QIO::t_frag(sdOt[buf], db, t, lane), pb, dvacc[db]);
        const frag qa = QIO::t_frag(sQt[buf], db, t, lane);
        dkacc[db] = E::mfma(qa, hi, dkacc[db]);
        if (PRECISE) dkacc[db] = E::mfma(qa, lo, dkacc[db]);
      }
    }

    if (more) store_step(gn, tn, buf ^ 1);
    __syncthreads();
    buf ^= 1;
    gc = gn;
    tc = tn;
    have = more;
  }

  if (key_ok) {
    float* dkrow = a.out0 + ((long)(b * L + krow) * a.Hkv + hkv) * D;
    float* dvrow = a.out1 + ((long)(b * L + krow) * a.Hkv + hkv) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 vk, vv;
#pragma unroll
        for (int c = 0; c < 4; ++c) {
          vk[c] = dkacc[db][4 * r4 + c];
          vv[c] = dvacc[db][4 * r4 + c];
        }
        *(f32x4*)(dkrow + 32 * db + 8 * r4 + 4 * hh) = vk;
        *(f32x4*)(dvrow + 32 * db + 8 * r4 + 4 * hh) = vv;
      }
    }
  }
}

template <typename T, int D, bool P>
static void dkv_cap(const KArgs& a, int cap, hipStream_t s) {
  dim3 grid(a.n_items), block(NTHREADS);
  switch (cap) {
    case 0: hipLaunchKernelGGL((dkv_kernel<T, D, 0, P>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((dkv_kernel<T, D, 1, P>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((dkv_kernel<T, D, 2, P>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((dkv_kernel<T, D, 3, P>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_dkv(const KArgs& a, int dtype, int head_dim, int cap, hipStream_t s) {
  if (dtype == 1) return launch_dkv_bf16(a, head_dim, cap, s);
  if (head_dim == 64) dkv_cap<float, 64, false>(a, cap, s);
  else dkv_cap<float, 128, false>(a, cap, s);
  return hipGetLastError();
}

}  // namespace attn
