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
// dQ
// ---------------------------------------------------------------------------
template <typename T, int D> struct DqCfg {
  static constexpr int BN = 32;   // keys per streamed tile
};

// DT: also accumulate this head's share of the temperature gradient,
// dtemp_i = sum_j dS'_ij c_ij with c the capped logit, c = ln2 (kmul f + kadd).
template <typename T, int D, int CAP, bool PRECISE, bool DT>
__global__ __launch_bounds__(NTHREADS, 2) void dq_kernel(KArgs a) {
  constexpr int BN = DqCfg<T, D>::BN;
  constexpr bool ACC = sizeof(T) == 4;
  using E = Elem<T>;
  using frag = typename E::frag;
  using KIO = TileIO<T, BN, D, NTHREADS>;
  using CapF = Cap<CAP, ACC>;
  constexpr int NKB = BN / 32;
  constexpr int NDB = D / 32;
  constexpr int NT16 = D / 16;

  __shared__ __attribute__((aligned(16))) T sK[2][KIO::ROW_ELEMS];
  __shared__ __attribute__((aligned(16))) T sV[2][KIO::ROW_ELEMS];
  __shared__ __attribute__((aligned(16))) T sKt[2][KIO::T_ELEMS];
  __shared__ int sSeg[2][BN];
  __shared__ unsigned char sFlag[MAX_TILES];
  __shared__ int sRange[2];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hh = lane >> 5, l32 = lane & 31;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= a.n_items) return;

  const int L = a.L, G = a.G;
  const int g = item % G;
  int rest = item / G;
  const int qt_rev = rest % a.n_q_tiles;
  rest /= a.n_q_tiles;
  const int hkv = rest % a.Hkv;
  const int b = rest / a.Hkv;
  const int qt = a.causal ? (a.n_q_tiles - 1 - qt_rev) : qt_rev;
  const int hq = hkv * G + g;
  const int q0 = qt * BM, q1 = imin(q0 + BM, L);
  const int qw0 = q0 + wave * 32;
  const int qrow = qw0 + l32;
  const bool row_ok = qrow < L;

  const long q_rs = (long)a.Hq * D, kv_rs = (long)a.Hkv * D;
  const T* Qb = (const T*)a.q + ((long)b * L * a.Hq + hq) * D;
  const T* dOb = (const T*)a.dout + ((long)b * L * a.Hq + hq) * D;
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

  frag qf[NT16], df[NT16];
#pragma unroll
  for (int t = 0; t < NT16; ++t) {
    qf[t] = global_frag<T>(Qb + (long)qrow * q_rs + 16 * t + 8 * hh, row_ok);
    df[t] = global_frag<T>(dOb + (long)qrow * q_rs + 16 * t + 8 * hh, row_ok);
  }
  float lse2 = ATTN_POS_INF, dlt = 0.f, tmp = 1.f;
  if (row_ok) {
    row_residuals(a, ((long)b * a.Hq + hq) * L + qrow, lse2, dlt);
    if (a.temp != nullptr) tmp = a.temp[(long)b * L + qrow];
  }
  const RowC rc = row_consts(a, tmp, lse2);
  const int seg_q = (has_seg && row_ok) ? segb[qrow] : 0;

  int t_lo = 0, t_hi = 0;
  bool any = key_tile_range(q0, q1, BN, ms, &t_lo, &t_hi);
  if (has_seg && any) {
    if (tid == 0) { sRange[0] = 0x7fffffff; sRange[1] = (int)0x80000000; }
    __syncthreads();
    if (tid < q1 - q0) {
      const int s = segb[q0 + tid];
      atomicMin(&sRange[0], s);
      atomicMax(&sRange[1], s);
    }
    for (int t = t_lo + tid; t < t_hi; t += NTHREADS) sFlag[t - t_lo] = 0;
    __syncthreads();
    const int smin = sRange[0], smax = sRange[1];
    const int k_end = imin(t_hi * BN, L);
    for (int kk = t_lo * BN + tid; kk < k_end; kk += NTHREADS) {
      const int s = segb[kk];
      if (s >= smin && s <= smax) sFlag[kk / BN - t_lo] = 1;
    }
    __syncthreads();
  }
  auto needed = [&](int t) -> bool {
    if (tile_class(q0, q1, t * BN, t * BN + BN, ms) == TILE_EMPTY) return false;
    if (has_seg && !sFlag[t - t_lo]) return false;
    return true;
  };
  auto next_needed = [&](int t) -> int {
    for (; t < t_hi; ++t)
      if (needed(t)) return t;
    return -1;
  };

  KIO kio, vio;
  float tacc = 0.f;
  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};

  int j = any ? next_needed(t_lo) : -1;
  if (j >= 0) {
    kio.load(Kb + (long)(j * BN) * kv_rs, kv_rs, L - j * BN, tid);
    vio.load(Vb + (long)(j * BN) * kv_rs, kv_rs, L - j * BN, tid);
    kio.store_rows(sK[0], tid);
    kio.store_T(sKt[0], tid);
    vio.store_rows(sV[0], tid);
    if (has_seg && tid < BN) sSeg[0][tid] = (j * BN + tid < L) ? segb[j * BN + tid] : -1;
  }
  __syncthreads();
  int buf = 0;
  while (j >= 0) {
    const int jn = next_needed(j + 1);
    if (jn >= 0) {
      kio.load(Kb + (long)(jn * BN) * kv_rs, kv_rs, L - jn * BN, tid);
      vio.load(Vb + (long)(jn * BN) * kv_rs, kv_rs, L - jn * BN, tid);
    }
    const int k0 = j * BN;
    const bool full = tile_class(qw0, qw0 + 32, k0, k0 + BN, ms) == TILE_FULL;

    f32x16 sacc[NKB], pacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = pacc[kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < NT16; ++t) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[kb] = E::mfma(KIO::row_frag(sK[buf], kb, t, lane), qf[t], sacc[kb]);
        pacc[kb] = E::mfma(KIO::row_frag(sV[buf], kb, t, lane), df[t], pacc[kb]);
      }
    }
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float aux;
        const float x = sacc[kb][r];
        const float fx = CapF::f(x, a, aux);
        float p = fast_exp2(__builtin_fmaf(fx, rc.Kf, rc.C2));
        if (!full) {
          const int koff = kb * 32 + prow(r, hh);
          bool vis = pair_visible(qrow, k0 + koff, ms);
          if (has_seg) vis = vis && (sSeg[buf][koff] == seg_q);
          p = vis ? p : 0.f;
        }
        const float dsp = p * (pacc[kb][r] - dlt);
        if (DT) tacc = __builtin_fmaf(dsp, __builtin_fmaf(fx, a.kmul, a.kadd), tacc);
        sacc[kb][r] = dsp * rc.R * CapF::g(aux, a);
      }
    }
    // dQ^T += K^T dS^T
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      frag hi, lo;
      if (PRECISE) {
        E::split_acc(sacc[t / 2], 8 * (t % 2), hi, lo);
      } else {
        hi = E::from_acc(sacc[t / 2], 8 * (t % 2));
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const frag ka = KIO::t_frag(sKt[buf], db, t, lane);
        dqacc[db] = E::mfma(ka, hi, dqacc[db]);
        if (PRECISE) dqacc[db] = E::mfma(ka, lo, dqacc[db]);
      }
    }

    if (jn >= 0) {
      kio.store_rows(sK[buf ^ 1], tid);
      kio.store_T(sKt[buf ^ 1], tid);
      vio.store_rows(sV[buf ^ 1], tid);
      if (has_seg && tid < BN) sSeg[buf ^ 1][tid] = (jn * BN + tid < L) ? segb[jn * BN + tid] : -1;
    }
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  if (DT) {
    // lanes l and l + 32 hold the same query's two key halves
    const float tot = tacc + __shfl_xor(tacc, 32);
    if (row_ok && hh == 0) a.out3[((long)b * a.Hq + hq) * L + qrow] = tot * LN2_F;
  }
  if (row_ok) {
    float* drow = a.out0 + ((long)(b * L + qrow) * a.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = dqacc[db][4 * r4 + c];
        *(f32x4*)(drow + 32 * db + 8 * r4 + 4 * hh) = v;
      }
    }
  }
}

template <typename T, int D, bool P, bool DT>
static void dq_cap(const KArgs& a, int cap, hipStream_t s) {
  dim3 grid(a.n_items), block(NTHREADS);
  switch (cap) {
    case 0: hipLaunchKernelGGL((dq_kernel<T, D, 0, P, DT>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((dq_kernel<T, D, 1, P, DT>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((dq_kernel<T, D, 2, P, DT>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((dq_kernel<T, D, 3, P, DT>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_dq(const KArgs& a, int dtype, int head_dim, int cap, hipStream_t s) {
  if (dtype == 1) return launch_dq_bf16(a, head_dim, cap, s);
  const bool dt = a.out3 != nullptr;
  if (head_dim == 64) dt ? dq_cap<float, 64, false, true>(a, cap, s) : dq_cap<float, 64, false, false>(a, cap, s);
  else dt ? dq_cap<float, 128, false, true>(a, cap, s) : dq_cap<float, 128, false, false>(a, cap, s);
  return hipGetLastError();
}

}  // namespace attn
