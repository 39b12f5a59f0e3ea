// Forward kernel: O, m, l of capped, masked, grouped-query softmax attention.
// This generic version serves float inputs; bfloat16 inputs use the gfx950
// data path of attn_bf16.hip (same mathematics).
//
// Method (triton_kernels.py page, make_triton_forward_kernel; caps from the
// mosaic_backward.py page, _apply_cap_mosaic): per query row, stream the key
// tiles that can hold a visible key, and keep the online-softmax state
// (running max m, running sum l, rescaled accumulator) in registers.
//
// gfx950 mapping: one workgroup = 4 waves = 128 query rows of one
// (batch, query head); a wave owns 32 query rows, one per lane column.
//   S^T (keys x queries) = K_tile Q^T   -- K from LDS (A), Q^T in registers (B)
//   O^T (d x queries)   += V^T_tile P^T -- V^T from LDS (A), P^T from the C
//                                          registers of S^T (B)
// so the row max and row sum of a query stay inside one lane plus one swap
// between the two wave halves.  K/V tiles are double-buffered in LDS and the
// next tile's global loads are issued before the current tile's MFMAs.
#include "attn_device.h"

namespace attn {

template <typename T, int D> struct FwdCfg {
  static constexpr int BN = (sizeof(T) == 2 || D == 64) ? 64 : 32;   // keys per tile
};

template <typename T, int D, int CAP>
__global__ __launch_bounds__(NTHREADS, 2) void fwd_kernel(KArgs a) {
  constexpr int BN = FwdCfg<T, D>::BN;
  constexpr bool ACC = sizeof(T) == 4;
  using E = Elem<T>;
  using frag = typename E::frag;
  using KIO = TileIO<T, BN, D, NTHREADS>;
  using CapF = Cap<CAP, ACC>;
  constexpr int NKB = BN / 32;     // 32-key blocks per tile
  constexpr int NDB = D / 32;      // 32-wide d blocks
  constexpr int NT16 = D / 16;     // reduction steps over D

  __shared__ __attribute__((aligned(16))) T sK[2][KIO::ROW_ELEMS];
  __shared__ __attribute__((aligned(16))) T sVt[2][KIO::T_ELEMS];
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

  // Query fragments (B operand of S^T), one per 16-wide step over D.
  frag qf[NT16];
#pragma unroll
  for (int t = 0; t < NT16; ++t) qf[t] = global_frag<T>(Qb + (long)qrow * q_rs + 16 * t + 8 * hh, row_ok);

  const float tmp = (a.temp != nullptr && row_ok) ? a.temp[(long)b * L + qrow] : 1.f;
  const RowC rc = row_consts(a, tmp, 0.f);
  const int seg_q = (has_seg && row_ok) ? segb[qrow] : 0;

  // Candidate key tiles: causal / window range, then ranker and segment skips.
  int t_lo = 0, t_hi = 0;
  bool any = key_tile_range(q0, q1, BN, ms, &t_lo, &t_hi);
  if (has_seg && any) {
    // Segment skip: a key tile is needed only if one of its keys carries an id
    // inside [min, max] of this workgroup's row ids (sound for any ids).
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
  float m_run = ATTN_NEG_INF, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};

  int j = any ? next_needed(t_lo) : -1;
  if (j >= 0) {
    kio.load(Kb + (long)(j * BN) * kv_rs, kv_rs, L - j * BN, tid);
    vio.load(Vb + (long)(j * BN) * kv_rs, kv_rs, L - j * BN, tid);
    kio.store_rows(sK[0], tid);
    vio.store_T(sVt[0], tid);
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
    const T* cK = sK[buf];
    const T* cVt = sVt[buf];
    const bool full = tile_class(qw0, qw0 + 32, k0, k0 + BN, ms) == TILE_FULL;

    // S^T = K Q^T
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
#pragma unroll
    for (int t = 0; t < NT16; ++t) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = E::mfma(KIO::row_frag(cK, kb, t, lane), qf[t], sacc[kb]);
    }

    // capped, tempered log2-domain logits; mask on partial tiles
    float mx = ATTN_NEG_INF;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float aux;
        float w = __builtin_fmaf(CapF::f(sacc[kb][r], a, aux), rc.Kf, rc.C2);
        if (!full) {
          const int koff = kb * 32 + prow(r, hh);
          bool vis = pair_visible(qrow, k0 + koff, ms);
          if (has_seg) vis = vis && (sSeg[buf][koff] == seg_q);
          w = vis ? w : ATTN_NEG_INF;
        }
        sacc[kb][r] = w;
        mx = fmaxf(mx, w);
      }
    }
    mx = fmaxf(mx, wave_half_swap(mx));
    const float m_new = fmaxf(m_run, mx);
    const float base = (m_new == ATTN_NEG_INF) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - base);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i) oacc[i] *= alpha;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(sacc[kb][r] - base);
        l_run += p;
        sacc[kb][r] = p;
      }
    }
    m_run = m_new;

    // O^T += V^T P^T
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      const frag pb = E::from_acc(sacc[t / 2], 8 * (t % 2));
#pragma unroll
      for (int db = 0; db < NDB; ++db) oacc[db] = E::mfma(KIO::t_frag(cVt, db, t, lane), pb, oacc[db]);
    }

    if (jn >= 0) {
      kio.store_rows(sK[buf ^ 1], tid);
      vio.store_T(sVt[buf ^ 1], tid);
      if (has_seg && tid < BN) sSeg[buf ^ 1][tid] = (jn * BN + tid < L) ? segb[jn * BN + tid] : -1;
    }
    __syncthreads();
    buf ^= 1;
    j = jn;
  }

  // finalize: O = acc / l; m in natural-log units
  const float l_tot = l_run + wave_half_swap(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    float* orow = a.out0 + ((long)(b * L + qrow) * a.Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4) {
        f32x4 v;
#pragma unroll
        for (int c = 0; c < 4; ++c) v[c] = oacc[db][4 * r4 + c] * inv;
        *(f32x4*)(orow + 32 * db + 8 * r4 + 4 * hh) = v;
      }
    }
    if (hh == 0) {
      const long mi = ((long)b * a.Hq + hq) * L + qrow;
      a.out1[mi] = (m_run == ATTN_NEG_INF) ? ATTN_NEG_INF : m_run * LN2_F;
      a.out2[mi] = l_tot;
    }
  }
}

template <typename T, int D>
static hipError_t launch_fwd_t(const KArgs& a, int cap, hipStream_t s) {
  dim3 grid(a.n_items), block(NTHREADS);
  switch (cap) {
    case 0: hipLaunchKernelGGL((fwd_kernel<T, D, 0>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((fwd_kernel<T, D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((fwd_kernel<T, D, 2>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((fwd_kernel<T, D, 3>), grid, block, 0, s, a); break;
  }
  return hipGetLastError();
}

hipError_t launch_fwd(const KArgs& a, int dtype, int head_dim, int cap, hipStream_t s) {
  if (dtype == 1) return launch_fwd_bf16(a, head_dim, cap, s);
  return head_dim == 64 ? launch_fwd_t<float, 64>(a, cap, s) : launch_fwd_t<float, 128>(a, cap, s);
}

int fwd_key_tile(int dtype, int head_dim) {
  if (dtype == 1) return 64;   // attn_bf16.hip
  return head_dim == 64 ? FwdCfg<float, 64>::BN : FwdCfg<float, 128>::BN;
}

}  // namespace attn
