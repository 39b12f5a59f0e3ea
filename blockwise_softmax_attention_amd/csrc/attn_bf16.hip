// bfloat16 kernels for gfx950: forward, dQ and dK/dV.
//
// Same mathematics and orientation as the float kernels (see attn_fwd.hip and
// attn_dq.hip / attn_dkv.hip for the method and its sources), with a
// gfx950-specific data path:
//   * K/V (forward, dQ) and Q/dO (dK/dV) tiles are loaded straight from HBM
//     into LDS (global_load_lds_dwordx4), double-buffered, with no staging
//     registers;
//   * each tile is stored once, row-major and swizzled; products that reduce
//     over the tile rows (P V, dS K, P^T dO, dS^T Q) read it transposed with
//     ds_read_b64_tr_b16;
//   * the score elementwise work has a branch-free FULL path for tiles whose
//     pairs are all visible and a MASKED path for boundary tiles;
//   * the forward rescales its accumulator only when a row maximum grows by
//     more than 2^8 (the exact m is tracked separately), so most tiles skip
//     the rescale;
//   * the forward and dQ loops are instantiated once per LDS stage (fragment
//     addresses become a per-lane register plus an immediate) and raise their
//     wave priority over MFMA bursts (two waves per SIMD).
#include <type_traits>

#include "attn.h"
#include "attn_bf16.h"
#include "attn_bwd_common.h"

// Per-kernel build choices: tile sizes, occupancy of the forward, address
// laundering (see BTile) and the MFMA-burst priority (mfma_phase).
#ifndef ATTN_LAUNDER_FWD
#define ATTN_LAUNDER_FWD 0
#endif
#ifndef ATTN_LAUNDER_DQ
#define ATTN_LAUNDER_DQ 0
#endif
#ifndef ATTN_LAUNDER_DKV
#define ATTN_LAUNDER_DKV 0
#endif
#ifndef ATTN_FWD_BN
#define ATTN_FWD_BN 64
#endif
#ifndef ATTN_FWD_WAVES_PER_SIMD
#define ATTN_FWD_WAVES_PER_SIMD 2
#endif
#ifndef ATTN_DKV_BQ
#define ATTN_DKV_BQ 128
#endif
#ifndef ATTN_DQ_BN
#define ATTN_DQ_BN 32
#endif
#ifndef ATTN_PRIO
#define ATTN_PRIO 1
#endif


namespace attn {

constexpr int BN16 = ATTN_FWD_BN;
constexpr int DKV_PLAN_MAX = 2048;   // dK/dV step-plan entries (query tiles per key block)
static_assert(DKV_PLAN_MAX * ATTN_DKV_BQ >= ATTN_MAX_SEQ_LEN, "a plan entry for every query tile");   // keys per tile (forward)
constexpr int BNQ16 = ATTN_DQ_BN;   // keys per tile (dQ: Q and dO fragments stay in registers)
constexpr int BQ16 = ATTN_DKV_BQ;   // queries per tile (dK/dV)
constexpr float RESCALE_TAU = 8.f;

// Wave priority around a burst of MFMAs: with two waves per SIMD, the one
// entering its matrix phase is issued first, so that its MFMAs run while the
// other wave does vector work.
__device__ __forceinline__ void mfma_phase(bool begin) {
  if (ATTN_PRIO) {
    __builtin_amdgcn_sched_barrier(0);
    if (begin) {
      __builtin_amdgcn_s_setprio(1);
    } else {
      __builtin_amdgcn_s_setprio(0);
    }
    __builtin_amdgcn_sched_barrier(0);
  }
}

// Segment tables: for the workgroup's own rows [r0, r1), flag the tiles of
// [t_lo, t_hi) (size bt over the other side) that can share a segment with
// them, and the tiles that hold an id other than the workgroup's minimum
// (mixed).  When the workgroup's rows all share one id and a tile is not
// mixed, every pair of the tile is in one segment and the segment test can be
// dropped for it.  The flag test is either "the tile holds an id inside the
// workgroup's [min, max]" (flags only) or, with a second table, the symmetric
// "the tile's [min, max] and the workgroup's overlap" (flags && flags2: some
// id <= max and some id >= min), which the query-tile and key-tile sides of
// the stored-dS backward evaluate identically; both are sound for any ids.
__device__ __forceinline__ void segment_flags(const int* segb, int r0, int r1, int t_lo, int t_hi,
                                              int bt, int L, int tid, unsigned char* flags,
                                              unsigned char* mixed, int* range,
                                              unsigned char* flags2 = nullptr) {
  if (tid == 0) {
    range[0] = 0x7fffffff;
    range[1] = (int)0x80000000;
  }
  __syncthreads();
  if (tid < r1 - r0) {
    const int s = segb[r0 + tid];
    atomicMin(&range[0], s);
    atomicMax(&range[1], s);
  }
  for (int t = t_lo + tid; t < t_hi; t += NTHREADS) {
    flags[t - t_lo] = mixed[t - t_lo] = 0;
    if (flags2 != nullptr) flags2[t - t_lo] = 0;
  }
  __syncthreads();
  const int smin = range[0], smax = range[1];
  const int end = imin(t_hi * bt, L);
  for (int x = t_lo * bt + tid; x < end; x += NTHREADS) {
    const int s = segb[x];
    if (flags2 != nullptr) {
      if (s <= smax) flags[x / bt - t_lo] = 1;
      if (s >= smin) flags2[x / bt - t_lo] = 1;
    } else if (s >= smin && s <= smax) {
      flags[x / bt - t_lo] = 1;
    }
    if (s != smin) mixed[x / bt - t_lo] = 1;
  }
  __syncthreads();
}

// Tile class of a block of tile t of a segment table, the segment test
// dropped where the table shows a single segment (see segment_flags).
__device__ __forceinline__ int seg_tile_class(int q0, int q1, int k0, int k1, MaskSpec ms, int t,
                                              int t_lo, const unsigned char* mixed, const int* range) {
  if (ms.has_seg && range[0] == range[1] && !mixed[t - t_lo]) ms.has_seg = false;
  return __builtin_amdgcn_readfirstlane(tile_class(q0, q1, k0, k1, ms));
}

struct RowItem {
  int b, hkv, hq, q0, q1, qw0, qrow;
};

// Ranker workloads: the batch rows ordered by history length, longest first
// (ties by index), into ord[0 .. B); returns false (and leaves ord alone)
// where the row order of decode_row_item stays the plain one.  A query tile
// of a ranker row sees about (hu - hl) / BN key tiles, so that length ranks
// the rows' items by work.  Wave-uniform; holds a workgroup barrier.
__device__ __forceinline__ bool ranker_row_order(const KArgs& a, int tid, int* ord) {
  const bool on = a.bounds != nullptr && a.B > 1 && a.B <= 64 && a.n_items % (8 * a.B) == 0;
  if (!on) return false;
  if (tid < a.B) {
    const int w = a.bounds[4 * tid + 1] - a.bounds[4 * tid];
    int rank = 0;
    for (int j = 0; j < a.B; ++j) {
      const int wj = a.bounds[4 * j + 1] - a.bounds[4 * j];
      rank += (wj > w || (wj == w && j < tid)) ? 1 : 0;
    }
    ord[rank] = tid;
  }
  __syncthreads();
  return true;
}

// Work item -> (batch row, head, query tile).  Each XCD receives a contiguous
// run of items (xcd_remap) covering every batch row.  By default the batch
// row varies fastest, so rows whose masks leave them different amounts of
// work (ranker bounds, segment lengths) are spread over the XCDs instead of
// loading some of them.  With a row order (ranker_row_order) the rows are
// instead the slowest index inside each run, heaviest first: the dispatcher
// hands out workgroups in order, in lockstep rounds over the XCDs, and rounds
// of equal items leave no slot waiting on a longer row (ranker workload:
// forward -3.7%, dQ -2% to -5%).  Each run covers the same heads and query
// tiles either way.
__device__ __forceinline__ RowItem decode_row_item(const KArgs& a, int item, int wave, int l32,
                                                   const int* ord) {
  RowItem it;
  int rest;
  if (ord != nullptr) {
    const int R = a.n_items / 8, per_b = R / a.B, run = item / R, loc = item - run * R;
    it.b = ord[loc / per_b];
    rest = run * per_b + loc % per_b;
  } else {
    it.b = item % a.B;
    rest = item / a.B;
  }
  const int g = rest % a.G;
  rest /= a.G;
  const int qt_rev = rest % a.n_q_tiles;
  it.hkv = rest / a.n_q_tiles;
  const int qt = a.causal ? (a.n_q_tiles - 1 - qt_rev) : qt_rev;
  it.hq = it.hkv * a.G + g;
  it.q0 = qt * BM;
  it.q1 = imin(it.q0 + BM, a.L);
  it.qw0 = it.q0 + wave * 32;
  it.qrow = it.qw0 + l32;
  return it;
}

// ---------------------------------------------------------------------------
// Forward
// ---------------------------------------------------------------------------
// Logits of one tile in the log2 domain (lane = query): s becomes
// fma(f(x), Kf, C2) (masked pairs -inf); returns this lane's maximum.
template <bool MASKED, bool SEG, int CAP, int NKB>
__device__ __forceinline__ float fwd_logits(f32x16 (&s)[NKB], const KArgs& a, const RowC& rc,
                                            const QMask& qm, int k0, int hh, const int* sseg,
                                            int seg_q) {
  using CapF = Cap<CAP, false>;
  float mx = ATTN_NEG_INF;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float aux;
      float w = __builtin_fmaf(CapF::f(s[kb][r], a, aux), rc.Kf, rc.C2);
      if (MASKED) {
        const int koff = kb * 32 + prow(r, hh);
        bool vis = qmask_vis(qm, k0 + koff);
        if (SEG) vis = vis && sseg[koff] == seg_q;
        w = vis ? w : ATTN_NEG_INF;
      }
      s[kb][r] = w;
      mx = fmaxf(mx, w);
    }
  }
  return mx;
}

// Sign of the logit's slope in the cap output f for the fast forms of
// Cap<> (logit = f kmul t + kadd t): kmul < 0 only for the tanh form.
template <int CAP> struct CapSlope {
  static constexpr float value = (CAP == 1) ? -1.f : 1.f;
};

// Full tiles whose rows all have a slope Kf of the sign CapSlope (temperature
// >= 0): s keeps the cap output f and the row maximum of the logits comes from
// the extreme f (the logit fma(f, Kf, C2) is monotone in f, and so is its
// rounding); the exponent later folds C2 - base into one fma.
template <int CAP, int NKB>
__device__ __forceinline__ float fwd_caps(f32x16 (&s)[NKB], const KArgs& a, const RowC& rc) {
  using CapF = Cap<CAP, false>;
  constexpr bool POS = CapSlope<CAP>::value > 0.f;
  float ext = POS ? ATTN_NEG_INF : ATTN_POS_INF;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float aux;
      const float f = CapF::f(s[kb][r], a, aux);
      s[kb][r] = f;
      ext = POS ? fmaxf(ext, f) : fminf(ext, f);
    }
  }
  return __builtin_fmaf(ext, rc.Kf, rc.C2);
}

// Online-softmax update of one tile (every tile class shares it): the
// running base m_base moves only when the tile's maximum exceeds it by more
// than RESCALE_TAU (then O and l are rescaled); m_true tracks the exact
// maximum.  Returns the base the exponents are taken against.
template <int NDB>
__device__ __forceinline__ float fwd_rescale(f32x16 (&o)[NDB], float mx, float& m_base, float& m_true,
                                             float& l_run) {
  mx = half_max(mx);
  m_true = fmaxf(m_true, mx);
  if (__ballot(mx > m_base + RESCALE_TAU) != 0) {
    const float m_new = fmaxf(m_base, mx);
    // 0 when the row saw its first key, 1 while it still has none
    const float alpha = (m_new == ATTN_NEG_INF) ? 1.f : fast_exp2(m_base - m_new);
    l_run *= alpha;
#pragma unroll
    for (int i = 0; i < NDB; ++i) o[i] *= alpha;
    m_base = m_new;
  }
  return (m_base == ATTN_NEG_INF) ? 0.f : m_base;
}

// s becomes P = exp2(logit - base) and its row sum is added to l; FDOM: s
// holds the cap output f (logit = fma(f, Kf, C2)), else the logit itself.
template <bool FDOM, int NKB>
__device__ __forceinline__ void fwd_exp(f32x16 (&s)[NKB], float base, const RowC& rc, float& l_run) {
  const float c2b = rc.C2 - base;
  // four partial sums: a single running sum would be one dependent chain
  float ls[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = FDOM ? fast_exp2(__builtin_fmaf(s[kb][r], rc.Kf, c2b)) : fast_exp2(s[kb][r] - base);
      ls[r & 3] += p;
      s[kb][r] = p;
    }
  }
  l_run += (ls[0] + ls[1]) + (ls[2] + ls[3]);
}

template <int D, int CAP, bool PRECISE>
__global__ __launch_bounds__(NTHREADS, ATTN_FWD_WAVES_PER_SIMD) void fwd_bf16_kernel(KArgs a) {
  constexpr int BN = BN16;
  using KT = BTile<BN, D, NWAVES, ATTN_LAUNDER_FWD>;
  constexpr int NKB = BN / 32, NDB = D / 32, NT16 = D / 16;

  __shared__ __attribute__((aligned(1024))) char sK[2][KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char sV[2][KT::BYTES];
  __shared__ int sSeg[2][BN];
  __shared__ unsigned char sFlag[MAX_TILES];
  __shared__ unsigned char sMixed[MAX_TILES];
  __shared__ int sRange[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= a.n_items) return;
  __shared__ int sOrd[64];
  const RowItem it = decode_row_item(a, item, wave, l32, ranker_row_order(a, tid, sOrd) ? sOrd : nullptr);
  const int L = a.L, b = it.b, qrow = it.qrow;
  const bool row_ok = qrow < L;

  const long q_rs = (long)a.Hq * D, kv_rs = (long)a.Hkv * D;
  const uint32_t kv_rsb = (uint32_t)(kv_rs * sizeof(bf16));   // K, V row stride in bytes
  const typename KT::Lane kln = KT::lane_of(kv_rsb, lane, wave);
  const bf16* Qb = (const bf16*)a.q + ((long)b * L * a.Hq + it.hq) * D;
  const bf16* Kb = (const bf16*)a.k + ((long)b * L * a.Hkv + it.hkv) * D;
  const bf16* Vb = (const bf16*)a.v + ((long)b * L * a.Hkv + it.hkv) * D;

  const MaskSpec ms = load_mask_spec(a, b);
  const bool has_seg = ms.has_seg;
  const bool seg_any = __builtin_amdgcn_readfirstlane((int)has_seg) != 0;
  const int* segb = has_seg ? a.seg + (long)b * L : nullptr;
  const QMask qm = query_mask(qrow, ms);

  bf16x8 qf[NT16];
#pragma unroll
  for (int t = 0; t < NT16; ++t) qf[t] = global_frag<bf16>(Qb + (long)qrow * q_rs + 16 * t + 8 * hh, row_ok);
  const float tmp = (a.temp != nullptr && row_ok) ? a.temp[(long)b * L + qrow] : 1.f;
  const RowC rc = row_consts(a, tmp, 0.f);
  // every row of the wave has a logit slope of the expected sign (temperature
  // >= 0, not NaN): full tiles may then take the row maximum over f
  const bool mono = __builtin_amdgcn_readfirstlane(
                        (int)(__ballot(!(rc.Kf * CapSlope<CAP>::value >= 0.f)) == 0)) != 0;
  const int seg_q = (has_seg && row_ok) ? segb[qrow] : 0;

  int t_lo = 0, t_hi = 0;
  const bool any = key_tile_range(it.q0, it.q1, BN, ms, &t_lo, &t_hi);
  if (has_seg && any) segment_flags(segb, it.q0, it.q1, t_lo, t_hi, BN, L, tid, sFlag, sMixed, sRange);
  auto next_needed = [&](int t) -> int {
    for (; t < t_hi; ++t) {
      if (tile_class(it.q0, it.q1, t * BN, t * BN + BN, ms) == TILE_EMPTY) continue;
      if (has_seg && !sFlag[t - t_lo]) continue;
      return t;
    }
    return -1;
  };
  int pseg = -1;
  auto issue = [&](int j, int st) {
    KT::issue(lds_offset(sK[st]), Kb + (long)(j * BN) * kv_rs, kv_rsb, L - j * BN, kln, wave);
    KT::issue(lds_offset(sV[st]), Vb + (long)(j * BN) * kv_rs, kv_rsb, L - j * BN, kln, wave);
  };
  // load i of this wave's 2 PER_WAVE loads of the K and V tiles of key tile j
  auto issue_one = [&](int j, int st, int i) {
    if (i < KT::PER_WAVE)
      KT::issue_one(lds_offset(sK[st]), Kb + (long)(j * BN) * kv_rs, kv_rsb, L - j * BN, kln, wave, i);
    else
      KT::issue_one(lds_offset(sV[st]), Vb + (long)(j * BN) * kv_rs, kv_rsb, L - j * BN, kln, wave,
                    i - KT::PER_WAVE);
  };
  constexpr int NDMA = 2 * KT::PER_WAVE;
  auto load_seg = [&](int j) {
    if (has_seg && tid < BN) pseg = (j * BN + tid < L) ? segb[j * BN + tid] : -1;
  };
  // the key segment ids go to LDS at the end of the step, after their load's
  // latency has passed
  auto store_seg = [&](int st) {
    if (has_seg && tid < BN) sSeg[st][tid] = pseg;
  };

  float m_base = ATTN_NEG_INF, m_true = ATTN_NEG_INF, l_run = 0.f;
  f32x16 oacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) oacc[i] = f32x16{};

  int j = any ? next_needed(t_lo) : -1;
  if (j >= 0) {
    issue(j, 0);
    load_seg(j);
    store_seg(0);
  }
  wait_vmcnt<0>();
  __syncthreads();
  // the loop body once per LDS stage, so that every fragment address is a
  // per-lane register plus an immediate offset
  auto step = [&](auto STC) {
    constexpr int st = decltype(STC)::value;
    const int jn = next_needed(j + 1);
    // tile loaded during this step: the next one, or (without one) the
    // current tile again into the idle stage, which keeps the body branch-free
    const int jl = jn >= 0 ? jn : j;
    const int k0 = j * BN;
    const char* Kt = sK[st];
    const char* Vt = sV[st];
    f32x16 sacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = f32x16{};
    // LDS fragments of step t + 1 requested before the MFMAs of step t (see
    // the dK/dV kernel)
    bf16x8 fk[2][NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) fk[0][kb] = KT::row_frag(Kt, kb, 0, lane);
    mfma_phase(true);
#pragma unroll
    for (int t = 0; t < NT16; ++t) {
      const int cur = t & 1;
      if (t + 1 < NT16) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) fk[cur ^ 1][kb] = KT::row_frag(Kt, kb, t + 1, lane);
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) sacc[kb] = Elem<bf16>::mfma(fk[cur][kb], qf[t], sacc[kb]);
      if (t + 1 < NT16) __builtin_amdgcn_sched_group_barrier(0x100, NKB, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, NKB, 0);
      // the next tile's loads, spread over the reduction steps: sent in one
      // burst they keep the wave waiting at issue
#pragma unroll
      for (int i = t * NDMA / NT16; i < (t + 1) * NDMA / NT16; ++i) issue_one(jl, st ^ 1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_phase(false);
    load_seg(jl);
    // the tile class is the same on every lane; readfirstlane lets the compiler
    // branch on it instead of running every variant under an exec mask
    const int tcls = seg_tile_class(it.qw0, it.qw0 + 32, k0, k0 + BN, ms, j, t_lo, sMixed, sRange);
    float mx;
    const bool fdom = tcls == TILE_FULL && mono;
    if (fdom) {
      mx = fwd_caps<CAP>(sacc, a, rc);
    } else if (tcls == TILE_FULL) {
      mx = fwd_logits<false, false, CAP>(sacc, a, rc, qm, k0, hh, nullptr, 0);
    } else if (!seg_any) {
      mx = fwd_logits<true, false, CAP>(sacc, a, rc, qm, k0, hh, nullptr, 0);
    } else {
      mx = fwd_logits<true, true, CAP>(sacc, a, rc, qm, k0, hh, sSeg[st], seg_q);
    }
    const float base = fwd_rescale(oacc, mx, m_base, m_true, l_run);
    if (fdom) {
      fwd_exp<true>(sacc, base, rc, l_run);
    } else {
      fwd_exp<false>(sacc, base, rc, l_run);
    }
    mfma_phase(true);
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      // With PRECISE, P enters as hi + lo bf16 parts so that O (and the delta
      // the backward derives from it) carries no bf16 rounding of P.
      bf16x8 phi, plo;
      if (PRECISE) {
        Elem<bf16>::split_acc(sacc[t / 2], 8 * (t % 2), phi, plo);
      } else {
        phi = Elem<bf16>::from_acc(sacc[t / 2], 8 * (t % 2));
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 va = KT::tr_frag(Vt, db, t, lane);
        oacc[db] = Elem<bf16>::mfma(va, phi, oacc[db]);
        if (PRECISE) oacc[db] = Elem<bf16>::mfma(va, plo, oacc[db]);
      }
    }
    mfma_phase(false);
    if (jn >= 0) store_seg(st ^ 1);
    wait_vmcnt<0>();
    __syncthreads();
    j = jn;
  };
  while (j >= 0) {
    step(std::integral_constant<int, 0>{});
    if (j >= 0) step(std::integral_constant<int, 1>{});
  }

  const float l_tot = half_sum(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    float* orow = a.out0 + ((long)(b * L + qrow) * a.Hq + it.hq) * D;
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
      const long mi = ((long)b * a.Hq + it.hq) * L + qrow;
      const bool seen = m_true != ATTN_NEG_INF;
      a.out1[mi] = seen ? m_true * LN2_F : ATTN_NEG_INF;
      a.out2[mi] = seen ? l_tot * fast_exp2(m_base - m_true) : 0.f;
    }
  }
}

// ---------------------------------------------------------------------------
// dQ
// ---------------------------------------------------------------------------
// DT: also accumulate this row's share of the temperature gradient,
// sum_j dS'_ij c_ij with c = ln2 (kmul f + kadd) (the ln2 is applied once at
// the end).
template <bool MASKED, bool SEG, int CAP, bool DT, int NKB>
__device__ __forceinline__ void dq_elementwise(f32x16 (&s)[NKB], const f32x16 (&dp)[NKB], const KArgs& a,
                                               const RowC& rc, float dlt, const QMask& qm, int k0,
                                               int hh, const int* sseg, int seg_q, float& tacc) {
  using CapF = Cap<CAP, false>;
  const float nrd = -rc.R * dlt;
#pragma unroll
  for (int kb = 0; kb < NKB; ++kb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float aux;
      const float fx = CapF::f(s[kb][r], a, aux);
      float p = fast_exp2(__builtin_fmaf(fx, rc.Kf, rc.C2));
      if (MASKED) {
        const int koff = kb * 32 + prow(r, hh);
        bool vis = qmask_vis(qm, k0 + koff);
        if (SEG) vis = vis && sseg[koff] == seg_q;
        p = vis ? p : 0.f;
      }
      if (DT) {
        const float dsp = p * (dp[kb][r] - dlt);
        tacc = __builtin_fmaf(dsp, __builtin_fmaf(fx, a.kmul, a.kadd), tacc);
      }
      // R (dP - delta) as one fma against the row constant -R delta (the same
      // expression with and without DT, so dQ does not depend on it)
      s[kb][r] = (p * __builtin_fmaf(dp[kb][r], rc.R, nrd)) * CapF::g(aux, a);
    }
  }
}

template <int D, int CAP, bool PRECISE, bool DT>
__global__ __launch_bounds__(NTHREADS, 2) void dq_bf16_kernel(KArgs a) {
  constexpr int BN = BNQ16;
  using KT = BTile<BN, D, NWAVES, ATTN_LAUNDER_DQ>;
  constexpr int NKB = BN / 32, NDB = D / 32, NT16 = D / 16;

  __shared__ __attribute__((aligned(1024))) char sK[2][KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char sV[2][KT::BYTES];
  __shared__ int sSeg[2][BN];
  __shared__ unsigned char sFlag[MAX_TILES];
  __shared__ unsigned char sMixed[MAX_TILES];
  __shared__ int sRange[2];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= a.n_items) return;
  __shared__ int sOrd[64];
  const RowItem it = decode_row_item(a, item, wave, l32, ranker_row_order(a, tid, sOrd) ? sOrd : nullptr);
  const int L = a.L, b = it.b, qrow = it.qrow;
  const bool row_ok = qrow < L;

  const long q_rs = (long)a.Hq * D, kv_rs = (long)a.Hkv * D;
  const uint32_t kv_rsb = (uint32_t)(kv_rs * sizeof(bf16));   // K, V row stride in bytes
  const typename KT::Lane kln = KT::lane_of(kv_rsb, lane, wave);
  const bf16* Qb = (const bf16*)a.q + ((long)b * L * a.Hq + it.hq) * D;
  const bf16* dOb = (const bf16*)a.dout + ((long)b * L * a.Hq + it.hq) * D;
  const bf16* Kb = (const bf16*)a.k + ((long)b * L * a.Hkv + it.hkv) * D;
  const bf16* Vb = (const bf16*)a.v + ((long)b * L * a.Hkv + it.hkv) * D;

  const MaskSpec ms = load_mask_spec(a, b);
  const bool has_seg = ms.has_seg;
  const bool seg_any = __builtin_amdgcn_readfirstlane((int)has_seg) != 0;
  const int* segb = has_seg ? a.seg + (long)b * L : nullptr;
  const QMask qm = query_mask(qrow, ms);

  bf16x8 qf[NT16], df[NT16];
#pragma unroll
  for (int t = 0; t < NT16; ++t) {
    qf[t] = global_frag<bf16>(Qb + (long)qrow * q_rs + 16 * t + 8 * hh, row_ok);
    df[t] = global_frag<bf16>(dOb + (long)qrow * q_rs + 16 * t + 8 * hh, row_ok);
  }
  float lse2 = ATTN_POS_INF, dlt = 0.f, tmp = 1.f;
  if (row_ok) {
    row_residuals(a, ((long)b * a.Hq + it.hq) * L + qrow, lse2, dlt);
    if (a.temp != nullptr) tmp = a.temp[(long)b * L + qrow];
  }
  const RowC rc = row_consts(a, tmp, lse2);
  const int seg_q = (has_seg && row_ok) ? segb[qrow] : 0;

  int t_lo = 0, t_hi = 0;
  const bool any = key_tile_range(it.q0, it.q1, BN, ms, &t_lo, &t_hi);
  if (has_seg && any) segment_flags(segb, it.q0, it.q1, t_lo, t_hi, BN, L, tid, sFlag, sMixed, sRange);
  auto next_needed = [&](int t) -> int {
    for (; t < t_hi; ++t) {
      if (tile_class(it.q0, it.q1, t * BN, t * BN + BN, ms) == TILE_EMPTY) continue;
      if (has_seg && !sFlag[t - t_lo]) continue;
      return t;
    }
    return -1;
  };
  int pseg = -1;
  auto issue = [&](int j, int st) {
    KT::issue(lds_offset(sK[st]), Kb + (long)(j * BN) * kv_rs, kv_rsb, L - j * BN, kln, wave);
    KT::issue(lds_offset(sV[st]), Vb + (long)(j * BN) * kv_rs, kv_rsb, L - j * BN, kln, wave);
  };
  // load i of this wave's 2 PER_WAVE loads of the K and V tiles of key tile j
  auto issue_one = [&](int j, int st, int i) {
    if (i < KT::PER_WAVE)
      KT::issue_one(lds_offset(sK[st]), Kb + (long)(j * BN) * kv_rs, kv_rsb, L - j * BN, kln, wave, i);
    else
      KT::issue_one(lds_offset(sV[st]), Vb + (long)(j * BN) * kv_rs, kv_rsb, L - j * BN, kln, wave,
                    i - KT::PER_WAVE);
  };
  constexpr int NDMA = 2 * KT::PER_WAVE;
  auto load_seg = [&](int j) {
    if (has_seg && tid < BN) pseg = (j * BN + tid < L) ? segb[j * BN + tid] : -1;
  };
  // the key segment ids go to LDS at the end of the step, after their load's
  // latency has passed
  auto store_seg = [&](int st) {
    if (has_seg && tid < BN) sSeg[st][tid] = pseg;
  };

  float tacc = 0.f;
  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};

  int j = any ? next_needed(t_lo) : -1;
  if (j >= 0) {
    issue(j, 0);
    load_seg(j);
    store_seg(0);
  }
  wait_vmcnt<0>();
  __syncthreads();
  // the loop body once per LDS stage, so that every fragment address is a
  // per-lane register plus an immediate offset
  auto step = [&](auto STC) {
    constexpr int st = decltype(STC)::value;
    const int jn = next_needed(j + 1);
    // tile loaded during this step: the next one, or (without one) the
    // current tile again into the idle stage, which keeps the body branch-free
    const int jl = jn >= 0 ? jn : j;
    const int k0 = j * BN;
    const char* Kt = sK[st];
    const char* Vt = sV[st];
    f32x16 sacc[NKB], pacc[NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) sacc[kb] = pacc[kb] = f32x16{};
    // LDS fragments of reduction step t + 1 requested before the MFMAs of
    // step t; the fences keep the compiler from sinking them next to their use
    bf16x8 fk[2][NKB], fv[2][NKB];
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      fk[0][kb] = KT::row_frag(Kt, kb, 0, lane);
      fv[0][kb] = KT::row_frag(Vt, kb, 0, lane);
    }
    mfma_phase(true);
#pragma unroll
    for (int t = 0; t < NT16; ++t) {
      const int cur = t & 1;
      if (t + 1 < NT16) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          fk[cur ^ 1][kb] = KT::row_frag(Kt, kb, t + 1, lane);
          fv[cur ^ 1][kb] = KT::row_frag(Vt, kb, t + 1, lane);
        }
      }
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        sacc[kb] = Elem<bf16>::mfma(fk[cur][kb], qf[t], sacc[kb]);
        pacc[kb] = Elem<bf16>::mfma(fv[cur][kb], df[t], pacc[kb]);
      }
      if (t + 1 < NT16) __builtin_amdgcn_sched_group_barrier(0x100, 2 * NKB, 0);
      __builtin_amdgcn_sched_group_barrier(0x008, 2 * NKB, 0);
      // the next tile's loads, spread over the reduction steps
#pragma unroll
      for (int i = t * NDMA / NT16; i < (t + 1) * NDMA / NT16; ++i) issue_one(jl, st ^ 1, i);
      __builtin_amdgcn_sched_barrier(0);
    }
    mfma_phase(false);
    load_seg(jl);
    // the tile class is the same on every lane; readfirstlane lets the compiler
    // branch on it instead of running every variant under an exec mask
    const int tcls = seg_tile_class(it.qw0, it.qw0 + 32, k0, k0 + BN, ms, j, t_lo, sMixed, sRange);
    if (tcls == TILE_FULL) {
      dq_elementwise<false, false, CAP, DT>(sacc, pacc, a, rc, dlt, qm, k0, hh, nullptr, 0, tacc);
    } else if (!seg_any) {
      dq_elementwise<true, false, CAP, DT>(sacc, pacc, a, rc, dlt, qm, k0, hh, nullptr, 0, tacc);
    } else {
      dq_elementwise<true, true, CAP, DT>(sacc, pacc, a, rc, dlt, qm, k0, hh, sSeg[st], seg_q, tacc);
    }
    mfma_phase(true);
#pragma unroll
    for (int t = 0; t < BN / 16; ++t) {
      bf16x8 hi, lo;
      if (PRECISE) {
        Elem<bf16>::split_acc(sacc[t / 2], 8 * (t % 2), hi, lo);
      } else {
        hi = Elem<bf16>::from_acc(sacc[t / 2], 8 * (t % 2));
      }
#pragma unroll
      for (int db = 0; db < NDB; ++db) {
        const bf16x8 ka = KT::tr_frag(Kt, db, t, lane);
        dqacc[db] = Elem<bf16>::mfma(ka, hi, dqacc[db]);
        if (PRECISE) dqacc[db] = Elem<bf16>::mfma(ka, lo, dqacc[db]);
      }
    }
    mfma_phase(false);
    if (jn >= 0) store_seg(st ^ 1);
    wait_vmcnt<0>();
    __syncthreads();
    j = jn;
  };
  while (j >= 0) {
    step(std::integral_constant<int, 0>{});
    if (j >= 0) step(std::integral_constant<int, 1>{});
  }

  if (DT) {
    const float tot = half_sum(tacc);   // the row's two key halves
    if (row_ok && hh == 0) a.out3[((long)b * a.Hq + it.hq) * L + qrow] = tot * LN2_F;
  }
  if (row_ok) {
    float* drow = a.out0 + ((long)(b * L + qrow) * a.Hq + it.hq) * D;
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

// ---------------------------------------------------------------------------
// dQ from stored dS
// ---------------------------------------------------------------------------
// dQ^T += K^T dS^T over the visited key tiles of two adjacent query tiles,
// dS taken from the tiles the dK/dV kernel stored (WDS): no recomputation of
// S, P or dP and no element work, so the kernel streams the stored tiles from
// HBM.  Both operands reduce over keys and are read transposed from LDS
// (ds_read_b64_tr_b16): the K tile (columns = d) and the dS tile in its
// stored order (columns = queries; wave w of a half takes its 32).
//
// A work-group is eight waves: waves 0-3 hold query tile 2p, waves 4-7 tile
// 2p + 1 of the same (batch row, query head), and the two halves share every
// K tile.  The K loads cost per instruction, wherever they hit: in a
// stand-alone copy of the load pattern on the long-context workload they took
// 15% of the dS stream's time with one query tile per work-group and 4% with
// two.  Two such work-groups fit a CU (about 74 KB of LDS each), so that one's
// wait, barrier and LDS latency hide behind the other's MFMAs; with one
// eight-wave work-group per CU the kernel was slower than with one query tile
// per work-group.  The key tiles either half visits are listed once per
// work-group, each entry with one visibility bit per half; a step covers
// DQS_BN keys of one listed tile.  Every wave issues the same loads in the
// same order at every step, so that one vmcnt wait before the barrier finds
// the step's tiles done: a half that does not visit the step's tile loads
// one of its own visited parts (or, without any, one of the other half's)
// into its stage and skips its MFMAs.  Step n loads K of step n + 1 and dS
// of step n + 2 (past the last step the last one is fetched again), so at
// step n's wait only dS(n + 1) was issued after K(n).  A shallow ring is
// enough: the dS stream alone reached the same rate with 3 stages as with
// 8.  The dS tiles, read once, are loaded non-temporal so that their stream
// does not push out of L2 the K tiles that are read again.
constexpr int DQS_BN = 32;                        // keys per step (a quarter of a stored tile)
constexpr int DQS_KST = 2;                        // K stages
constexpr int DQS_SST = 3;                        // dS stages (each: both halves)
constexpr int DQS_NW = 2 * NWAVES;                // waves per work-group
constexpr int DQS_THREADS = 64 * DQS_NW;
constexpr int DQS_FLAGS = ATTN_MAX_SEQ_LEN_SEGMENTS / DS_T;

// Work item -> (batch row, KV head, query head, query-tile pair p), with the
// row order of decode_row_item (pairs in place of query tiles; causal pairs
// longest first).
struct PairItem {
  int b, hkv, hq, p;
};
__device__ __forceinline__ PairItem decode_pair_item(const KArgs& a, int item, int P, const int* ord) {
  PairItem it;
  int rest;
  if (ord != nullptr) {
    const int R = a.n_items / 8, per_b = R / a.B, run = item / R, loc = item - run * R;
    it.b = ord[loc / per_b];
    rest = run * per_b + loc % per_b;
  } else {
    it.b = item % a.B;
    rest = item / a.B;
  }
  const int g = rest % a.G;
  rest /= a.G;
  const int p_rev = rest % P;
  it.hkv = rest / P;
  it.p = a.causal ? (P - 1 - p_rev) : p_rev;
  it.hq = it.hkv * a.G + g;
  return it;
}

template <int D>
__global__ __launch_bounds__(DQS_THREADS, 2) void dq_ds_bf16_kernel(KArgs a) {
  constexpr int BN = DQS_BN, KST = DQS_KST, SST = DQS_SST, PARTS = DS_T / BN;
  constexpr int PSH = PARTS == 4 ? 2 : 1;   // log2(PARTS)
  static_assert(PARTS == 2 || PARTS == 4, "a stored tile splits into 2 or 4 steps");
  // waves that load K: all eight where the tile splits into eight 1 KB loads
  constexpr int KNW = (BN * D * 2) / 1024 >= DQS_NW ? DQS_NW : NWAVES;
  using KT = BTile<BN, D, KNW>;
  using ST = BTile<BN, DS_T, NWAVES>;   // one half's part of a dS stage
  constexpr int NDB = D / 32, NK = KT::PER_WAVE, NS = ST::PER_WAVE;
  static_assert(BM == DS_T, "a half's query tile is one stored query tile");
  static_assert(KST == 2 && SST == 3, "load order of the two rings");
  static_assert(BN % 32 == 0 && ST::BYTES == BN * DS_T * 2, "dS load pattern");

  __shared__ __attribute__((aligned(1024))) char sK[KST][KT::BYTES];
  __shared__ __attribute__((aligned(1024))) char sS[SST][2][ST::BYTES];
  __shared__ unsigned char sFlag[2][DQS_FLAGS];
  __shared__ unsigned char sFlag2[2][DQS_FLAGS];
  __shared__ unsigned char sMixed[2][DQS_FLAGS];
  __shared__ unsigned short sList[ATTN_MAX_SEQ_LEN / DS_T];   // tile - t_min | visibility << 14
  __shared__ int sRange[2][3];
  __shared__ int sFirst1;
  __shared__ int sOrd[64];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = wave >> 2, w4 = wave & 3;
  const int l32 = lane & 31, hh = lane >> 5;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= a.n_items) return;
  const int P = (a.n_q_tiles + 1) / 2;
  const PairItem it = decode_pair_item(a, item, P, ranker_row_order(a, tid, sOrd) ? sOrd : nullptr);
  const int L = a.L, b = it.b;

  const long kv_rs = (long)a.Hkv * D;
  const uint32_t kv_rsb = (uint32_t)(kv_rs * sizeof(bf16));
  const bool kload = wave < KNW;
  const typename KT::Lane kln = KT::lane_of(kv_rsb, lane, kload ? wave : 0);
  const bf16* Kb = (const bf16*)a.k + ((long)b * L * a.Hkv + it.hkv) * D;
  const DsBand band = ds_band(L, a.causal, a.window);
  const MaskSpec ms = load_mask_spec(a, b);
  const bool has_seg = ms.has_seg;
  const int* segb = has_seg ? a.seg + (long)b * L : nullptr;

  // the two query tiles (the second may lie past the sequence)
  int qtx[2], q0x[2], q1x[2], tlo[2], thi[2];
#pragma unroll
  for (int x = 0; x < 2; ++x) {
    qtx[x] = 2 * it.p + x;
    q0x[x] = qtx[x] * BM;
    q1x[x] = imin(q0x[x] + BM, L);
    const bool live = q0x[x] < L;
    tlo[x] = live ? ds_lo(qtx[x], band) : 0;
    thi[x] = live ? ds_hi(qtx[x], band) : 0;
  }
  const bool live1 = q0x[1] < L;
  const int tmin = live1 ? imin(tlo[0], tlo[1]) : tlo[0];
  const int tmax = live1 ? imax(thi[0], thi[1]) : thi[0];
  // (segment_flags strides by NTHREADS: the threads past it repeat writes of
  // the same flag values, and only the first BM threads take part in the id
  // range, so the 512-thread work-group computes the same tables)
  if (has_seg) {
#pragma unroll
    for (int x = 0; x < 2; ++x)
      if (x == 0 || live1)
        segment_flags(segb, q0x[x], q1x[x], tmin, tmax, DS_T, L, tid, sFlag[x], sMixed[x], sRange[x],
                      sFlag2[x]);
  }
  // The blocks the dK/dV kernel visited (and stored), per half: the same tile
  // class and symmetric segment test, evaluated from the query side once, by
  // wave 0, into a compact list of key tiles (the loop then only indexes it).
  if (wave == 0) {
    int cnt = 0, first0 = -1, first1 = -1;   // each half's first visited tile
    for (int t0 = tmin; t0 < tmax; t0 += 64) {
      const int t = t0 + lane;
      int vis = 0;
#pragma unroll
      for (int x = 0; x < 2; ++x) {
        bool v = t >= tlo[x] && t < thi[x] &&
                 tile_class(q0x[x], q1x[x], t * DS_T, t * DS_T + DS_T, ms) != TILE_EMPTY;
        if (v && has_seg) v = sFlag[x][t - tmin] && sFlag2[x][t - tmin];
        vis |= v ? (1 << x) : 0;
      }
      const uint64_t m = __ballot(vis != 0);
      const uint64_t m0 = __ballot(vis & 1), m1 = __ballot(vis & 2);
      if (first0 < 0 && m0 != 0) first0 = t0 + __builtin_ctzll(m0);
      if (first1 < 0 && m1 != 0) first1 = t0 + __builtin_ctzll(m1);
      const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                           __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
      if (vis != 0) sList[pos] = (unsigned short)((t - tmin) | (vis << 14));
      cnt += __builtin_popcountll(m);
    }
    if (lane == 0) {
      sRange[0][2] = cnt;
      sRange[1][2] = first0;
      sFirst1 = first1;
    }
  }
  __syncthreads();
  const int ntiles = sRange[0][2];
  // a step is one BN-key part of a listed tile; the parts of the sequence's
  // last tile that start at or past L are dropped
  const int last = ntiles > 0 ? tmin + (sList[ntiles - 1] & 0x3fff) : 0;
  const int last_parts = imin(PARTS, (L - last * DS_T + BN - 1) / BN);
  const int nsteps = ntiles > 0 ? PARTS * (ntiles - 1) + last_parts : 0;

  // this half's dS: its band's first slot, and a part it can always load (its
  // first visited one, else the other half's first visited one)
  const bf16* Sx[2];
#pragma unroll
  for (int x = 0; x < 2; ++x)
    Sx[x] = (const bf16*)a.ds +
            (((long long)b * a.Hq + it.hq) * a.ds_slots + (q0x[x] < L ? ds_offset(qtx[x], band) : 0)) *
                DS_ELEMS;
  const bf16* fb = nullptr;
  if (nsteps > 0) {
    const int first[2] = {sRange[1][2], sFirst1};
    const int xs = first[half] >= 0 ? half : half ^ 1;
    fb = Sx[xs] + (long long)(first[xs] - tlo[xs]) * DS_ELEMS;
  }
  const bf16* Sh = Sx[half];
  const int tloh = tlo[half];

  auto issue_k = [&](int n, int stg, int e) {
    if (!kload) return;
    const int kt = tmin + (e & 0x3fff);
    const int kr0 = kt * DS_T + (n & (PARTS - 1)) * BN;
#pragma unroll
    for (int i = 0; i < NK; ++i)
      KT::issue_one(lds_offset(sK[stg]), Kb + (long)kr0 * kv_rs, kv_rsb, L - kr0, kln, wave, i);
  };
  // The dS ring holds each step's BN keys (BN / 32 groups of the stored tile,
  // contiguous) as stored: 1 KB loads, LDS image = global image.
  auto issue_s = [&](int n, int stg, int e) {
    const bool vis = (e >> (14 + half)) & 1;
    const int kt = tmin + (e & 0x3fff);
    const bf16* g = vis ? Sh + ((long long)(kt - tloh) * DS_ELEMS + (long long)(n & (PARTS - 1)) * BN * DS_T)
                        : fb;
#pragma unroll
    for (int i = 0; i < NS; ++i) {   // read once: non-temporal, K stays in L2
      const uint32_t j = (uint32_t)(w4 + NWAVES * i);
      const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane(lds_offset(sS[stg][half]) + j * 1024);
      dma16_nt(uniform_ptr(g), j * 1024 + 16 * (uint32_t)lane, m0);
    }
  };
  // B operand of dQ^T += K^T dS^T for step t: this wave's 32 queries
  // (columns) and the keys of K's LDS rows 16 t .. 16 t + 15 (rows; the K
  // tile holds key pi32(x) in row x), gathered from the stored order by
  // transposed reads (see BTile::tr_frag for the lane roles).
  auto ds_frag = [&](const char* lds, int t) -> bf16x8 {
    const int h = lane >> 5, mh = (lane >> 4) & 1, e = (lane & 15) >> 2, s = lane & 3;
    const int c = 4 * w4 + 2 * mh + (s >> 1);
    const int r1 = 16 * t + 4 * h + e, r2 = r1 + 8;
    const int k1 = (r1 & ~31) | pi32(r1 & 31), k2 = (r2 & ~31) | pi32(r2 & 31);
    const char* a1 = lds + (k1 >> 5) * 8192 + ds_chunk_offset(k1 & 31, c) + ((s & 1) << 3);
    const char* a2 = lds + (k2 >> 5) * 8192 + ds_chunk_offset(k2 & 31, c) + ((s & 1) << 3);
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a1);
    const s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a2);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
    return __builtin_bit_cast(bf16x8, v);
  };

  f32x16 dqacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) dqacc[i] = f32x16{};

  if (nsteps > 0) {
    // prologue: dS(0), K(0), dS(1); step n loads K(n+1) and dS(n+2), so the
    // only loads after K(n) at step n's wait are those of dS(n+1) (waves
    // without K loads: the same); step numbers past the last step repeat the
    // last one
    const int nl = nsteps - 1;
    auto entry = [&](int n) -> int { return sList[n >> PSH]; };
    issue_s(0, 0, entry(0));
    issue_k(0, 0, entry(0));
    issue_s(imin(1, nl), 1, entry(imin(1, nl)));
    // the list entries of the next step's loads, read one step ahead so that
    // their LDS latency passes during a step's MFMAs
    int ek = entry(imin(1, nl)), es = entry(imin(2, nl));
    int ks = 0, ss = 0;   // stages of the current step
    for (int n = 0; n < nsteps; ++n) {
      wait_vmcnt<NS>();
      __syncthreads();
      const int ec = entry(n);
      issue_k(imin(n + 1, nl), ks ^ 1, ek);
      issue_s(imin(n + 2, nl), ss == 0 ? 2 : ss - 1, es);
      ek = entry(imin(n + 2, nl));
      es = entry(imin(n + 3, nl));
      if ((ec >> (14 + half)) & 1) {
        const char* Kt = sK[ks];
        const char* St = sS[ss][half];
#pragma unroll
        for (int t = 0; t < BN / 16; ++t) {
          const bf16x8 sf = ds_frag(St, t);
#pragma unroll
          for (int db = 0; db < NDB; ++db) {
            const bf16x8 ka = KT::tr_frag(Kt, db, t, lane);
            dqacc[db] = Elem<bf16>::mfma(ka, sf, dqacc[db]);
          }
        }
      }
      ks = ks + 1 == KST ? 0 : ks + 1;
      ss = ss + 1 == SST ? 0 : ss + 1;
    }
    wait_vmcnt<0>();
  }

  const int qrow = q0x[half] + 32 * w4 + l32;
  if (qrow < L) {
    float* drow = a.out0 + ((long)(b * L + qrow) * a.Hq + it.hq) * D;
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

// ---------------------------------------------------------------------------
// dK / dV
// ---------------------------------------------------------------------------
template <bool MASKED, bool SEG, int CAP, int NQB>
__device__ __forceinline__ void dkv_elementwise(f32x16 (&s)[NQB], f32x16 (&dp)[NQB], const KArgs& a,
                                                const float* cKf, const float* cC2, const float* cNrd,
                                                const float* cR, const KMask& km, int q0, int hh,
                                                const int* sseg, int seg_k) {
  using CapF = Cap<CAP, false>;
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qoff = qb * 32 + prow(r, hh);
      const float Kf = cKf[qoff], C2 = cC2[qoff], nrd = cNrd[qoff], R = cR[qoff];
      float aux;
      float p = fast_exp2(__builtin_fmaf(CapF::f(s[qb][r], a, aux), Kf, C2));
      if (MASKED) {
        bool vis = kmask_vis(km, q0 + qoff);
        if (SEG) vis = vis && sseg[qoff] == seg_k;
        p = vis ? p : 0.f;
      }
      // R (dP - delta) as one fma against the query constant -R delta
      dp[qb][r] = (p * __builtin_fmaf(dp[qb][r], R, nrd)) * CapF::g(aux, a);
      s[qb][r] = p;
    }
  }
}

// One dV / dK unit: dv += oa x pb, dk += qa x hi (and + qa x lo with the
// split dS), in one asm block so that the two accumulators stay in AGPRs
// while the S / dP chains of the same loop use the VGPR form of the MFMA
// (this source is built with that form as the default).  Left to the compiler,
// the dK / dV accumulators were moved between the two register files on every
// step.  The compiler does not see into the block, so it carries its own wait
// states: an operand written by a VALU instruction (the bf16 packing, or the
// zeroing of an accumulator) needs two before an MFMA reads it, which the
// leading s_nop 1 gives; the dK MFMA that follows overwrites exactly its own
// srcC with the same opcode and needs none.  The accumulators are read only
// after the step loop, behind dkv_acc_fence.
template <bool PRECISE>
__device__ __forceinline__ void dvdk_mfma(f32x16& dv, f32x16& dk, const bf16x8& oa, const bf16x8& pb,
                                          const bf16x8& qa, const bf16x8& hi, const bf16x8& lo) {
  if (PRECISE) {
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %4, %6, %1"
        : "+a"(dv), "+a"(dk)
        : "v"(oa), "v"(pb), "v"(qa), "v"(hi), "v"(lo));
  } else {
    asm volatile(
        "s_nop 1\n\t"
        "v_mfma_f32_32x32x16_bf16 %0, %2, %3, %0\n\t"
        "v_mfma_f32_32x32x16_bf16 %1, %4, %5, %1"
        : "+a"(dv), "+a"(dk)
        : "v"(oa), "v"(pb), "v"(qa), "v"(hi));
  }
}

// Before anything reads an accumulator that dvdk_mfma wrote: an MFMA result
// read by a VALU or memory instruction needs up to about a dozen wait states;
// the first block gives 24.  Each accumulator then passes through an empty
// block of its own, ordered after the first, so that no read of it can be
// scheduled above the wait.  (One block with all of them as operands made the
// register allocator copy them between AGPRs first, reads the wait would not
// cover.)
template <int NDB>
__device__ __forceinline__ void dkv_acc_fence(f32x16 (&dk)[NDB], f32x16 (&dv)[NDB]) {
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    asm volatile("" : "+a"(dk[i]));
    asm volatile("" : "+a"(dv[i]));
  }
}

// WDS: also store this step's bf16 dS, in the order of ds_chunk_offset, into
// the stored-dS workspace (slot of block (query tile, key tile), see ds_slot), for the dQ
// kernel of the stored-dS backward; the segment skip then takes the symmetric
// test of segment_flags, which that kernel evaluates the same way.
template <int D, int CAP, bool PRECISE, bool WDS>
__global__ __launch_bounds__(NTHREADS, 1) void dkv_bf16_kernel(KArgs a) {
  static_assert(!(WDS && PRECISE), "the stored dS is a single bf16");
  static_assert(!WDS || (BQ16 == DS_T && BKV == DS_T), "stored tiles are the dK/dV query and key tiles");
  constexpr int BQ = BQ16;
  using QT = BTile<BQ, D, NWAVES, ATTN_LAUNDER_DKV>;
  constexpr int NQB = BQ / 32, NDB = D / 32, NT16 = D / 16;

  __shared__ __attribute__((aligned(1024))) char sQ[2][QT::BYTES];
  __shared__ __attribute__((aligned(1024))) char sO[2][QT::BYTES];   // dO tile
  __shared__ __attribute__((aligned(16))) float sKf[2][BQ];
  __shared__ __attribute__((aligned(16))) float sC2[2][BQ];
  __shared__ __attribute__((aligned(16))) float sNrd[2][BQ];   // -R delta
  __shared__ __attribute__((aligned(16))) float sR[2][BQ];
  __shared__ int sSeg[2][BQ];
  __shared__ unsigned char sFlag[MAX_TILES];
  __shared__ unsigned char sMixed[MAX_TILES];
  __shared__ unsigned char sFlag2[WDS ? MAX_TILES : 1];
  __shared__ int sRange[2];
  __shared__ int sPlan[DKV_PLAN_MAX];
  __shared__ int sPlanN;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hh = lane >> 5, l32 = lane & 31;
  const int item = xcd_remap(blockIdx.x, gridDim.x);
  if (item >= a.n_items) return;

  const int L = a.L, G = a.G;
  // batch row fastest (see decode_row_item), then key tile, then KV head
  const int b = item % a.B;
  const int rest = item / a.B;
  const int kt = rest % a.n_kv_tiles;
  const int hkv = rest / a.n_kv_tiles;
  const int k0 = kt * BKV, k1 = imin(k0 + BKV, L);
  const int kw0 = k0 + wave * 32;
  const int krow = kw0 + l32;
  const bool key_ok = krow < L;

  const long q_rs = (long)a.Hq * D, kv_rs = (long)a.Hkv * D;
  const uint32_t q_rsb = (uint32_t)(q_rs * sizeof(bf16));     // Q, dO row stride in bytes
  const typename QT::Lane qln = QT::lane_of(q_rsb, lane, wave);
  const bf16* Kb = (const bf16*)a.k + ((long)b * L * a.Hkv + hkv) * D;
  const bf16* Vb = (const bf16*)a.v + ((long)b * L * a.Hkv + hkv) * D;

  const MaskSpec ms = load_mask_spec(a, b);
  const bool has_seg = ms.has_seg;
  const bool seg_any = __builtin_amdgcn_readfirstlane((int)has_seg) != 0;
  const int* segb = has_seg ? a.seg + (long)b * L : nullptr;
  const KMask km = key_mask(krow, ms);

  bf16x8 kf[NT16], vf[NT16];
#pragma unroll
  for (int t = 0; t < NT16; ++t) {
    kf[t] = global_frag<bf16>(Kb + (long)krow * kv_rs + 16 * t + 8 * hh, key_ok);
    vf[t] = global_frag<bf16>(Vb + (long)krow * kv_rs + 16 * t + 8 * hh, key_ok);
  }
  const int seg_k = (has_seg && key_ok) ? segb[krow] : 0;

  int t_lo = 0, t_hi = 0;
  const bool any = query_tile_range(k0, k1, BQ, ms, &t_lo, &t_hi);
  if (has_seg && any)
    segment_flags(segb, k0, k1, t_lo, t_hi, BQ, L, tid, sFlag, sMixed, sRange, WDS ? sFlag2 : nullptr);
  // The step plan: the query tiles this key block visits, in order, each with
  // the tile class every wave's 32 keys see, built once by wave 0 (one
  // ballot per 64 tiles), so that a step only reads its entry.  The steps
  // are the plan's tiles for each group head in turn.  Entry: tile index
  // (bits 0-15), then 2 bits of class per wave.
  if (wave == 0) {
    int cnt = 0;
    if (any) {
      for (int t0 = t_lo; t0 < t_hi; t0 += 64) {
        const int t = t0 + lane;
        bool vis = t < t_hi && tile_class(t * BQ, t * BQ + BQ, k0, k1, ms) != TILE_EMPTY;
        if (vis && has_seg) vis = sFlag[t - t_lo] && (!WDS || sFlag2[t - t_lo]);
        int e = t;
        if (vis) {
          MaskSpec mt = ms;
          if (ms.has_seg && sRange[0] == sRange[1] && !sMixed[t - t_lo]) mt.has_seg = false;
#pragma unroll
          for (int w = 0; w < NWAVES; ++w)
            e |= tile_class(t * BQ, t * BQ + BQ, k0 + 32 * w, k0 + 32 * w + 32, mt) << (16 + 2 * w);
        }
        const uint64_t m = __ballot(vis);
        const int pos = cnt + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                             __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        if (vis && pos < DKV_PLAN_MAX) sPlan[pos] = e;
        cnt += __builtin_popcountll(m);
      }
    }
    if (lane == 0) sPlanN = cnt;
  }
  __syncthreads();
  // (never above DKV_PLAN_MAX while L <= ATTN_MAX_SEQ_LEN; clamped all the same)
  const int nplan = imin(__builtin_amdgcn_readfirstlane(sPlanN), DKV_PLAN_MAX);
  auto plan_entry = [&](int i) -> int { return __builtin_amdgcn_readfirstlane(sPlan[i]); };
  // Per-query inputs of the next step (m, l, delta, temperature, segment id):
  // each wave loads BQ / NWAVES of them into registers when the step's tile
  // loads are issued, and derives the constants from them only after the
  // current step's compute, so that their latency hides behind it.
  constexpr int CPW = BQ / NWAVES;
  static_assert(CPW <= 64 && BQ % NWAVES == 0, "constant fetch layout");
  const int cq = wave * CPW + lane;
  const bool cthr = lane < CPW;
  float pM = 0.f, pL = 0.f, pD = 0.f, pT = 1.f;
  int pSeg = -1;
  auto fetch_consts = [&](int g, int t) {
    if (cthr) {
      const int hq = hkv * G + g;
      const int qq = t * BQ + cq;
      pL = 0.f;
      pT = 1.f;
      pSeg = -1;
      if (qq < L) {
        const long idx = ((long)b * a.Hq + hq) * L + qq;
        pM = a.m_in[idx];
        pL = a.l_in[idx];
        pD = a.delta_in[idx];
        if (a.temp != nullptr) pT = a.temp[(long)b * L + qq];
        if (has_seg) pSeg = segb[qq];
      }
    }
  };
  auto store_consts = [&](int stg) {
    if (cthr) {
      float lse2, dlt;
      residuals_from(pM, pL, pD, a.zw, lse2, dlt);
      const RowC rc = row_consts(a, pT, lse2);
      sKf[stg][cq] = rc.Kf;
      sC2[stg][cq] = rc.C2;
      sNrd[stg][cq] = -rc.R * dlt;
      sR[stg][cq] = rc.R;
      sSeg[stg][cq] = pSeg;
    }
  };
  auto issue = [&](int g, int t, int stg) {
    const int hq = hkv * G + g;
    const int qb0 = t * BQ;
    QT::issue(lds_offset(sQ[stg]), (const bf16*)a.q + (((long)b * L + qb0) * a.Hq + hq) * D, q_rsb,
              L - qb0, qln, wave);
    QT::issue(lds_offset(sO[stg]), (const bf16*)a.dout + (((long)b * L + qb0) * a.Hq + hq) * D, q_rsb,
              L - qb0, qln, wave);
  };
  // Load i of the 2 PER_WAVE loads of this wave for the Q and dO tiles of
  // step (g, t): the first PER_WAVE go to Q, the rest to dO.
  auto issue_one = [&](int g, int t, int stg, int i) {
    const int hq = hkv * G + g;
    const int qb0 = t * BQ;
    if (i < QT::PER_WAVE) {
      QT::issue_one(lds_offset(sQ[stg]), (const bf16*)a.q + (((long)b * L + qb0) * a.Hq + hq) * D, q_rsb,
                    L - qb0, qln, wave, i);
    } else {
      QT::issue_one(lds_offset(sO[stg]), (const bf16*)a.dout + (((long)b * L + qb0) * a.Hq + hq) * D, q_rsb,
                    L - qb0, qln, wave, i - QT::PER_WAVE);
    }
  };
  constexpr int NDMA = 2 * QT::PER_WAVE;

  f32x16 dkacc[NDB], dvacc[NDB];
#pragma unroll
  for (int i = 0; i < NDB; ++i) {
    dkacc[i] = dvacc[i] = f32x16{};
    // zeroed once, in the AGPRs the MFMAs accumulate into (a constant would be
    // rematerialised on the path that skips the step loop, and the two paths
    // then merged by copies between AGPRs after the loop)
    asm volatile("" : "+a"(dkacc[i]));
    asm volatile("" : "+a"(dvacc[i]));
  }

  // Stored dS: lane (key kw0 + l32, half hh) holds, for query block qb, the
  // queries 32 qb + 16 h + 8 hh + 0..7 in its dS operand hi[h] (h = 0, 1):
  // query chunk c = 4 qb + 2 h + hh of its key, which ds_chunk_offset places
  // so that each of the block's two stores writes 1 KB of whole lines.  The
  // stores are non-temporal: the 8.6 GB dS stream of the long-context
  // workload then no longer evicts from L2 the Q / dO tiles the XCD's other
  // workgroups read again.
  const DsBand band = ds_band(L, a.causal, a.window);
  const long ds_lane = (long)wave * 32 * DS_T + ds_chunk_offset(l32, hh) / 2;
  // the second half's slot of this lane, relative to the first half's
  const int ds_d1 = (ds_chunk_offset(l32, 2 + hh) - ds_chunk_offset(l32, hh)) / 2;
  // Every visited block lies inside the band of stored tiles (the band comes
  // from the same causal / window bounds that decide the visit), so the dS
  // stores are unconditional: the compiler then counts them exactly in its
  // vmcnt waits instead of assuming the worst over a branch.  (A slot outside
  // the band, which no visited block has, would be clamped to the band's
  // first tile, never written out of bounds.)
  auto ds_row = [&](int g, int t) -> bf16* {
    if (!WDS) return nullptr;
    long long slot = ds_slot(t, kt, band);
    if (slot < 0) slot = 0;
    const long long head = (long long)b * a.Hq + hkv * G + g;
    return (bf16*)a.ds + (head * a.ds_slots + slot) * DS_ELEMS + ds_lane;
  };
  auto store_ds = [&](bf16* row, int qb, const bf16x8 (&hi)[2]) {
    if (WDS) {
      __builtin_nontemporal_store(hi[0], (bf16x8*)(row + 1024 * qb));
      __builtin_nontemporal_store(hi[1], (bf16x8*)(row + 1024 * qb + ds_d1));
    }
  };

  // A step is (group head g, plan index p, entry e).  The step after (g, p):
  // the next entry, or the first one for the next group head; false past the
  // last head.  Branch-free, so that it runs beside the MFMAs of block 1.
  auto advance = [&](int g, int p, int& g2, int& p2, int& e2) -> bool {
    const bool wrap = p + 1 == nplan;
    p2 = wrap ? 0 : p + 1;
    g2 = wrap ? g + 1 : g;
    e2 = plan_entry(p2);
    return g2 < G;
  };
  int gc = 0, pc = 0, ec = 0, tc = -1;
  if (nplan > 0) {
    ec = plan_entry(0);
    tc = ec & 0xffff;
  }
  bool have = tc >= 0;
  // the next step; without one, the loads of the last step refetch its own
  // tile into the idle stage (branch-free loop body; once per work-group)
  int gn = gc, pn = pc, en = ec;
  bool more = have && advance(gc, pc, gn, pn, en);
  if (!more) {
    gn = gc;
    pn = pc;
    en = ec;
  }
  int tn = en & 0xffff;
  bf16* dsrow = have ? ds_row(gc, tc) : nullptr;
  if (have) {
    issue(gc, tc, 0);
    fetch_consts(gc, tc);
    store_consts(0);
  }
  wait_vmcnt<0>();
  __syncthreads();
  int stg = 0;
  while (have) {
    const int q0 = tc * BQ;
    // the step after the next and the next step's dS row, worked out during
    // block 1 (scalar work beside its MFMAs, ready when the next step starts)
    int g2 = gn, p2 = pn, e2 = en;
    bool more2 = false;
    bf16* dsrow_n = dsrow;
    const char* Qt = sQ[stg];
    const char* Ot = sO[stg];
    // the tile class is the same on every lane; readfirstlane lets the compiler
    // branch on it instead of running every variant under an exec mask
    const int tcls = (ec >> (16 + 2 * wave)) & 3;
    auto elementwise = [&](f32x16 (&sa)[1], f32x16 (&pa)[1], int qb) {
      const int o = 32 * qb;
      if (tcls == TILE_FULL) {
        dkv_elementwise<false, false, CAP>(sa, pa, a, sKf[stg] + o, sC2[stg] + o, sNrd[stg] + o,
                                           sR[stg] + o, km, q0 + o, hh, nullptr, 0);
      } else if (!seg_any) {
        dkv_elementwise<true, false, CAP>(sa, pa, a, sKf[stg] + o, sC2[stg] + o, sNrd[stg] + o,
                                          sR[stg] + o, km, q0 + o, hh, nullptr, 0);
      } else {
        dkv_elementwise<true, true, CAP>(sa, pa, a, sKf[stg] + o, sC2[stg] + o, sNrd[stg] + o,
                                         sR[stg] + o, km, q0 + o, hh, sSeg[stg] + o, seg_k);
      }
    };
    // bf16 operands of dV / dK for one block: P (pb) and dS (hi [+ lo]) per
    // 16-query half h
    auto pack = [&](const f32x16& sa, const f32x16& pa, bf16x8 (&pb)[2], bf16x8 (&hi)[2],
                    bf16x8 (&lo)[2]) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        pb[h] = Elem<bf16>::from_acc(sa, 8 * h);
        if (PRECISE) {
          Elem<bf16>::split_acc(pa, 8 * h, hi[h], lo[h]);
        } else {
          hi[h] = Elem<bf16>::from_acc(pa, 8 * h);
        }
      }
    };
    // dV / dK unit u = (h, db) of a block: 2 MFMAs (3 with PRECISE)
    auto dvdk_unit = [&](int u, const bf16x8 (&pb)[2], const bf16x8 (&hi)[2], const bf16x8 (&lo)[2],
                         const bf16x8& oa, const bf16x8& qa) {
      const int h = u / NDB, db = u % NDB;
      dvdk_mfma<PRECISE>(dvacc[db], dkacc[db], oa, pb[h], qa, hi[h], lo[h]);
    };
    auto tr_pair = [&](int qb, int u, bf16x8& oa, bf16x8& qa) {
      const int h = u / NDB, db = u % NDB, tt = 2 * qb + h;
      oa = QT::tr_frag(Ot, db, tt, lane);
      qa = QT::tr_frag(Qt, db, tt, lane);
    };
    constexpr int NU = 2 * NDB;   // dV / dK units per block
    static_assert(NU == NT16 || NU * 2 == NT16, "units per reduction step");
    static_assert(NQB >= 2, "the next step is worked out during block 1");
    constexpr int UPT = NU / NT16 > 0 ? NU / NT16 : 1;   // units per S/dP reduction step
    constexpr int TPU = NT16 / NU > 0 ? NT16 / NU : 1;   // reduction steps per unit
    // this step's tile loads, spread over the reduction steps of all blocks
    auto dma = [&](int qb, int t) {
      constexpr int NS = NQB * NT16;
#pragma unroll
      for (int i = (qb * NT16 + t) * NDMA / NS; i < (qb * NT16 + t + 1) * NDMA / NS; ++i)
        issue_one(gn, tn, stg ^ 1, i);
    };

    // Block 0: S / dP (two MFMA chains, LDS fragments one step ahead), then
    // its element work.
    f32x16 s0[1] = {f32x16{}}, p0[1] = {f32x16{}};
    {
      bf16x8 fq[2], fo[2];
      fq[0] = QT::row_frag(Qt, 0, 0, lane);
      fo[0] = QT::row_frag(Ot, 0, 0, lane);
#pragma unroll
      for (int t = 0; t < NT16; ++t) {
        const int cur = t & 1;
        if (t + 1 < NT16) {
          fq[cur ^ 1] = QT::row_frag(Qt, 0, t + 1, lane);
          fo[cur ^ 1] = QT::row_frag(Ot, 0, t + 1, lane);
        }
        s0[0] = Elem<bf16>::mfma(fq[cur], kf[t], s0[0]);
        p0[0] = Elem<bf16>::mfma(fo[cur], vf[t], p0[0]);
        if (t + 1 < NT16) __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
        __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);
        dma(0, t);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    fetch_consts(gn, tn);
    elementwise(s0, p0, 0);
    bf16x8 pbp[2], hip[2], lop[2];   // P and dS of the previous block
    pack(s0[0], p0[0], pbp, hip, lop);
    store_ds(dsrow, 0, hip);
    // Blocks 1 ..: each block's S / dP with the previous block's dV / dK
    // between them (~10 independent MFMA chains in flight; only one block's
    // S / dP accumulators live), then its element work.
#pragma unroll
    for (int qb = 1; qb < NQB; ++qb) {
      f32x16 s1[1] = {f32x16{}}, p1[1] = {f32x16{}};
      {
        bf16x8 fq[2], fo[2], ta[2], tb[2];
        fq[0] = QT::row_frag(Qt, qb, 0, lane);
        fo[0] = QT::row_frag(Ot, qb, 0, lane);
        tr_pair(qb - 1, 0, ta[0], tb[0]);
#pragma unroll
        for (int t = 0; t < NT16; ++t) {
          const int cur = t & 1;
          if (qb == 1 && t == 0) {
            // (also on the last step, where its result is not used)
            more2 = advance(gn, pn, g2, p2, e2) & more;
            dsrow_n = ds_row(gn, tn);
          }
          if (t + 1 < NT16) {
            fq[cur ^ 1] = QT::row_frag(Qt, qb, t + 1, lane);
            fo[cur ^ 1] = QT::row_frag(Ot, qb, t + 1, lane);
          }
          s1[0] = Elem<bf16>::mfma(fq[cur], kf[t], s1[0]);
          p1[0] = Elem<bf16>::mfma(fo[cur], vf[t], p1[0]);
          if (t % TPU == 0) {
#pragma unroll
            for (int k = 0; k < UPT; ++k) {
              const int u = (t / TPU) * UPT + k;
              const int c = u & 1;
              if (u + 1 < NU) tr_pair(qb - 1, u + 1, ta[c ^ 1], tb[c ^ 1]);
              dvdk_unit(u, pbp, hip, lop, ta[c], tb[c]);
            }
          }
          dma(qb, t);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      elementwise(s1, p1, qb);
      pack(s1[0], p1[0], pbp, hip, lop);
      store_ds(dsrow, qb, hip);
      // the next step's constants, two blocks after their loads were sent
      if (qb == 1 && more) store_consts(stg ^ 1);
    }
    // the last block's dV / dK
    {
      bf16x8 ta[2], tb[2];
      tr_pair(NQB - 1, 0, ta[0], tb[0]);
#pragma unroll
      for (int u = 0; u < NU; ++u) {
        const int c = u & 1;
        if (u + 1 < NU) tr_pair(NQB - 1, u + 1, ta[c ^ 1], tb[c ^ 1]);
        dvdk_unit(u, pbp, hip, lop, ta[c], tb[c]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    if (NQB < 2 && more) store_consts(stg ^ 1);
    // Vector memory operations complete in issue order, and the last block's
    // two dS stores are the only ones issued after this step's last tile
    // load: waiting down to two outstanding finds the next tiles in LDS
    // without waiting for those stores to reach L2.
    if (WDS)
      wait_vmcnt<2>();
    else
      wait_vmcnt<0>();
    __syncthreads();
    stg ^= 1;
    gc = gn;
    tc = tn;
    pc = pn;
    ec = en;
    dsrow = dsrow_n;
    have = more;
    more = more2;
    if (more) {
      gn = g2;
      pn = p2;
      en = e2;
    } else {
      gn = gc;
      pn = pc;
      en = ec;
    }
    tn = en & 0xffff;
  }

  dkv_acc_fence(dkacc, dvacc);
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

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
template <int D, bool P>
static void fwd_bf16_d(const KArgs& a, int cap, hipStream_t s) {
  dim3 grid(a.n_items), block(NTHREADS);
  switch (cap) {
    case 0: hipLaunchKernelGGL((fwd_bf16_kernel<D, 0, P>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((fwd_bf16_kernel<D, 1, P>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((fwd_bf16_kernel<D, 2, P>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((fwd_bf16_kernel<D, 3, P>), grid, block, 0, s, a); break;
  }
}

template <int D, bool P>
static void dq_bf16_d(const KArgs& a, int cap, hipStream_t s) {
  dim3 grid(a.n_items), block(NTHREADS);
  if (a.out3 != nullptr) {
    switch (cap) {
      case 0: hipLaunchKernelGGL((dq_bf16_kernel<D, 0, P, true>), grid, block, 0, s, a); break;
      case 1: hipLaunchKernelGGL((dq_bf16_kernel<D, 1, P, true>), grid, block, 0, s, a); break;
      case 2: hipLaunchKernelGGL((dq_bf16_kernel<D, 2, P, true>), grid, block, 0, s, a); break;
      default: hipLaunchKernelGGL((dq_bf16_kernel<D, 3, P, true>), grid, block, 0, s, a); break;
    }
    return;
  }
  switch (cap) {
    case 0: hipLaunchKernelGGL((dq_bf16_kernel<D, 0, P, false>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((dq_bf16_kernel<D, 1, P, false>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((dq_bf16_kernel<D, 2, P, false>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((dq_bf16_kernel<D, 3, P, false>), grid, block, 0, s, a); break;
  }
}

template <int D, bool P, bool W = false>
static void dkv_bf16_d(const KArgs& a, int cap, hipStream_t s) {
  dim3 grid(a.n_items), block(NTHREADS);
  switch (cap) {
    case 0: hipLaunchKernelGGL((dkv_bf16_kernel<D, 0, P, W>), grid, block, 0, s, a); break;
    case 1: hipLaunchKernelGGL((dkv_bf16_kernel<D, 1, P, W>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((dkv_bf16_kernel<D, 2, P, W>), grid, block, 0, s, a); break;
    default: hipLaunchKernelGGL((dkv_bf16_kernel<D, 3, P, W>), grid, block, 0, s, a); break;
  }
}

hipError_t launch_fwd_bf16(const KArgs& a, int head_dim, int cap, hipStream_t s) {
  const bool p = a.precise_ds != 0;
  if (head_dim == 64) p ? fwd_bf16_d<64, true>(a, cap, s) : fwd_bf16_d<64, false>(a, cap, s);
  else p ? fwd_bf16_d<128, true>(a, cap, s) : fwd_bf16_d<128, false>(a, cap, s);
  return hipGetLastError();
}

hipError_t launch_dq_bf16(const KArgs& a, int head_dim, int cap, hipStream_t s) {
  const bool p = a.precise_ds != 0;
  if (head_dim == 64) p ? dq_bf16_d<64, true>(a, cap, s) : dq_bf16_d<64, false>(a, cap, s);
  else p ? dq_bf16_d<128, true>(a, cap, s) : dq_bf16_d<128, false>(a, cap, s);
  return hipGetLastError();
}

hipError_t launch_dkv_bf16(const KArgs& a, int head_dim, int cap, hipStream_t s) {
  const bool p = a.precise_ds != 0;
  if (head_dim == 64) p ? dkv_bf16_d<64, true>(a, cap, s) : dkv_bf16_d<64, false>(a, cap, s);
  else p ? dkv_bf16_d<128, true>(a, cap, s) : dkv_bf16_d<128, false>(a, cap, s);
  return hipGetLastError();
}

hipError_t launch_dkv_ds_bf16(const KArgs& a, int head_dim, int cap, hipStream_t s) {
  if (head_dim == 64) dkv_bf16_d<64, false, true>(a, cap, s);
  else dkv_bf16_d<128, false, true>(a, cap, s);
  return hipGetLastError();
}

hipError_t launch_dq_ds_bf16(const KArgs& a, int head_dim, hipStream_t s) {
  // one work-group per pair of query tiles (a.n_items counts query tiles)
  KArgs c = a;
  c.n_items = a.B * a.Hq * ((a.n_q_tiles + 1) / 2);
  dim3 grid(c.n_items), block(DQS_THREADS);
  if (head_dim == 64) hipLaunchKernelGGL((dq_ds_bf16_kernel<64>), grid, block, 0, s, c);
  else hipLaunchKernelGGL((dq_ds_bf16_kernel<128>), grid, block, 0, s, c);
  return hipGetLastError();
}

}  // namespace attn
