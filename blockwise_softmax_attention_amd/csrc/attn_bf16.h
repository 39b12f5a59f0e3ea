// bfloat16 building blocks for gfx950: direct global->LDS tile loads,
// swizzled LDS tiles read both row-wise and transposed, lane mask contexts.
//
// Tile layout.  A tile of ROWS rows x D bf16 columns occupies ROWS * 2D bytes
// of LDS with no padding.  LDS row lr holds the tile's row pi(lr) (bits 2 and 3
// swapped inside each 32-row block, see attn_device.h), and its 16-byte chunk c
// sits at position c ^ swz(lr), where the bits of swz(lr) (mod D / 8) are
//   bit 0 = lr2,  bit 1 = lr0,  bit 2 = lr1,  bit 3 = lr0 ^ lr3.
// With 256-byte rows (D = 128) both access patterns then hit distinct banks,
// whether the LDS serves 128 or 256 bytes per clock (32 or 64 banks):
//   * row fragments (A operand, reduction over D): 16 consecutive LDS rows,
//     one chunk each -> 16 distinct chunk positions (bits 0-3 of swz are a
//     bijection of lr bits 0-3);
//   * transposed fragments (ds_read_b64_tr_b16, reduction over the tile rows):
//     32 lanes read 4 consecutive rows x 4 adjacent chunks (an aligned group,
//     differing in chunk bits 0-1) -> 16 distinct positions, because as lr
//     bits 0-1 run over the 4 rows, swz bits 2-3 (and, for 16 lanes, bits 1-2)
//     take 4 distinct values.
// (The previous form 2 (lr & 3) + ((lr >> 2) & 1) + 8 ((lr >> 3) & 1) left
// the transposed reads two-way conflicted on 64 banks: only swz bit 2 varied
// with lr bits 0-1.)
//
// Loads.  global_load_lds_dwordx4 writes lane l's 16 bytes to LDS address
// M0 + 16 l, so each instruction fills 1 KB of LDS; the lane -> (row, chunk)
// choice realises the layout above.  The instruction is issued from inline
// assembly so that the compiler does not force a full vmcnt wait before every
// LDS read; the kernels wait for their own loads explicitly (wait_vmcnt)
// before the workgroup barrier that publishes a stage.  Rows past the end of
// the sequence are clamped to the last row (finite data that the masks zero).
//
// Transposed reads (ds_read_b64_tr_b16).  In each group of 16 lanes, lane
// 4e + s supplies the address of 4 consecutive bf16 of LDS row r0 + e,
// columns c0 + 4s .. c0 + 4s + 3; lane i of the group then receives column
// c0 + i of rows r0 .. r0 + 3.  Two such reads give the 8 reduction elements
// of an MFMA A-operand fragment.
#pragma once

#include "attn_device.h"

namespace attn {

__device__ __forceinline__ uint32_t imin_u(uint32_t a, uint32_t b) { return a < b ? a : b; }

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)p;
}

// One 16-byte direct load per lane into LDS[m0 + 16 * lane] from the address
// sbase + voff: sbase wave-uniform (scalar registers), voff a per-lane 32-bit
// byte offset, so the address costs no 64-bit vector arithmetic; m0 uniform.
__device__ __forceinline__ void dma16(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}
// The same load marked non-temporal (nt): for data read once, so that it does
// not evict lines that other workgroups of the XCD read again from L2.
__device__ __forceinline__ void dma16_nt(const void* sbase, uint32_t voff, uint32_t m0) {
  asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1 nt" ::"v"(voff), "s"(sbase), "s"(m0)
               : "memory", "m0");
}

// A pointer the caller knows to be the same on every lane, moved to scalar
// registers.
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t u = (uint64_t)(uintptr_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)u);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(u >> 32));
  return (const void*)(uintptr_t)(((uint64_t)hi << 32) | lo);
}

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Sum and max across the two 32-lane halves of a wave: permlane32_swap(x, x)
// returns {own, other} (in some order) on every lane.
__device__ __forceinline__ float half_max(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// LAUNDER: pass the lane index through an empty asm before each fragment
// address so that the swizzled addresses are recomputed where they are used
// instead of being hoisted out of the tile loop (where they would hold dozens
// of registers); kernels short of registers set it, the others do not.
template <int ROWS, int D, int NW, bool LAUNDER = false>
struct BTile {
  static constexpr int RB = 2 * D;            // bytes per row
  static constexpr int CPR = D / 8;           // 16-byte chunks per row
  static constexpr int BYTES = ROWS * RB;
  static constexpr int NINST = BYTES / 1024;  // 1 KB loads per tile
  static constexpr int PER_WAVE = NINST / NW;
  static_assert(ROWS % 32 == 0, "tile rows must be a multiple of 32");
  static_assert(NINST % NW == 0, "tile must split evenly over the waves");

  __device__ __forceinline__ static int swz(int lr) {
    return (((lr >> 2) & 1) | ((lr & 1) << 1) | (((lr >> 1) & 1) << 2) | (((lr ^ (lr >> 3)) & 1) << 3)) &
           (CPR - 1);
  }

  // Per-lane part of every load address, computed once: load n = wave + NW i
  // fills LDS rows 4n .. 4n+3 (for 256-byte rows); with that interleaving a
  // lane's row inside each group of RPI*NW rows and its chunk are the same for
  // all of its loads, so its byte offset is off0 plus a uniform i * step.
  struct Lane {
    uint32_t off0;    // byte offset of this lane's 16 bytes in load 0
    uint32_t cbyte;   // byte offset of its chunk inside a row
  };
  static constexpr int LPR = RB / 16;              // lanes per row in one load
  static constexpr int RPI = 64 / LPR;             // rows per load
  static_assert(RPI * NW <= 32 && 32 % (RPI * NW) == 0, "load pattern must tile 32-row blocks");

  // rsb: global row stride in bytes.
  __device__ __forceinline__ static Lane lane_of(uint32_t rsb, int lane, int wave) {
    const int x = wave * RPI + lane / LPR;         // LDS row inside the group of RPI*NW rows
    const int c = (lane % LPR) ^ swz(x);
    Lane l;
    l.cbyte = (uint32_t)c * 16u;
    l.off0 = (uint32_t)pi32(x) * rsb + l.cbyte;    // pi keeps groups of 16 rows
    return l;
  }

  // Load i (0 <= i < PER_WAVE) of this wave's share of one tile.  gbase:
  // element (0, 0) of the tile (wave-uniform); rows >= rows_valid read row
  // rows_valid - 1 (finite data the masks zero; only the last tile of a
  // sequence has such rows).
  template <bool NT = false>
  __device__ __forceinline__ static void issue_one(uint32_t lds_base, const bf16* gbase, uint32_t rsb,
                                                   int rows_valid, const Lane& ln, int wave, int i) {
    const int n = wave + NW * i;
    const uint32_t lim = (uint32_t)(rows_valid - 1) * rsb + ln.cbyte;
    const uint32_t off = imin_u(ln.off0 + (uint32_t)(i * RPI * NW) * rsb, lim);
    const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane(lds_base + n * 1024);
    if (NT) {
      dma16_nt(uniform_ptr(gbase), off, m0);
    } else {
      dma16(uniform_ptr(gbase), off, m0);
    }
  }

  // All of this wave's loads of one tile.
  __device__ __forceinline__ static void issue(uint32_t lds_base, const bf16* gbase, uint32_t rsb,
                                               int rows_valid, const Lane& ln, int wave) {
#pragma unroll
    for (int i = 0; i < PER_WAVE; ++i) issue_one(lds_base, gbase, rsb, rows_valid, ln, wave, i);
  }

  // A operand, reduction over D: rows blk*32 + lane%32 (LDS order), step t.
  __device__ __forceinline__ static bf16x8 row_frag(const char* lds, int blk, int t, int lane) {
    if (LAUNDER) asm volatile("" : "+v"(lane));
    const int lr = blk * 32 + (lane & 31);
    const int c = 2 * t + (lane >> 5);
    return *(const bf16x8*)(lds + lr * RB + ((c ^ swz(lr)) << 4));
  }

  // A operand, reduction over the tile rows: columns blk*32 + lane%32, step t
  // (rows 16t .. 16t+15 in the product's order).
  __device__ __forceinline__ static bf16x8 tr_frag(const char* lds, int blk, int t, int lane) {
    if (LAUNDER) asm volatile("" : "+v"(lane));
    const int h = lane >> 5, mh = (lane >> 4) & 1, e = (lane & 15) >> 2, s = lane & 3;
    const int chunk = 4 * blk + 2 * mh + (s >> 1);
    const int r1 = 16 * t + 4 * h + e, r2 = r1 + 8;
    const char* a1 = lds + r1 * RB + ((chunk ^ swz(r1)) << 4) + ((s & 1) << 3);
    const char* a2 = lds + r2 * RB + ((chunk ^ swz(r2)) << 4) + ((s & 1) << 3);
    const s16x4 v1 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a1);
    const s16x4 v2 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)a2);
    typedef short s16x8 __attribute__((ext_vector_type(8)));
    const s16x8 v = {v1[0], v1[1], v1[2], v1[3], v2[0], v2[1], v2[2], v2[3]};
    return __builtin_bit_cast(bf16x8, v);
  }
};

// Visible keys of one query row (lane = query): [lo, hi] plus the single key dg.
struct QMask {
  int lo, hi, dg;
};

__device__ __forceinline__ QMask query_mask(int q, const MaskSpec& s) {
  QMask m;
  m.lo = 0;
  m.hi = s.L - 1;
  m.dg = -1;
  if (s.causal) m.hi = imin(m.hi, q);
  if (s.window > 0) m.lo = imax(m.lo, q - s.window + 1);
  if (s.ranker) {
    const bool qh = q >= s.hl && q < s.hu, qc = q >= s.cl && q < s.cu;
    if (qh || qc) {
      m.lo = imax(m.lo, s.hl);
      m.hi = imin(m.hi, s.hu - 1);
    } else {
      m.lo = 1;
      m.hi = 0;
    }
    if (qc) m.dg = q;   // itself: always inside the causal / window range
  }
  if (q >= s.L) {
    m.lo = 1;
    m.hi = 0;
    m.dg = -1;
  }
  return m;
}

__device__ __forceinline__ bool qmask_vis(const QMask& m, int k) {
  return (k >= m.lo && k <= m.hi) || k == m.dg;
}

// Visible queries of one key (lane = key): [a0, a1] or [b0, b1] or the query dg.
struct KMask {
  int a0, a1, b0, b1, dg;
};

__device__ __forceinline__ KMask key_mask(int k, const MaskSpec& s) {
  KMask m;
  int lo = 0, hi = s.L - 1;
  if (s.causal) lo = imax(lo, k);
  if (s.window > 0) hi = imin(hi, k + s.window - 1);
  m.a0 = lo;
  m.a1 = hi;
  m.b0 = 1;
  m.b1 = 0;
  m.dg = -1;
  if (s.ranker) {
    const bool kh = k >= s.hl && k < s.hu, kc = k >= s.cl && k < s.cu;
    if (kh) {   // rows of the history or the candidates
      m.a0 = imax(lo, s.hl);
      m.a1 = imin(hi, s.hu - 1);
      m.b0 = imax(lo, s.cl);
      m.b1 = imin(hi, s.cu - 1);
    } else {
      m.a0 = 1;
      m.a1 = 0;
    }
    if (kc) m.dg = k;   // a candidate key is seen by itself
  }
  if (k >= s.L) {
    m.a0 = m.b0 = 1;
    m.a1 = m.b1 = 0;
    m.dg = -1;
  }
  return m;
}

__device__ __forceinline__ bool kmask_vis(const KMask& m, int q) {
  return (q >= m.a0 && q <= m.a1) || (q >= m.b0 && q <= m.b1) || q == m.dg;
}

__device__ __forceinline__ MaskSpec load_mask_spec(const KArgs& a, int b) {
  MaskSpec ms;
  ms.L = a.L;
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
  ms.has_seg = a.seg != nullptr;
  return ms;
}

}  // namespace attn
