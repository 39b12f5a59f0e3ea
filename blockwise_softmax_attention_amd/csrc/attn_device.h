// Device building blocks for the gfx950 attention kernels.
//
// MFMA shape: every contraction is a sequence of 32x32 output blocks with a
// 16-deep reduction step.  For bfloat16 one step is one
// v_mfma_f32_32x32x16_bf16; for float it is eight v_mfma_f32_32x32x2_f32 over
// the same per-lane fragment of 8 values, so both element types share every
// index computation below.
//
// Operand layout of a step (lane l of a 64-wide wave, h = l / 32):
//   A (32 x 16): lane l holds row l % 32, reduction indices 8h .. 8h+7
//   B (16 x 32): lane l holds column l % 32, reduction indices 8h .. 8h+7
//   C (32 x 32): lane l, register r holds column l % 32,
//                row 8 (r / 4) + 4 h + r % 4
// A and B use the same reduction-index convention, so any consistent
// permutation of the reduction index leaves the product unchanged.
//
// Orientation: the forward and dQ kernels compute S^T = K Q^T so that a lane
// owns one query (column) and its row statistics stay in-lane; the dK/dV
// kernel computes S = Q K^T so that a lane owns one key.  The C registers of
// a score block are then reused directly as the B operand of the next
// product (P^T for O^T = V^T P^T, dS^T for dQ^T = K^T dS^T, P and dS for
// dV^T = dO^T P and dK^T = Q^T dS) once the rows of the first product are
// loaded in the permuted order pi (bits 2 and 3 of the row index swapped):
// C register r of half h then holds row 16 (r / 8) + 8 h + r % 8, exactly the
// reduction index the B operand wants.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_internal.h"
#include "attn_tiles.h"

namespace attn {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float LOG2E_F = 1.4426950408889634f;
constexpr float LN2_F = 0.6931471805599453f;
#define ATTN_NEG_INF (-__builtin_huge_valf())
#define ATTN_POS_INF (__builtin_huge_valf())

// Row of the C block held in register r by lane half h, after pi.
__device__ __forceinline__ constexpr int prow(int r, int h) { return 16 * (r / 8) + 8 * h + (r % 8); }
// pi: swap bits 2 and 3 of a row index inside a 32-row block (an involution).
__device__ __forceinline__ constexpr int pi32(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

template <typename T> struct Elem;

template <> struct Elem<bf16> {
  using frag = bf16x8;
  static constexpr int CE = 8;  // elements per 16-byte chunk
  __device__ __forceinline__ static f32x16 mfma(const frag& a, const frag& b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ __forceinline__ static frag load(const bf16* p) { return *(const frag*)p; }
  __device__ __forceinline__ static frag zero() { return frag{}; }
  // Two floats rounded to bf16 (RNE) as one packed pair: one
  // v_cvt_pk_bf16_f32 (element-wise casts become one conversion per value
  // plus a v_perm_b32 per pair).
  __device__ __forceinline__ static uint32_t pack2(float a, float b) {
    typedef float f32x2 __attribute__((ext_vector_type(2)));
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
  }
  // Eight consecutive C registers starting at r0, rounded to bf16 (RNE).
  __device__ __forceinline__ static frag from_acc(const f32x16& c, int r0) {
    uint4 w;
    w.x = pack2(c[r0 + 0], c[r0 + 1]);
    w.y = pack2(c[r0 + 2], c[r0 + 3]);
    w.z = pack2(c[r0 + 4], c[r0 + 5]);
    w.w = pack2(c[r0 + 6], c[r0 + 7]);
    return __builtin_bit_cast(frag, w);
  }
  // hi + lo split: lo carries the rounding error of hi.
  __device__ __forceinline__ static void split_acc(const f32x16& c, int r0, frag& hi, frag& lo) {
    hi = from_acc(c, r0);
    f32x16 r;
#pragma unroll
    for (int i = 0; i < 8; ++i) r[r0 + i] = c[r0 + i] - (float)hi[i];
    lo = from_acc(r, r0);
  }
};

template <> struct Elem<float> {
  using frag = f32x8;
  static constexpr int CE = 4;
  __device__ __forceinline__ static f32x16 mfma(const frag& a, const frag& b, f32x16 c) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c = __builtin_amdgcn_mfma_f32_32x32x2f32(a[j], b[j], c, 0, 0, 0);
    return c;
  }
  __device__ __forceinline__ static frag load(const float* p) {
    f32x4 x = *(const f32x4*)p, y = *(const f32x4*)(p + 4);
    return frag{x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  }
  __device__ __forceinline__ static frag zero() { return frag{}; }
  __device__ __forceinline__ static frag from_acc(const f32x16& c, int r0) {
    frag f;
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = c[r0 + i];
    return f;
  }
  __device__ __forceinline__ static void split_acc(const f32x16& c, int r0, frag& hi, frag& lo) {
    hi = from_acc(c, r0);
    lo = frag{};
  }
};

// ---------------------------------------------------------------------------
// Workgroup -> work item.  Workgroups are dealt to the 8 XCDs round-robin
// (id % 8); this remap gives each XCD one contiguous run of work items, so
// items that share K/V (the query tiles and grouped heads of one KV head) run
// on the same XCD and hit its L2.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int xcd_remap(int bid, int n) {
  const int a = n / 8, r = n % 8, x = bid % 8, slot = bid / 8;
  return x * a + (x < r ? x : r) + slot;
}

// ---------------------------------------------------------------------------
// Logit cap in the log2 domain.  With per-row constants
//   Kf = kmul t,  C2 = kadd t - lse2,  R = rmul t,
// the capped, tempered logit in log2 units minus lse2 is fma(f(x), Kf, C2) for
// the raw dot product x = <q, k>, and the chain factor of the backward is
// temp cap'(sm_scale x) sm_scale = R g(aux).  The bfloat16 path uses the
// hardware exp2 / reciprocal (errors near 1 ulp, far below bf16 operand
// rounding); the float path uses libm formulations that avoid cancellation
// near zero.  Host-side constants per cap (attn_api.hip, make_args):
//   none            f = x                 kmul = sm log2e            kadd = 0
//   tanh, fast      f = 1/(1+e^{2y})      kmul = -2 cap log2e        kadd = cap log2e
//   tanh, float     f = tanh(y)           kmul = cap log2e           kadd = 0
//   soft-sign       f = x/(1+|x|sm/cap)   kmul = sm log2e            kadd = 0
//   alsc, fast      f = sig(z)            kmul = cap log2e / denom   kadd = -sig(ab) kmul
//   alsc, float     f = (sig(z)-sig(ab)) / (1-sig(ab))
//                                         kmul = cap log2e (1-sig(ab)) / denom, kadd = 0
// with y = sm x / cap and z = alpha (sm x / cap + beta).
// ---------------------------------------------------------------------------
struct RowC {
  float Kf;
  float C2;
  float R;
};

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_rcp(float x) { return __builtin_amdgcn_rcpf(x); }

__device__ __forceinline__ RowC row_consts(const KArgs& a, float t, float lse2) {
  RowC rc;
  rc.Kf = a.kmul * t;
  rc.C2 = a.kadd * t - lse2;
  rc.R = a.rmul * t;
  return rc;
}

template <int CAP, bool ACCURATE> struct Cap;

template <bool ACC> struct Cap<0, ACC> {   // none
  __device__ __forceinline__ static float f(float x, const KArgs&, float& aux) {
    aux = 0.f;
    return x;
  }
  __device__ __forceinline__ static float g(float, const KArgs&) { return 1.f; }
};

template <> struct Cap<1, false> {         // tanh(y) = 1 - 2 / (e^{2y} + 1)
  __device__ __forceinline__ static float f(float x, const KArgs& a, float& aux) {
    const float r = fast_rcp(1.f + fast_exp2(x * a.cx));
    aux = r;
    return r;
  }
  // 1 - tanh^2 = 4 r (1 - r); the 4 is in rmul.  r - r^2 in one fma (single rounding).
  __device__ __forceinline__ static float g(float r, const KArgs&) { return __builtin_fmaf(-r, r, r); }
};

template <> struct Cap<1, true> {
  __device__ __forceinline__ static float f(float x, const KArgs& a, float& aux) {
    const float th = tanhf(x * a.acc_inv_cap);
    aux = th;
    return th;
  }
  __device__ __forceinline__ static float g(float th, const KArgs&) { return 1.f - th * th; }
};

template <> struct Cap<2, false> {         // s / (1 + |s| / cap)
  __device__ __forceinline__ static float f(float x, const KArgs& a, float& aux) {
    const float r = fast_rcp(__builtin_fmaf(__builtin_fabsf(x), a.cx, 1.f));
    aux = r;
    return x * r;
  }
  __device__ __forceinline__ static float g(float r, const KArgs&) { return r * r; }
};

template <> struct Cap<2, true> {
  __device__ __forceinline__ static float f(float x, const KArgs& a, float& aux) {
    const float r = 1.f / (1.f + __builtin_fabsf(x) * a.acc_inv_cap);
    aux = r;
    return x * r;
  }
  __device__ __forceinline__ static float g(float r, const KArgs&) { return r * r; }
};

template <> struct Cap<3, false> {         // cap (sig(z) - sig(ab)) / denom
  __device__ __forceinline__ static float f(float x, const KArgs& a, float& aux) {
    const float r = fast_rcp(1.f + fast_exp2(__builtin_fmaf(x, a.cx, a.cb)));   // sig(z)
    aux = r;
    return r;
  }
  // sig(z)(1 - sig(z)) = r - r^2 in one fma; alpha / denom is in rmul
  __device__ __forceinline__ static float g(float r, const KArgs&) { return __builtin_fmaf(-r, r, r); }
};

template <> struct Cap<3, true> {
  // (sig(z) - sig(c)) / (1 - sig(c)) with z = u + c, c = alpha beta, A = e^{-c}:
  //   u >= 0 : -expm1(-u) / (1 + A e^{-u})
  //   u <  0 :  expm1(u) / (e^{u} + A)
  // (no overflow, no cancellation near u = 0).
  __device__ __forceinline__ static float f(float x, const KArgs& a, float& aux) {
    const float u = x * a.acc_u;
    aux = u;
    if (u >= 0.f) return -expm1f(-u) / (1.f + a.acc_a * expf(-u));
    return expm1f(u) / (expf(u) + a.acc_a);
  }
  // sig(z)(1 - sig(z)) = e^{-|z|} / (1 + e^{-|z|})^2
  __device__ __forceinline__ static float g(float u, const KArgs& a) {
    const float e = expf(-__builtin_fabsf(u + a.acc_alpha_beta));
    const float d = 1.f + e;
    return e / (d * d);
  }
};

// ---------------------------------------------------------------------------
// LDS tiles.  A streamed tile of ROWS rows x D columns is loaded from global
// memory as "tasks" of 4 consecutive rows x one 16-byte column chunk (lanes
// walk the chunks of a row first, so each row is read contiguously) and
// stored in one or both of:
//   * row-major, rows in pi order, stride D + 16 bytes (A operand with the
//     reduction over D);
//   * transposed [D][ROWS], 4-element units XOR-swizzled by the row d so that
//     both the transposing stores and the 16-byte fragment reads spread over
//     the banks (A operand with the reduction over the tile rows).
// ---------------------------------------------------------------------------
template <typename T, int ROWS, int D, int NT>
struct TileIO {
  static constexpr int CE = 16 / (int)sizeof(T);
  static constexpr int CPR = D / CE;               // 16-byte chunks per row
  static constexpr int NTASK = (ROWS / 4) * CPR;
  static constexpr int NPER = (NTASK + NT - 1) / NT;
  static constexpr int RS = D + CE;                // row-major stride (elements)
  static constexpr int NPAIR = ROWS / 8;           // 8-element pairs per transposed row
  static constexpr int ROW_ELEMS = ROWS * RS;
  static constexpr int T_ELEMS = D * ROWS;
  static_assert(ROWS % 32 == 0, "tile rows must be a multiple of 32");
  static_assert(NPAIR >= 2 && (NPAIR & (NPAIR - 1)) == 0, "pairs per row must be a power of 2");

  uint4 r[NPER][4];

  // base: element (row 0, col 0) of the tile; rows >= rows_valid read as 0.
  __device__ __forceinline__ void load(const T* base, long row_stride, int rows_valid, int tid) {
#pragma unroll
    for (int u = 0; u < NPER; ++u) {
      const int task = tid + u * NT;
      const int dc = task % CPR, kq = task / CPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * kq + i;
        if (task < NTASK && row < rows_valid) {
          r[u][i] = *(const uint4*)(base + (long)row * row_stride + dc * CE);
        } else {
          r[u][i] = make_uint4(0, 0, 0, 0);
        }
      }
    }
  }

  __device__ __forceinline__ void store_rows(T* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < NPER; ++u) {
      const int task = tid + u * NT;
      if (NTASK % NT != 0 && task >= NTASK) continue;
      const int dc = task % CPR, kq = task / CPR;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = 4 * kq + i;
        const int lrow = (row & ~31) | pi32(row & 31);
        *(uint4*)(lds + lrow * RS + dc * CE) = r[u][i];
      }
    }
  }

  // Swizzled position (in elements) of the 4-element unit `unit` of row d.
  __device__ __forceinline__ static int t_offset(int d, int unit) {
    const int f = 2 * ((d ^ (d / NPAIR)) & (NPAIR - 1));
    return d * ROWS + ((unit ^ f) << 2);
  }

  __device__ __forceinline__ void store_T(T* lds, int tid) const {
#pragma unroll
    for (int u = 0; u < NPER; ++u) {
      const int task = tid + u * NT;
      if (NTASK % NT != 0 && task >= NTASK) continue;
      const int dc = task % CPR, kq = task / CPR;
      if constexpr (sizeof(T) == 2) {
        // 8 columns x 4 rows of 16-bit values -> per column, 4 rows = 8 bytes
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const int w = e >> 1;
          uint32_t a0 = ((const uint32_t*)&r[u][0])[w], a1 = ((const uint32_t*)&r[u][1])[w];
          uint32_t a2 = ((const uint32_t*)&r[u][2])[w], a3 = ((const uint32_t*)&r[u][3])[w];
          uint2 o;
          if (e & 1) {
            o.x = (a0 >> 16) | (a1 & 0xffff0000u);
            o.y = (a2 >> 16) | (a3 & 0xffff0000u);
          } else {
            o.x = (a0 & 0xffffu) | (a1 << 16);
            o.y = (a2 & 0xffffu) | (a3 << 16);
          }
          const int d = dc * 8 + e;
          *(uint2*)(lds + t_offset(d, kq)) = o;
        }
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint4 o;
          o.x = ((const uint32_t*)&r[u][0])[e];
          o.y = ((const uint32_t*)&r[u][1])[e];
          o.z = ((const uint32_t*)&r[u][2])[e];
          o.w = ((const uint32_t*)&r[u][3])[e];
          const int d = dc * 4 + e;
          *(uint4*)(lds + t_offset(d, kq)) = o;
        }
      }
    }
  }

  // A-operand fragment, reduction over D: 32-row block `blk`, step t.
  __device__ __forceinline__ static typename Elem<T>::frag row_frag(const T* lds, int blk, int t,
                                                                  int lane) {
    return Elem<T>::load(lds + (blk * 32 + (lane & 31)) * RS + 16 * t + 8 * (lane >> 5));
  }
  // A-operand fragment, reduction over the tile rows: d block `blk`, step t.
  __device__ __forceinline__ static typename Elem<T>::frag t_frag(const T* lds, int blk, int t,
                                                                int lane) {
    const int d = blk * 32 + (lane & 31);
    const int unit = 4 * t + 2 * (lane >> 5);
    return Elem<T>::load(lds + t_offset(d, unit));
  }
};

// Global fragment of one row: 8 consecutive elements starting at p (or zero).
template <typename T>
__device__ __forceinline__ typename Elem<T>::frag global_frag(const T* p, bool valid) {
  return valid ? Elem<T>::load(p) : Elem<T>::zero();
}

__device__ __forceinline__ float wave_half_swap(float x) { return __shfl_xor(x, 32); }

}  // namespace attn
