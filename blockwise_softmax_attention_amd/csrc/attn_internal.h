// Host/device shared definitions: kernel argument block, tile sizes, launchers.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace attn {

// Tile geometry.  A workgroup of 4 waves (256 threads) owns BM_FWD query rows
// (32 per wave) in the forward and dQ kernels, and 32 * DKV_WAVES keys in the
// dK/dV kernel; key tiles (forward, dQ) and query tiles (dK/dV) stream through
// LDS in steps of BN rows.
constexpr int NWAVES = 4;
constexpr int NTHREADS = 64 * NWAVES;
constexpr int BM = 32 * NWAVES;          // query rows per forward / dQ workgroup
constexpr int BKV = 32 * NWAVES;         // key rows per dK/dV workgroup
constexpr int MAX_TILES = 4096;          // segment-skip flags per workgroup (key or query tiles)

// Kernel argument block (passed by value).
struct KArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* temp;       // (B, L) or null
  const int32_t* seg;      // (B, L) or null
  const int32_t* bounds;   // (B, 4) or null
  const float* o_in;       // preprocess: O
  const float* m_in;       // backward: m, l, delta (B, Hq, L)
  const float* l_in;
  const float* delta_in;
  float* out0;             // fwd: O      dq: dQ    dkv: dK   pre: delta
  float* out1;             // fwd: m                dkv: dV
  float* out2;             // fwd: l
  float* out3;             // dq: this head's share of the temperature gradient (B, Hq, L), or null
  int B, L, Hq, Hkv, G;
  int causal, window;
  float sm_scale;
  float zw;                // z-loss weight
  // Cap constants.  For a raw dot product x = <q, k> and a row with
  // temperature t, the log2-domain logit minus the row's log2 LSE is
  //   fma(f(x), kmul * t, kadd * t - lse2)
  // where f depends on the cap (see Cap<> in attn_device.h), and
  //   cap'(sm_scale x) * sm_scale * t = rmul * t * g(x).
  float kmul, kadd, rmul;
  float cx;                // coefficient of x inside exp2 / the soft-sign denominator
  float cb;                // additive exponent term (alsc)
  float acc_a;             // float path, alsc: exp(-alpha beta)
  float acc_inv_cap;       // float path: sm_scale / cap
  float acc_alpha_beta;    // float path, alsc: alpha * beta
  float acc_u;             // float path, alsc: alpha * sm_scale / cap
  int precise_ds;
  int n_items;             // workgroups doing real work
  int n_q_tiles;           // ceil(L / BM)
  int n_kv_tiles;          // ceil(L / BKV)
  // Stored-dS backward: bf16 dS tiles (see DS_T in attn_tiles.h), written by
  // the dK/dV kernel and read by the dQ kernel of that path.
  void* ds;
  long long ds_slots;      // tiles per (batch row, query head)
};

// Launchers (one per kernel family); dtype 0 = f32, 1 = bf16; cap 0..3.
hipError_t launch_fwd(const KArgs& a, int dtype, int head_dim, int cap, hipStream_t s);
hipError_t launch_preprocess(const KArgs& a, int dtype, int head_dim, hipStream_t s);
hipError_t launch_dq(const KArgs& a, int dtype, int head_dim, int cap, hipStream_t s);
hipError_t launch_dkv(const KArgs& a, int dtype, int head_dim, int cap, hipStream_t s);
hipError_t launch_reduce_heads(const float* x, float* out, int B, int H, int L, hipStream_t s);
hipError_t launch_stream_probe(const void* src, long long bytes, int blocks, float* out, hipStream_t s);
hipError_t launch_ranker_bounds(const int32_t* seg, int32_t* bounds, int B, int L, int32_t hist_id,
                                int32_t cand_id, hipStream_t s);
int fwd_key_tile(int dtype, int head_dim);   // keys per forward tile
// bfloat16 kernels (attn_bf16.hip)
hipError_t launch_fwd_bf16(const KArgs& a, int head_dim, int cap, hipStream_t s);
hipError_t launch_dq_bf16(const KArgs& a, int head_dim, int cap, hipStream_t s);
hipError_t launch_dkv_bf16(const KArgs& a, int head_dim, int cap, hipStream_t s);
// stored-dS backward (bf16, single-bf16 dS): dK/dV that also writes a.ds, and
// dQ = dS K from it
hipError_t launch_dkv_ds_bf16(const KArgs& a, int head_dim, int cap, hipStream_t s);
hipError_t launch_dq_ds_bf16(const KArgs& a, int head_dim, hipStream_t s);

}  // namespace attn
