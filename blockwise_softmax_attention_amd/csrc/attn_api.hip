// C ABI: validation, cap constants, launches, and the host planner.
#include <math.h>
#include <stdio.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <unordered_map>
#include <vector>

#include "../../include/attn.h"
#include "attn_internal.h"
#include "attn_tiles.h"

namespace {

thread_local std::string g_last_error;

attn_status fail(attn_status s, const std::string& msg) {
  g_last_error = msg;
  return s;
}

bool finite(float x) { return std::isfinite(x); }

attn_status check_params(const attn_params* p) {
  if (p == nullptr) return fail(ATTN_ERR_NULL_PTR, "params is NULL");
  if (p->batch < 1 || p->seq_len < 1 || p->q_heads < 1 || p->kv_heads < 1)
    return fail(ATTN_ERR_SHAPE, "batch, seq_len, q_heads and kv_heads must be >= 1");
  if (p->seq_len > ATTN_MAX_SEQ_LEN)
    return fail(ATTN_ERR_SHAPE, "seq_len exceeds ATTN_MAX_SEQ_LEN");
  if ((long long)p->batch * p->q_heads * p->seq_len > (1LL << 36))
    return fail(ATTN_ERR_SHAPE, "batch * q_heads * seq_len too large");
  // tile loads address a tile as base + 32-bit byte offset (rows * Hq * D * 2)
  if ((long long)p->q_heads * p->head_dim > (1LL << 22))
    return fail(ATTN_ERR_SHAPE, "q_heads * head_dim exceeds 2^22");
  if (p->dtype != ATTN_F32 && p->dtype != ATTN_BF16)
    return fail(ATTN_ERR_DTYPE, "dtype must be ATTN_F32 or ATTN_BF16");
  if (p->head_dim != 64 && p->head_dim != 128)
    return fail(ATTN_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (p->q_heads % p->kv_heads != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "q_heads must be a multiple of kv_heads");
  if (p->cap_method < ATTN_CAP_NONE || p->cap_method > ATTN_CAP_ALSC)
    return fail(ATTN_ERR_PARAM, "unknown cap_method");
  if (!finite(p->sm_scale) || p->sm_scale <= 0.f) return fail(ATTN_ERR_PARAM, "sm_scale must be > 0");
  if (p->window_len < 0) return fail(ATTN_ERR_PARAM, "window_len must be >= 0");
  if (!finite(p->z_loss_weight) || p->z_loss_weight < 0.f)
    return fail(ATTN_ERR_PARAM, "z_loss_weight must be finite and >= 0");
  if (!finite(p->cap) || !finite(p->alpha) || !finite(p->beta))
    return fail(ATTN_ERR_PARAM, "cap, alpha and beta must be finite");
  return ATTN_OK;
}

attn_status check_ptr(const void* ptr, const char* name, size_t align) {
  if (ptr == nullptr) return fail(ATTN_ERR_NULL_PTR, std::string(name) + " is NULL");
  if (((uintptr_t)ptr) % align != 0)
    return fail(ATTN_ERR_ALIGN, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
  return ATTN_OK;
}

attn_status check_opt(const void* ptr, const char* name) {
  if (ptr != nullptr && ((uintptr_t)ptr) % 4 != 0)
    return fail(ATTN_ERR_ALIGN, std::string(name) + " is not 4-byte aligned");
  return ATTN_OK;
}

#define ATTN_TRY(expr)              \
  do {                              \
    attn_status _s = (expr);        \
    if (_s != ATTN_OK) return _s;   \
  } while (0)

int effective_cap(const attn_params* p) {
  return (p->cap_method == ATTN_CAP_NONE || p->cap <= 0.f) ? ATTN_CAP_NONE : p->cap_method;
}

// Kernel arguments common to every call: sizes, masks and cap constants
// (the fma form of attn_device.h: logit2 - lse2 = fma(f(x), kmul t, kadd t - lse2)).
attn::KArgs make_args(const attn_params* p, const float* temp, const int32_t* seg,
                      const int32_t* bounds) {
  attn::KArgs a;
  memset(&a, 0, sizeof(a));
  a.temp = temp;
  a.seg = seg;
  a.bounds = bounds;
  a.B = p->batch;
  a.L = p->seq_len;
  a.Hq = p->q_heads;
  a.Hkv = p->kv_heads;
  a.G = p->q_heads / p->kv_heads;
  a.causal = p->causal != 0;
  a.window = p->window_len;
  a.sm_scale = p->sm_scale;
  a.zw = p->z_loss_weight;
  a.precise_ds = p->precise_ds != 0;
  const bool acc = p->dtype == ATTN_F32;
  const double log2e = 1.4426950408889634;
  const double sm = p->sm_scale, cap = p->cap, al = p->alpha, be = p->beta;
  switch (effective_cap(p)) {
    case ATTN_CAP_NONE:
      a.kmul = (float)(sm * log2e);
      a.kadd = 0.f;
      a.rmul = (float)sm;
      break;
    case ATTN_CAP_TANH:
      a.acc_inv_cap = (float)(sm / cap);
      if (acc) {
        a.kmul = (float)(cap * log2e);
        a.kadd = 0.f;
        a.rmul = (float)sm;
      } else {
        a.cx = (float)(2.0 * sm * log2e / cap);
        a.kmul = (float)(-2.0 * cap * log2e);
        a.kadd = (float)(cap * log2e);
        a.rmul = (float)(4.0 * sm);
      }
      break;
    case ATTN_CAP_SOFT_SIGN:
      a.cx = (float)(sm / cap);
      a.acc_inv_cap = (float)(sm / cap);
      a.kmul = (float)(sm * log2e);
      a.kadd = 0.f;
      a.rmul = (float)sm;
      break;
    default: {  // ALSC
      const double ab = al * be;
      const double e = exp(-ab);
      const double sb = 1.0 / (1.0 + e);          // sig(alpha beta)
      const double one_m_sb = e / (1.0 + e);      // 1 - sig(alpha beta), no cancellation
      const double denom = sb * one_m_sb + 1e-12;
      a.rmul = (float)(al * sm / denom);
      if (acc) {
        a.kmul = (float)(cap * log2e * one_m_sb / denom);
        a.kadd = 0.f;
        a.acc_u = (float)(al * sm / cap);
        a.acc_a = (float)e;
        a.acc_alpha_beta = (float)ab;
      } else {
        const double km = cap * log2e / denom;
        a.kmul = (float)km;
        a.kadd = (float)(-sb * km);
        a.cx = (float)(-al * sm * log2e / cap);
        a.cb = (float)(-ab * log2e);
      }
      break;
    }
  }
  a.n_q_tiles = (a.L + attn::BM - 1) / attn::BM;
  a.n_kv_tiles = (a.L + attn::BKV - 1) / attn::BKV;
  return a;
}

attn_status check_common(const attn_params* p, const float* temp, const int32_t* seg,
                         const int32_t* bounds) {
  ATTN_TRY(check_params(p));
  ATTN_TRY(check_opt(temp, "temperature"));
  ATTN_TRY(check_opt(seg, "segment_ids"));
  ATTN_TRY(check_opt(bounds, "ranker_bounds"));
  if (seg != nullptr && p->seq_len > ATTN_MAX_SEQ_LEN_SEGMENTS)
    return fail(ATTN_ERR_UNSUPPORTED, "seq_len exceeds ATTN_MAX_SEQ_LEN_SEGMENTS with segment ids");
  return ATTN_OK;
}

attn_status hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess)
    return fail(ATTN_ERR_HIP, std::string(what) + ": " + hipGetErrorString(e));
  return ATTN_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// Allocation-free stored-dS backward: the dS workspace is this fixed device
// array.  Host code never passes `scratch` itself to a kernel (on the host
// it names a stand-in, not device memory): the device address comes from
// hipGetSymbolAddress, once per device, and only that address is used.
// ---------------------------------------------------------------------------
static __device__ __align__(256) unsigned char scratch[ATTN_STATIC_DS_BYTES];

namespace {
constexpr int MAX_DEVICES = 64;
std::mutex g_scratch_mu;
void* g_scratch[MAX_DEVICES] = {};

// Device address of `scratch` on the current device (looked up on the first
// call with that device current, then kept).
attn_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return fail(ATTN_ERR_HIP, std::string("hipGetDevice: ") + hipGetErrorString(e));
  if (dev < 0 || dev >= MAX_DEVICES)
    return fail(ATTN_ERR_HIP, "device index " + std::to_string(dev) + " out of range");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch[dev] == nullptr) {
    void* ptr = nullptr;
    e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    if (e != hipSuccess || ptr == nullptr)
      return fail(ATTN_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}
}  // namespace

extern "C" {

attn_status attn_check_params(const attn_params* params) { return check_params(params); }

attn_status attn_fwd(const attn_params* p, const void* q, const void* k, const void* v,
                     const float* temperature, const int32_t* segment_ids,
                     const int32_t* ranker_bounds, float* o, float* m, float* l, void* stream) {
  ATTN_TRY(check_common(p, temperature, segment_ids, ranker_bounds));
  ATTN_TRY(check_ptr(q, "q", 16));
  ATTN_TRY(check_ptr(k, "k", 16));
  ATTN_TRY(check_ptr(v, "v", 16));
  ATTN_TRY(check_ptr(o, "o", 16));
  ATTN_TRY(check_ptr(m, "m", 4));
  ATTN_TRY(check_ptr(l, "l", 4));
  attn::KArgs a = make_args(p, temperature, segment_ids, ranker_bounds);
  a.q = q;
  a.k = k;
  a.v = v;
  a.out0 = o;
  a.out1 = m;
  a.out2 = l;
  a.n_items = a.B * a.Hq * a.n_q_tiles;
  return hip_status(attn::launch_fwd(a, p->dtype, p->head_dim, effective_cap(p), (hipStream_t)stream),
                    "attn_fwd launch");
}

attn_status attn_bwd_preprocess(const attn_params* p, const float* o, const void* d_o,
                                float* delta, void* stream) {
  ATTN_TRY(check_params(p));
  ATTN_TRY(check_ptr(o, "o", 16));
  ATTN_TRY(check_ptr(d_o, "d_o", 16));
  ATTN_TRY(check_ptr(delta, "delta", 4));
  attn::KArgs a = make_args(p, nullptr, nullptr, nullptr);
  a.o_in = o;
  a.dout = d_o;
  a.out0 = delta;
  return hip_status(attn::launch_preprocess(a, p->dtype, p->head_dim, (hipStream_t)stream),
                    "attn_bwd_preprocess launch");
}

static attn_status check_bwd_inputs(const attn_params* p, const void* q, const void* k,
                                    const void* v, const float* temperature,
                                    const int32_t* segment_ids, const int32_t* ranker_bounds,
                                    const void* d_o, const float* m, const float* l,
                                    const float* delta) {
  ATTN_TRY(check_common(p, temperature, segment_ids, ranker_bounds));
  ATTN_TRY(check_ptr(q, "q", 16));
  ATTN_TRY(check_ptr(k, "k", 16));
  ATTN_TRY(check_ptr(v, "v", 16));
  ATTN_TRY(check_ptr(d_o, "d_o", 16));
  ATTN_TRY(check_ptr(m, "m", 4));
  ATTN_TRY(check_ptr(l, "l", 4));
  ATTN_TRY(check_ptr(delta, "delta", 4));
  return ATTN_OK;
}

attn_status attn_bwd_dq(const attn_params* p, const void* q, const void* k, const void* v,
                        const float* temperature, const int32_t* segment_ids,
                        const int32_t* ranker_bounds, const void* d_o, const float* m,
                        const float* l, const float* delta, float* dq, float* dtemp_h,
                        void* stream) {
  ATTN_TRY(check_bwd_inputs(p, q, k, v, temperature, segment_ids, ranker_bounds, d_o, m, l, delta));
  ATTN_TRY(check_ptr(dq, "dq", 16));
  ATTN_TRY(check_opt(dtemp_h, "dtemp_h"));
  attn::KArgs a = make_args(p, temperature, segment_ids, ranker_bounds);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = d_o;
  a.m_in = m;
  a.l_in = l;
  a.delta_in = delta;
  a.out0 = dq;
  a.out3 = dtemp_h;
  a.n_items = a.B * a.Hq * a.n_q_tiles;
  return hip_status(attn::launch_dq(a, p->dtype, p->head_dim, effective_cap(p), (hipStream_t)stream),
                    "attn_bwd_dq launch");
}

attn_status attn_reduce_heads(const attn_params* p, const float* x, float* out, void* stream) {
  ATTN_TRY(check_params(p));
  ATTN_TRY(check_ptr(x, "x", 4));
  ATTN_TRY(check_ptr(out, "out", 4));
  return hip_status(attn::launch_reduce_heads(x, out, p->batch, p->q_heads, p->seq_len,
                                              (hipStream_t)stream),
                    "attn_reduce_heads launch");
}

attn_status attn_probe_stream(const void* src, int64_t bytes, int32_t blocks, float* out, void* stream) {
  if (blocks < 1 || blocks > 65536) return fail(ATTN_ERR_SHAPE, "blocks must be in [1, 65536]");
  if (bytes < 1 || bytes % (1024LL * blocks) != 0)
    return fail(ATTN_ERR_SHAPE, "bytes must be a positive multiple of 1024 * blocks");
  ATTN_TRY(check_ptr(src, "src", 16));
  ATTN_TRY(check_ptr(out, "out", 4));
  return hip_status(attn::launch_stream_probe(src, (long long)bytes, blocks, out, (hipStream_t)stream),
                    "attn_probe_stream launch");
}

attn_status attn_ranker_bounds(const int32_t* segment_ids, int32_t batch, int32_t seq_len,
                               int32_t history_id, int32_t candidate_id, int32_t* ranker_bounds,
                               void* stream) {
  if (batch < 1 || seq_len < 1) return fail(ATTN_ERR_SHAPE, "batch and seq_len must be >= 1");
  if (seq_len > ATTN_MAX_SEQ_LEN) return fail(ATTN_ERR_SHAPE, "seq_len exceeds ATTN_MAX_SEQ_LEN");
  if (history_id == candidate_id)
    return fail(ATTN_ERR_PARAM, "history_id and candidate_id must differ");
  ATTN_TRY(check_ptr(segment_ids, "segment_ids", 4));
  ATTN_TRY(check_ptr(ranker_bounds, "ranker_bounds", 4));
  return hip_status(attn::launch_ranker_bounds(segment_ids, ranker_bounds, batch, seq_len, history_id,
                                               candidate_id, (hipStream_t)stream),
                    "attn_ranker_bounds launch");
}

attn_status attn_bwd_dkv(const attn_params* p, const void* q, const void* k, const void* v,
                         const float* temperature, const int32_t* segment_ids,
                         const int32_t* ranker_bounds, const void* d_o, const float* m,
                         const float* l, const float* delta, float* dk, float* dv, void* stream) {
  ATTN_TRY(check_bwd_inputs(p, q, k, v, temperature, segment_ids, ranker_bounds, d_o, m, l, delta));
  ATTN_TRY(check_ptr(dk, "dk", 16));
  ATTN_TRY(check_ptr(dv, "dv", 16));
  attn::KArgs a = make_args(p, temperature, segment_ids, ranker_bounds);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = d_o;
  a.m_in = m;
  a.l_in = l;
  a.delta_in = delta;
  a.out0 = dk;
  a.out1 = dv;
  a.n_items = a.B * a.Hkv * a.n_kv_tiles;
  return hip_status(attn::launch_dkv(a, p->dtype, p->head_dim, effective_cap(p), (hipStream_t)stream),
                    "attn_bwd_dkv launch");
}

static attn_status check_ds_params(const attn_params* p) {
  ATTN_TRY(check_params(p));
  if (p->dtype != ATTN_BF16)
    return fail(ATTN_ERR_DTYPE, "the stored-dS backward takes bfloat16 inputs");
  if (p->precise_ds != 0)
    return fail(ATTN_ERR_UNSUPPORTED, "the stored-dS backward stores a single bf16 dS: precise_ds must be 0");
  return ATTN_OK;
}

static long long ds_slots(const attn_params* p) {
  return attn::ds_slots_per_head(attn::ds_band(p->seq_len, p->causal != 0, p->window_len));
}

attn_status attn_bwd_ds_workspace_size(const attn_params* p, uint64_t* bytes) {
  ATTN_TRY(check_ds_params(p));
  if (bytes == nullptr) return fail(ATTN_ERR_NULL_PTR, "bytes is NULL");
  const long long tiles = (long long)p->batch * p->q_heads * ds_slots(p);
  if (tiles > (1LL << 40)) return fail(ATTN_ERR_SHAPE, "stored-dS workspace too large");
  *bytes = (uint64_t)tiles * attn::DS_ELEMS * 2;
  return ATTN_OK;
}

static attn_status check_ds_workspace(const attn_params* p, const void* ds, uint64_t ds_bytes) {
  ATTN_TRY(check_ptr(ds, "ds", 16));
  uint64_t need = 0;
  ATTN_TRY(attn_bwd_ds_workspace_size(p, &need));
  if (ds_bytes < need)
    return fail(ATTN_ERR_SHAPE, "ds workspace of " + std::to_string(ds_bytes) + " bytes, " +
                                    std::to_string(need) + " needed");
  return ATTN_OK;
}

attn_status attn_bwd_dkv_ds(const attn_params* p, const void* q, const void* k, const void* v,
                            const float* temperature, const int32_t* segment_ids,
                            const int32_t* ranker_bounds, const void* d_o, const float* m,
                            const float* l, const float* delta, float* dk, float* dv, void* ds,
                            uint64_t ds_bytes, void* stream) {
  ATTN_TRY(check_ds_params(p));
  ATTN_TRY(check_bwd_inputs(p, q, k, v, temperature, segment_ids, ranker_bounds, d_o, m, l, delta));
  ATTN_TRY(check_ptr(dk, "dk", 16));
  ATTN_TRY(check_ptr(dv, "dv", 16));
  ATTN_TRY(check_ds_workspace(p, ds, ds_bytes));
  attn::KArgs a = make_args(p, temperature, segment_ids, ranker_bounds);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = d_o;
  a.m_in = m;
  a.l_in = l;
  a.delta_in = delta;
  a.out0 = dk;
  a.out1 = dv;
  a.ds = ds;
  a.ds_slots = ds_slots(p);
  a.n_items = a.B * a.Hkv * a.n_kv_tiles;
  return hip_status(attn::launch_dkv_ds_bf16(a, p->head_dim, effective_cap(p), (hipStream_t)stream),
                    "attn_bwd_dkv_ds launch");
}

attn_status attn_bwd_dq_ds(const attn_params* p, const void* k, const int32_t* segment_ids,
                           const int32_t* ranker_bounds, const void* ds, uint64_t ds_bytes,
                           float* dq, void* stream) {
  ATTN_TRY(check_ds_params(p));
  ATTN_TRY(check_common(p, nullptr, segment_ids, ranker_bounds));
  ATTN_TRY(check_ptr(k, "k", 16));
  ATTN_TRY(check_ds_workspace(p, ds, ds_bytes));
  ATTN_TRY(check_ptr(dq, "dq", 16));
  attn::KArgs a = make_args(p, nullptr, segment_ids, ranker_bounds);
  a.k = k;
  a.ds = const_cast<void*>(ds);
  a.ds_slots = ds_slots(p);
  a.out0 = dq;
  a.n_items = a.B * a.Hq * a.n_q_tiles;
  return hip_status(attn::launch_dq_ds_bf16(a, p->head_dim, (hipStream_t)stream),
                    "attn_bwd_dq_ds launch");
}

attn_status attn_bwd_ds_static(const attn_params* p, const void* q, const void* k, const void* v,
                               const float* temperature, const int32_t* segment_ids,
                               const int32_t* ranker_bounds, const void* d_o, const float* m,
                               const float* l, const float* delta, float* dq, float* dk, float* dv,
                               void* stream) {
  ATTN_TRY(check_ds_params(p));
  ATTN_TRY(check_bwd_inputs(p, q, k, v, temperature, segment_ids, ranker_bounds, d_o, m, l, delta));
  ATTN_TRY(check_ptr(dq, "dq", 16));
  ATTN_TRY(check_ptr(dk, "dk", 16));
  ATTN_TRY(check_ptr(dv, "dv", 16));
  uint64_t need = 0;
  ATTN_TRY(attn_bwd_ds_workspace_size(p, &need));
  if (need > ATTN_STATIC_DS_BYTES)
    return fail(ATTN_ERR_SHAPE, "the stored-dS workspace of this shape (" + std::to_string(need) +
                                    " bytes) exceeds the library's fixed array (" +
                                    std::to_string((unsigned long long)ATTN_STATIC_DS_BYTES) +
                                    " bytes): use attn_bwd_dkv_ds / attn_bwd_dq_ds with a caller "
                                    "workspace");
  void* ws = nullptr;
  ATTN_TRY(scratch_address(&ws));
  attn::KArgs a = make_args(p, temperature, segment_ids, ranker_bounds);
  a.q = q;
  a.k = k;
  a.v = v;
  a.dout = d_o;
  a.m_in = m;
  a.l_in = l;
  a.delta_in = delta;
  a.out0 = dk;
  a.out1 = dv;
  a.ds = ws;
  a.ds_slots = ds_slots(p);
  a.n_items = a.B * a.Hkv * a.n_kv_tiles;
  ATTN_TRY(hip_status(attn::launch_dkv_ds_bf16(a, p->head_dim, effective_cap(p), (hipStream_t)stream),
                      "attn_bwd_ds_static dK/dV launch"));
  attn::KArgs b = make_args(p, nullptr, segment_ids, ranker_bounds);
  b.k = k;
  b.ds = ws;
  b.ds_slots = ds_slots(p);
  b.out0 = dq;
  b.n_items = b.B * b.Hq * b.n_q_tiles;
  return hip_status(attn::launch_dq_ds_bf16(b, p->head_dim, (hipStream_t)stream),
                    "attn_bwd_ds_static dQ launch");
}

attn_status attn_plan_count(const attn_params* p, const int32_t* seg, const int32_t* bounds,
                            int64_t* unmasked_pairs, int64_t* visited_tiles) {
  ATTN_TRY(check_params(p));
  if (unmasked_pairs == nullptr || visited_tiles == nullptr)
    return fail(ATTN_ERR_NULL_PTR, "output counters are NULL");
  const int L = p->seq_len;
  const int BN = attn::fwd_key_tile(p->dtype, p->head_dim);
  long long pairs = 0, tiles = 0;
  for (int b = 0; b < p->batch; ++b) {
    attn::MaskSpec ms;
    ms.L = L;
    ms.causal = p->causal != 0;
    ms.window = p->window_len;
    ms.ranker = bounds != nullptr;
    ms.hl = ms.hu = ms.cl = ms.cu = 0;
    if (ms.ranker) {
      ms.hl = bounds[4 * b];
      ms.hu = bounds[4 * b + 1];
      ms.cl = bounds[4 * b + 2];
      ms.cu = bounds[4 * b + 3];
    }
    const int32_t* sb = seg ? seg + (size_t)b * L : nullptr;
    ms.has_seg = sb != nullptr;
    // positions of each segment id, for counting keys of one id in an interval
    std::unordered_map<int32_t, std::vector<int>> pos;
    if (sb)
      for (int j = 0; j < L; ++j) pos[sb[j]].push_back(j);
    auto count_in = [&](int i, int lo, int hi) -> long long {  // keys in [lo, hi] visible by id
      if (lo > hi) return 0;
      if (!sb) return (long long)hi - lo + 1;
      const std::vector<int>& v = pos[sb[i]];
      return (long long)(std::upper_bound(v.begin(), v.end(), hi) -
                         std::lower_bound(v.begin(), v.end(), lo));
    };
    for (int i = 0; i < L; ++i) {
      int kmin = 0, kmax = L - 1;
      if (ms.causal) kmax = std::min(kmax, i);
      if (ms.window > 0) kmin = std::max(kmin, i - ms.window + 1);
      if (kmin > kmax) continue;
      if (!ms.ranker) {
        pairs += count_in(i, kmin, kmax);
        continue;
      }
      const bool qh = i >= ms.hl && i < ms.hu, qc = i >= ms.cl && i < ms.cu;
      int lo = kmin, hi = kmax;
      long long c = 0;
      if (qh || qc) {
        lo = std::max(kmin, ms.hl);
        hi = std::min(kmax, ms.hu - 1);
        c = count_in(i, lo, hi);
      } else {
        lo = 1;
        hi = 0;
      }
      // the diagonal key i, for candidate rows, unless already counted
      if (qc && i >= kmin && i <= kmax && !(i >= lo && i <= hi)) c += 1;
      pairs += c;
    }
    // tiles the forward kernel visits
    const int nqt = (L + attn::BM - 1) / attn::BM;
    for (int qt = 0; qt < nqt; ++qt) {
      const int q0 = qt * attn::BM, q1 = std::min(q0 + attn::BM, L);
      int t0, t1;
      if (!attn::key_tile_range(q0, q1, BN, ms, &t0, &t1)) continue;
      int smin = 0, smax = 0;
      if (sb) {
        smin = *std::min_element(sb + q0, sb + q1);
        smax = *std::max_element(sb + q0, sb + q1);
      }
      for (int t = t0; t < t1; ++t) {
        if (attn::tile_class(q0, q1, t * BN, t * BN + BN, ms) == attn::TILE_EMPTY) continue;
        if (sb) {
          bool hit = false;
          for (int kk = t * BN; kk < std::min((t + 1) * BN, L) && !hit; ++kk)
            hit = sb[kk] >= smin && sb[kk] <= smax;
          if (!hit) continue;
        }
        ++tiles;
      }
    }
  }
  *unmasked_pairs = pairs * p->q_heads;
  *visited_tiles = tiles * p->q_heads;
  return ATTN_OK;
}

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ATTN_OK";
    case ATTN_ERR_NULL_PTR: return "ATTN_ERR_NULL_PTR";
    case ATTN_ERR_SHAPE: return "ATTN_ERR_SHAPE";
    case ATTN_ERR_DTYPE: return "ATTN_ERR_DTYPE";
    case ATTN_ERR_UNSUPPORTED: return "ATTN_ERR_UNSUPPORTED";
    case ATTN_ERR_ALIGN: return "ATTN_ERR_ALIGN";
    case ATTN_ERR_PARAM: return "ATTN_ERR_PARAM";
    case ATTN_ERR_HIP: return "ATTN_ERR_HIP";
  }
  return "unknown attn_status";
}

const char* attn_last_error(void) { return g_last_error.c_str(); }

const char* attn_build_info(void) {
  static std::string info;
  if (info.empty()) {
    char buf[256];
    snprintf(buf, sizeof(buf),
             "gfx950; fwd/dq rows per workgroup %d; dkv keys per workgroup %d; "
             "fwd key tile bf16 %d",
             attn::BM, attn::BKV, attn::fwd_key_tile(1, 128));
    info = buf;
  }
  return info.c_str();
}

}  // extern "C"
