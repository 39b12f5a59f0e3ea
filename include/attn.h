/*
 * Blockwise online-softmax attention for AMD Instinct MI355X (gfx950): C ABI.
 *
 * Self-attention over packed rows, with an optional logit cap, per-query
 * temperature, segment / causal / sliding-window / ranker masks, grouped-query
 * heads, and the exact backward pass (plus an optional z-loss term).
 *
 * What is computed (web pages on unified blockwise attention):
 *   - triton_kernels.py page, make_triton_forward_kernel: s = sm_scale q.k,
 *     segment-equality, causal (i >= j) and window (j > i - W) predicates,
 *     online softmax with the (l, m) residuals;
 *   - mosaic_backward.py page, _apply_cap_mosaic: the caps
 *       none : s             tanh : cap tanh(s/cap)     soft_sign : s/(1+|s|/cap)
 *       alsc : cap (sig(a(s/cap+b)) - sig(ab)) / (sig(ab)(1-sig(ab)) + 1e-12);
 *   - triton_kernels.py page (dq and dkv kernels) and the module docstring of
 *     the mosaic_backward.py page: the backward chain
 *       dP = dO V^T, dS' = P (dP - delta) + w P LSE,
 *       dS = dS' temp cap'(s) sm_scale, dQ = dS K, dK = dS^T Q, dV = P^T dO;
 *   - mosaic_backward.py page, ranker_mask_mosaic_kv_q: the ranker mask;
 *   - mosaic_backward.py page, make_mosaic_backward_dq_kernel: the GQA map
 *     kv_head = q_head / (Hq / Hkv), dK and dV summed over each group.
 *
 * Definitions used here for every row i of (batch b, query head h), with
 * g = h / (Hq/Hkv):
 *   S'_ij = temp[b,i] * cap(sm_scale * <Q[b,i,h,:], K[b,j,g,:]>)   (visible j)
 *   m_i = max_j S'_ij,  l_i = sum_j exp(S'_ij - m_i),  LSE_i = m_i + ln l_i
 *   P_ij = exp(S'_ij - LSE_i) (0 for masked pairs),  O_i = sum_j P_ij V_j
 *   The backward is the gradient of sum(O * dO) + (w/2) sum_i LSE_i^2.
 *   A row that sees no key has O = 0, m = -inf, l = 0 and no gradient.
 *   The ALSC derivative is the exact one, a sig(z)(1-sig(z))/denom.
 *
 * Layouts (all contiguous, row-major, device memory):
 *   Q, dO, O, dQ : (B, L, Hq, D)      K, V, dK, dV : (B, L, Hkv, D)
 *   m, l, delta  : (B, Hq, L) float   temperature  : (B, L) float
 *   segment_ids  : (B, L) int32       ranker_bounds: (B, 4) int32 = hl, hu, cl, cu
 *   Q, K, V, dO are float or bfloat16 (params.dtype); O, m, l, delta, dQ, dK,
 *   dV are always float.
 *
 * Ownership: the caller allocates and owns every buffer; the library keeps
 * no state between calls and allocates no device memory (the one exception,
 * attn_bwd_ds_static, uses a fixed device array of the library instead of a
 * caller's workspace).  Every compute call
 * only enqueues kernels on `stream` (a hipStream_t; NULL = default stream) and
 * returns; the caller synchronises.  Outputs are overwritten, never
 * accumulated, and no call uses atomics: results are bitwise reproducible.
 *
 * Ranker bounds and segment ids may hold any int32 values: they only enter
 * the visibility predicates, never an address.
 *
 * Errors: every argument is validated on the host before any launch; on a
 * non-OK status nothing was enqueued, and attn_last_error() returns a
 * thread-local message.  A launch failure reported by the HIP runtime returns
 * ATTN_ERR_HIP.
 */
#ifndef BLOCKWISE_ATTN_H
#define BLOCKWISE_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  ATTN_OK = 0,
  ATTN_ERR_NULL_PTR = -1,    /* a required pointer is NULL */
  ATTN_ERR_SHAPE = -2,       /* a size is < 1 (L, B, heads) or too large (L, B*Hq*L > 2^36,
                                Hq*D > 2^22) */
  ATTN_ERR_DTYPE = -3,       /* dtype is neither ATTN_F32 nor ATTN_BF16 */
  ATTN_ERR_UNSUPPORTED = -4, /* head_dim not 64 or 128, or Hq not a multiple of Hkv */
  ATTN_ERR_ALIGN = -5,       /* a tensor pointer is not 16-byte aligned */
  ATTN_ERR_PARAM = -6,       /* unknown cap, window < 0, z-loss < 0, sm_scale <= 0,
                                or a non-finite scalar parameter */
  ATTN_ERR_HIP = -7          /* the HIP runtime reported an error at launch */
} attn_status;

typedef enum {
  ATTN_CAP_NONE = 0,
  ATTN_CAP_TANH = 1,
  ATTN_CAP_SOFT_SIGN = 2,
  ATTN_CAP_ALSC = 3
} attn_cap;

typedef enum { ATTN_F32 = 0, ATTN_BF16 = 1 } attn_dtype;

typedef struct {
  int32_t batch;        /* B >= 1 */
  int32_t seq_len;      /* L >= 1, <= ATTN_MAX_SEQ_LEN; queries and keys share it */
  int32_t q_heads;      /* Hq >= 1 */
  int32_t kv_heads;     /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;     /* D: 64 or 128 */
  int32_t dtype;        /* attn_dtype of Q, K, V, dO */
  float sm_scale;       /* > 0 */
  int32_t causal;       /* nonzero: key j visible from row i only if j <= i */
  int32_t window_len;   /* 0: off; else key j visible only if j > i - window_len */
  int32_t cap_method;   /* attn_cap; a cap <= 0 means no cap whatever the method */
  float cap, alpha, beta;
  float z_loss_weight;  /* w >= 0 */
  int32_t precise_ds;   /* bf16 only: nonzero feeds P (forward P V) and dS (dQ, dK)
                           to the MFMAs as a hi+lo pair of bf16 operands (two
                           MFMAs), zero as one bf16 each (faster, less precise) */
} attn_params;

#define ATTN_MAX_SEQ_LEN 262144
/* With segment ids the workgroup-local segment-skip table bounds L further. */
#define ATTN_MAX_SEQ_LEN_SEGMENTS 131072

/* Forward (triton_kernels.py page, make_triton_forward_kernel: scores, cap and
 * temperature inside the online-softmax update, the (l, m) residuals; caps from
 * the mosaic_backward.py page, _apply_cap_mosaic; ranker mask from its
 * ranker_mask_mosaic_kv_q).  temperature NULL means 1 everywhere; segment_ids
 * NULL means one segment; ranker_bounds NULL means no ranker mask.  Writes o
 * (B, L, Hq, D) float and m, l (B, Hq, L) float, m in natural-log units; a
 * row that sees no key gets o = 0, m = -inf, l = 0. */
attn_status attn_fwd(const attn_params* params, const void* q, const void* k, const void* v,
                     const float* temperature, const int32_t* segment_ids,
                     const int32_t* ranker_bounds, float* o, float* m, float* l,
                     void* stream);

/* Backward preprocess (mosaic_backward.py page, make_preprocess_backward_kernel):
 * delta[b,h,i] = sum_d O[b,i,h,d] * dO[b,i,h,d], with the normalised O that
 * attn_fwd writes. */
attn_status attn_bwd_preprocess(const attn_params* params, const float* o, const void* d_o,
                                float* delta, void* stream);

/* dQ (triton_kernels.py page, make_triton_backward_kernel_dq): recomputes P
 * from m and l and writes dq (B, L, Hq, D).
 * dtemp_h (optional, NULL skips it): (B, Hq, L) float, 4-byte aligned; row i
 * of head h receives that head's share of the temperature gradient,
 *   dtemp_h[b,h,i] = sum_j dS'_ij c_ij   (c = cap(sm_scale q.k), dS' as above),
 * since S' = temp * c.  The gradient of temperature[b,i] is the sum over h
 * (attn_reduce_heads).  The pages' orchestrator (mosaic_backward.py page,
 * mosaic_attention_backward) returns a dtemp slot filled with zeros; this is
 * the actual derivative. */
attn_status attn_bwd_dq(const attn_params* params, const void* q, const void* k, const void* v,
                        const float* temperature, const int32_t* segment_ids,
                        const int32_t* ranker_bounds, const void* d_o, const float* m,
                        const float* l, const float* delta, float* dq, float* dtemp_h,
                        void* stream);

/* out[b,i] = sum over h = 0 .. Hq-1 of x[b,h,i] in that fixed order (no
 * atomics), for x (B, Hq, L) and out (B, L) float, both 4-byte aligned; B, Hq
 * and L come from params.  Turns the per-head dtemp_h of attn_bwd_dq into the
 * gradient of the (B, L) temperature. */
attn_status attn_reduce_heads(const attn_params* params, const float* x, float* out, void* stream);

/* Ranker bounds from segment ids, on the device (the mosaic_backward.py page's
 * test marks history and candidate positions with two reserved segment ids;
 * the page prints neither the values nor how they map to bounds).  For each
 * batch row b of segment_ids (batch, seq_len) int32, writes ranker_bounds
 * (batch, 4) int32 = hl, hu, cl, cu where [hl, hu) is the smallest interval
 * holding every position whose id is history_id and [cl, cu) likewise for
 * candidate_id; an id that does not occur gives [0, 0).  For contiguous runs
 * (the page's layout) that is exactly the run.  Both pointers are device
 * memory, 4-byte aligned.  ATTN_ERR_PARAM if the two ids are equal. */
attn_status attn_ranker_bounds(const int32_t* segment_ids, int32_t batch, int32_t seq_len,
                               int32_t history_id, int32_t candidate_id, int32_t* ranker_bounds,
                               void* stream);

/* Measurement helper, not part of attention: the rate at which HBM feeds the
 * direct-to-LDS, non-temporal 16-byte loads the kernels stream their tiles
 * with.  blocks work-groups each read a contiguous bytes / blocks slice of src
 * (device memory, 16-byte aligned) into LDS that nothing reads, and write one
 * float per work-group to out (device memory, blocks floats, 4-byte aligned):
 * the first float of the slice's last 1 KB.  ATTN_ERR_SHAPE unless
 * 1 <= blocks <= 65536 and bytes is a positive multiple of 1024 * blocks.
 * Nothing is allocated; the caller times the call on its stream. */
attn_status attn_probe_stream(const void* src, int64_t bytes, int32_t blocks, float* out, void* stream);

/* dK and dV (triton_kernels.py page, make_triton_backward_kernel_dkv), each
 * summed over the Hq/Hkv query heads of a key/value head inside one
 * workgroup (no atomics).  Writes dk, dv (B, L, Hkv, D). */
attn_status attn_bwd_dkv(const attn_params* params, const void* q, const void* k, const void* v,
                         const float* temperature, const int32_t* segment_ids,
                         const int32_t* ranker_bounds, const void* d_o, const float* m,
                         const float* l, const float* delta, float* dk, float* dv,
                         void* stream);

/* Stored-dS backward: the same dQ, dK, dV as attn_bwd_dq + attn_bwd_dkv
 * (triton_kernels.py page, dq and dkv kernels; the chain of the
 * mosaic_backward.py page's module docstring), with dS computed once.
 * attn_bwd_dkv_ds does the work of attn_bwd_dkv and also stores dS, rounded
 * to bfloat16 exactly as it enters the dK product, into the caller's
 * workspace `ds`; attn_bwd_dq_ds then forms dQ = dS K from it, with no
 * recomputation of S, P or dP.  Call them in that order on one stream; the
 * workspace holds no state beyond that pair of calls and may be reused.
 *
 * Requirements: params.dtype == ATTN_BF16 (else ATTN_ERR_DTYPE) and
 * params.precise_ds == 0 (else ATTN_ERR_UNSUPPORTED: the stored dS is a single
 * bf16; with precise_ds use attn_bwd_dq, whose dS enters as hi + lo).
 *
 * Workspace: device memory of attn_bwd_ds_workspace_size() bytes, 16-byte
 * aligned, owned by the caller.  Layout (opaque to callers): per (batch row,
 * query head), one 128 x 128 bf16 tile per block of 128 queries x
 * 128 keys inside the causal / window band of its query block; blocks with
 * no visible pair are neither written nor read.  Size: B * Hq * tiles * 32 KiB
 * with tiles = T (T + 1) / 2 for causal attention without a window,
 * T = ceil(L / 128) (about L^2 bytes per head), T^2 without a mask, and about
 * T (W / 128 + 2) with a window W.
 *
 * ds_bytes is the size of the caller's workspace; ATTN_ERR_SHAPE (nothing
 * launched) if it is smaller than attn_bwd_ds_workspace_size().
 *
 * attn_bwd_dq_ds reads only k, segment_ids, ranker_bounds and ds (the same
 * segment ids and ranker bounds as the attn_bwd_dkv_ds call that wrote ds)
 * and writes dq (B, L, Hq, D) float. */
attn_status attn_bwd_ds_workspace_size(const attn_params* params, uint64_t* bytes);
attn_status attn_bwd_dkv_ds(const attn_params* params, const void* q, const void* k, const void* v,
                            const float* temperature, const int32_t* segment_ids,
                            const int32_t* ranker_bounds, const void* d_o, const float* m,
                            const float* l, const float* delta, float* dk, float* dv, void* ds,
                            uint64_t ds_bytes, void* stream);
attn_status attn_bwd_dq_ds(const attn_params* params, const void* k, const int32_t* segment_ids,
                           const int32_t* ranker_bounds, const void* ds, uint64_t ds_bytes,
                           float* dq, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the
 * stored-dS backward, attn_bwd_dkv_ds then attn_bwd_dq_ds on `stream`, with
 * the dS workspace taken from a fixed device array of the library instead of
 * a caller's buffer.  Same inputs as attn_bwd_dkv_ds (and the same
 * requirements: bf16, precise_ds == 0); writes dq (B, L, Hq, D), dk and dv
 * (B, L, Hkv, D) float, bit for bit what that pair of calls writes.
 *
 * Limit: attn_bwd_ds_workspace_size(params) must not exceed
 * ATTN_STATIC_DS_BYTES (128 MiB), else ATTN_ERR_SHAPE and nothing is
 * launched (the packed-causal B2 Hq8 L2048 and window B1 Hq16 L4096 W512
 * shapes need 68 and 75 MiB; the long-context and ranker shapes do not fit).
 * The array is reserved on each GPU the library runs on and held until the
 * process ends; its address is looked up once per device, on the first call
 * with that device current.  This call makes no hipMalloc, hipFree or other
 * allocating call.  Every call on one GPU shares that GPU's array, which keeps
 * the last call's contents (no part of it needs to start at zero: the dK/dV
 * kernel writes every tile the dQ kernel then reads), so calls that overlap
 * on one GPU (two streams or two host threads) race: the caller serialises
 * them. */
#define ATTN_STATIC_DS_BYTES (128ull << 20)
attn_status attn_bwd_ds_static(const attn_params* params, const void* q, const void* k,
                               const void* v, const float* temperature, const int32_t* segment_ids,
                               const int32_t* ranker_bounds, const void* d_o, const float* m,
                               const float* l, const float* delta, float* dq, float* dk, float* dv,
                               void* stream);

/* Host only, no GPU needed: exact number of visible (query, key) pairs summed
 * over batch rows and query heads, and the number of (query tile, key tile)
 * pairs the forward kernel visits, summed likewise.  segment_ids_host and
 * ranker_bounds_host are host pointers (or NULL). */
attn_status attn_plan_count(const attn_params* params, const int32_t* segment_ids_host,
                            const int32_t* ranker_bounds_host, int64_t* unmasked_pairs,
                            int64_t* visited_tiles);

/* Host only: validates params as the compute calls do, without any pointer. */
attn_status attn_check_params(const attn_params* params);

const char* attn_status_str(attn_status status);
const char* attn_last_error(void);   /* thread-local detail of the last non-OK status */
const char* attn_build_info(void);   /* tile sizes and target, for logs */

#ifdef __cplusplus
}
#endif

#endif /* BLOCKWISE_ATTN_H */
