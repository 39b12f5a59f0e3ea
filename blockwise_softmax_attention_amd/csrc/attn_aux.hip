// Small HBM-bound helpers around the attention kernels.
//
// reduce_heads: out[b, i] = sum over h of x[b, h, i], heads added in the
// order 0 .. Hq-1 by one thread per (b, i), so the result does not depend on
// scheduling.  Used for the temperature gradient: one temperature row serves
// every query head, and attn_bwd_dq writes each head's share separately.
//
// ranker_bounds: per batch row, [hl, hu) = the smallest interval holding
// every position whose segment id is history_id, [cl, cu) likewise for
// candidate_id, [0, 0) for an id that does not occur.  (mosaic_backward.py
// page, test harness: the ranker's history and candidate rows are marked by
// two reserved segment ids; the page prints neither the values nor the
// mapping, so both ids are arguments and the interval is this reading.)
//
// stream_probe: a read-rate reference, not part of attention.  Each
// work-group reads its own contiguous slice of src with the direct-to-LDS,
// non-temporal 16-byte loads the kernels use (1 KB per wave instruction, at
// most 8 in flight per wave) into a 64 KB LDS ring that nothing else reads,
// then writes the first float of its slice's last 1 KB to out[block].
#include "attn_internal.h"
#include "attn_tiles.h"
#include "attn_bf16.h"

namespace attn {

__global__ __launch_bounds__(256) void reduce_heads_kernel(const float* __restrict__ x,
                                                           float* __restrict__ out, int B, int H,
                                                           int L) {
  const long n = (long)B * L;
  for (long e = (long)blockIdx.x * blockDim.x + threadIdx.x; e < n; e += (long)gridDim.x * blockDim.x) {
    const long b = e / L, i = e - b * L;
    const float* src = x + b * H * (long)L + i;
    float s = 0.f;
    for (int h = 0; h < H; ++h) s += src[(long)h * L];
    out[e] = s;
  }
}

// One workgroup per batch row: each thread scans a strided share of the row,
// then a min / max reduction in LDS (integer min / max: order-independent).
__global__ __launch_bounds__(256) void ranker_bounds_kernel(const int32_t* __restrict__ seg,
                                                            int32_t* __restrict__ bounds, int L,
                                                            int32_t hist_id, int32_t cand_id) {
  __shared__ int r_hmin[256], r_hmax[256], r_cmin[256], r_cmax[256];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int32_t* row = seg + (long)b * L;
  int hmin = L, hmax = -1, cmin = L, cmax = -1;
  for (int i = tid; i < L; i += blockDim.x) {
    const int32_t s = row[i];
    if (s == hist_id) {
      hmin = imin(hmin, i);
      hmax = imax(hmax, i);
    }
    if (s == cand_id) {
      cmin = imin(cmin, i);
      cmax = imax(cmax, i);
    }
  }
  r_hmin[tid] = hmin;
  r_hmax[tid] = hmax;
  r_cmin[tid] = cmin;
  r_cmax[tid] = cmax;
  __syncthreads();
  for (int w = blockDim.x / 2; w > 0; w >>= 1) {
    if (tid < w) {
      r_hmin[tid] = imin(r_hmin[tid], r_hmin[tid + w]);
      r_hmax[tid] = imax(r_hmax[tid], r_hmax[tid + w]);
      r_cmin[tid] = imin(r_cmin[tid], r_cmin[tid + w]);
      r_cmax[tid] = imax(r_cmax[tid], r_cmax[tid + w]);
    }
    __syncthreads();
  }
  if (tid == 0) {
    const bool h = r_hmax[0] >= 0, c = r_cmax[0] >= 0;
    bounds[4 * b + 0] = h ? r_hmin[0] : 0;
    bounds[4 * b + 1] = h ? r_hmax[0] + 1 : 0;
    bounds[4 * b + 2] = c ? r_cmin[0] : 0;
    bounds[4 * b + 3] = c ? r_cmax[0] + 1 : 0;
  }
}

__global__ __launch_bounds__(256) void stream_probe_kernel(const char* __restrict__ src, long long per_wg,
                                                           float* __restrict__ out) {
  __shared__ __attribute__((aligned(1024))) char ring[64 * 1024];
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const char* base = src + blockIdx.x * per_wg;
  const long long nchunks = per_wg / 1024;
  const uint32_t ring0 = lds_offset(ring);
  for (long long c = wave; c < nchunks; c += 4) {
    // slot (wave, (c / 4) % 16): 16 KB of the ring per wave
    const uint32_t m0 = (uint32_t)__builtin_amdgcn_readfirstlane(ring0 + (uint32_t)(wave * 16 + ((c >> 2) & 15)) * 1024u);
    dma16_nt(uniform_ptr(base + c * 1024), 16u * (uint32_t)lane, m0);
    wait_vmcnt<8>();
  }
  wait_vmcnt<0>();
  __syncthreads();
  if (threadIdx.x == 0) {
    const long long c = nchunks - 1;
    const int w = (int)(c & 3);
    out[blockIdx.x] = *(const float*)(ring + (w * 16 + ((c >> 2) & 15)) * 1024);
  }
}

hipError_t launch_stream_probe(const void* src, long long bytes, int blocks, float* out, hipStream_t s) {
  hipLaunchKernelGGL(stream_probe_kernel, dim3(blocks), dim3(256), 0, s, (const char*)src,
                     bytes / blocks, out);
  return hipGetLastError();
}

hipError_t launch_reduce_heads(const float* x, float* out, int B, int H, int L, hipStream_t s) {
  const long n = (long)B * L;
  const long want = (n + 255) / 256;
  const int grid = (int)(want < 4096 ? want : 4096);
  hipLaunchKernelGGL(reduce_heads_kernel, dim3(grid), dim3(256), 0, s, x, out, B, H, L);
  return hipGetLastError();
}

hipError_t launch_ranker_bounds(const int32_t* seg, int32_t* bounds, int B, int L, int32_t hist_id,
                                int32_t cand_id, hipStream_t s) {
  hipLaunchKernelGGL(ranker_bounds_kernel, dim3(B), dim3(256), 0, s, seg, bounds, L, hist_id,
                     cand_id);
  return hipGetLastError();
}

}  // namespace attn
