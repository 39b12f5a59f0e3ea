// Backward preprocess: delta = rowsum(O * dO) (mosaic_backward.py page,
// make_preprocess_backward_kernel).  Memory-bound streaming kernel.
#include "attn_device.h"

namespace attn {

// ---------------------------------------------------------------------------
// Preprocess: delta = rowsum(O * dO).  16 lanes per (b, i, h) row.
// ---------------------------------------------------------------------------
template <typename T, int D>
__global__ __launch_bounds__(256) void preprocess_kernel(KArgs a) {
  constexpr int LPR = 16;            // lanes per row
  constexpr int EPL = D / LPR;       // elements per lane (4 or 8)
  const long row = (long)blockIdx.x * (256 / LPR) + threadIdx.x / LPR;
  const int sub = threadIdx.x % LPR;
  const long n_rows = (long)a.B * a.L * a.Hq;
  float acc = 0.f;
  if (row < n_rows) {
    const float* o = a.o_in + row * D + sub * EPL;
    const T* d = (const T*)a.dout + row * D + sub * EPL;
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc = __builtin_fmaf(o[e], (float)d[e], acc);
  }
#pragma unroll
  for (int off = LPR / 2; off > 0; off >>= 1) acc += __shfl_xor(acc, off);
  if (row < n_rows && sub == 0) {
    const int h = (int)(row % a.Hq);
    const long bi = row / a.Hq;
    const int i = (int)(bi % a.L), b = (int)(bi / a.L);
    a.out0[((long)b * a.Hq + h) * a.L + i] = acc;
  }
}

hipError_t launch_preprocess(const KArgs& a, int dtype, int head_dim, hipStream_t s) {
  const long n_rows = (long)a.B * a.L * a.Hq;
  dim3 grid((unsigned)((n_rows + 15) / 16)), block(256);
  if (dtype == 1) {
    if (head_dim == 64) hipLaunchKernelGGL((preprocess_kernel<bf16, 64>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((preprocess_kernel<bf16, 128>), grid, block, 0, s, a);
  } else {
    if (head_dim == 64) hipLaunchKernelGGL((preprocess_kernel<float, 64>), grid, block, 0, s, a);
    else hipLaunchKernelGGL((preprocess_kernel<float, 128>), grid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace attn
