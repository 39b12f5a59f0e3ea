// Shared by the backward kernels.
#pragma once

#include "attn_device.h"

namespace attn {

// Per-row backward constants from the forward residuals: log2 LSE, and
// delta' = delta - w LSE.  A row with l == 0 saw no key: lse2 = +inf makes P
// vanish and delta' = 0.
__device__ __forceinline__ void residuals_from(float m, float l, float d, float zw, float& lse2,
                                               float& dlt) {
  if (l > 0.f) {
    const float lse = m + logf(l);
    lse2 = lse * LOG2E_F;
    dlt = d - zw * lse;
  } else {
    lse2 = ATTN_POS_INF;
    dlt = 0.f;
  }
}

__device__ __forceinline__ void row_residuals(const KArgs& a, long idx, float& lse2, float& dlt) {
  residuals_from(a.m_in[idx], a.l_in[idx], a.delta_in[idx], a.zw, lse2, dlt);
}

}  // namespace attn
