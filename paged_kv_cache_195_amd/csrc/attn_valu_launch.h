// Template dispatch of the vector-ALU attention kernel over (D, page size,
// rows per workgroup).  Included once per element type.
#pragma once

#include "attn_valu.h"

namespace pa {

constexpr int kValuWaves = 4;

template <typename T, int D, int PS>
hipError_t launch_attn_valu_dp(const AttnParams& p, const AttnPlan& plan, int batch,
                               hipStream_t stream) {
  const dim3 grid(plan.num_splits * plan.row_groups, p.num_kv_heads, batch);
  const dim3 block(kValuWaves * 64);
  switch (plan.rows_per_wg) {
    case 1: attn_valu_kernel<T, D, PS, 1, kValuWaves><<<grid, block, 0, stream>>>(p); break;
    case 2: attn_valu_kernel<T, D, PS, 2, kValuWaves><<<grid, block, 0, stream>>>(p); break;
    case 4: attn_valu_kernel<T, D, PS, 4, kValuWaves><<<grid, block, 0, stream>>>(p); break;
    case 8: attn_valu_kernel<T, D, PS, 8, kValuWaves><<<grid, block, 0, stream>>>(p); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn_valu_t(const AttnParams& p, const AttnPlan& plan, int head_dim,
                              int page_size, int batch, hipStream_t stream) {
  if (page_size == 16) {
    if (head_dim == 32) return launch_attn_valu_dp<T, 32, 16>(p, plan, batch, stream);
    if (head_dim == 64) return launch_attn_valu_dp<T, 64, 16>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_valu_dp<T, 128, 16>(p, plan, batch, stream);
  } else if (page_size == 32) {
    if (head_dim == 32) return launch_attn_valu_dp<T, 32, 32>(p, plan, batch, stream);
    if (head_dim == 64) return launch_attn_valu_dp<T, 64, 32>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_valu_dp<T, 128, 32>(p, plan, batch, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
