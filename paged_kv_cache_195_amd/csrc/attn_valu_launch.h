// Template dispatch of the vector-ALU attention kernel over (D, page size,
// rows per workgroup).  Included by the f32 instantiation.
#pragma once

#include "attn_valu.h"

namespace pa {

template <typename T, int D, int PS, int MR>
hipError_t launch_attn_valu_cfg(const AttnParams& p, const AttnPlan& plan, int batch,
                                hipStream_t stream) {
  constexpr ValuConfig cfg = valu_config(sizeof(T), D, PS, MR);
  if (plan.waves != cfg.waves || cfg.waves % plan.heads_per_wg != 0 ||
      p.num_kv_heads % plan.heads_per_wg != 0)
    return hipErrorInvalidValue;
  const dim3 grid(plan.num_splits * plan.row_groups, p.num_kv_heads / plan.heads_per_wg, batch);
  const dim3 block(cfg.waves * 64);
  attn_valu_kernel<T, D, PS, MR, cfg.waves, cfg.pages_ahead, true><<<grid, block, 0, stream>>>(p);
  return hipGetLastError();
}

template <typename T, int D, int PS>
hipError_t launch_attn_valu_dp(const AttnParams& p, const AttnPlan& plan, int batch,
                               hipStream_t stream) {
  switch (plan.rows_per_wg) {
    case 1: return launch_attn_valu_cfg<T, D, PS, 1>(p, plan, batch, stream);
    case 2: return launch_attn_valu_cfg<T, D, PS, 2>(p, plan, batch, stream);
    case 4: return launch_attn_valu_cfg<T, D, PS, 4>(p, plan, batch, stream);
    case 8:
      if constexpr (valu_max_rows(sizeof(T), D, PS) >= 8)
        return launch_attn_valu_cfg<T, D, PS, 8>(p, plan, batch, stream);
      else
        return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
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
