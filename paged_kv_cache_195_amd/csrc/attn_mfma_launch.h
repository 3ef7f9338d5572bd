// Template dispatch of the MFMA attention kernel over (D, page size).
// Included once per 16-bit element type.
#pragma once

#include "attn_mfma.h"
#include "attn_prefill.h"

namespace pa {

template <typename T, int D, int PS>
hipError_t launch_attn_mfma_dp(const AttnParams& p, const AttnPlan& plan, int batch,
                               hipStream_t stream) {
  if (plan.waves != kMfmaWaves || plan.rows_per_wg != 16 || kMfmaWaves % plan.heads_per_wg != 0 ||
      p.num_kv_heads % plan.heads_per_wg != 0)
    return hipErrorInvalidValue;
  const dim3 grid(plan.num_splits * plan.row_groups, p.num_kv_heads / plan.heads_per_wg, batch);
  attn_mfma_kernel<T, D, PS, kMfmaWaves><<<grid, dim3(kMfmaWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

template <typename T, int D, int PS>
hipError_t launch_attn_prefill_dp(const AttnParams& p, const AttnPlan& plan, int batch,
                                  hipStream_t stream) {
  if (plan.waves != kPrefillWaves || plan.rows_per_wg != 16 * kPrefillRowBlocks * kPrefillWaves ||
      plan.heads_per_wg != 1)
    return hipErrorInvalidValue;
  const dim3 grid(plan.num_splits * plan.row_groups, p.num_kv_heads, batch);
  attn_prefill_kernel<T, D, PS, kPrefillWaves, kPrefillRowBlocks>
      <<<grid, dim3(kPrefillWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_attn_prefill_t(const AttnParams& p, const AttnPlan& plan, int head_dim,
                                 int page_size, int batch, hipStream_t stream) {
  if (page_size == 16) {
    if (head_dim == 64) return launch_attn_prefill_dp<T, 64, 16>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_prefill_dp<T, 128, 16>(p, plan, batch, stream);
  } else if (page_size == 32) {
    if (head_dim == 64) return launch_attn_prefill_dp<T, 64, 32>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_prefill_dp<T, 128, 32>(p, plan, batch, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_attn_mfma_t(const AttnParams& p, const AttnPlan& plan, int head_dim,
                              int page_size, int batch, hipStream_t stream) {
  if (plan.prefill) return launch_attn_prefill_t<T>(p, plan, head_dim, page_size, batch, stream);
  if (page_size == 16) {
    if (head_dim == 32) return launch_attn_mfma_dp<T, 32, 16>(p, plan, batch, stream);
    if (head_dim == 64) return launch_attn_mfma_dp<T, 64, 16>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_mfma_dp<T, 128, 16>(p, plan, batch, stream);
  } else if (page_size == 32) {
    if (head_dim == 32) return launch_attn_mfma_dp<T, 32, 32>(p, plan, batch, stream);
    if (head_dim == 64) return launch_attn_mfma_dp<T, 64, 32>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_mfma_dp<T, 128, 32>(p, plan, batch, stream);
  }
  return hipErrorInvalidValue;
}

}  // namespace pa
