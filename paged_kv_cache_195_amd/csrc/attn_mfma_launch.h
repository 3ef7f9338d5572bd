// Template dispatch of the MFMA attention kernel over (D, page size).
// Included once per 16-bit element type.
#pragma once

#include "attn_mfma.h"
#include "attn_mfma_rows.h"
#include "attn_prefill.h"
#include "attn_prefill_pp.h"

namespace pa {

template <typename T, typename KV, int D, int PS, int NW, int RB>
hipError_t launch_attn_mfma_dpw(const AttnParams& p, const AttnPlan& plan, int batch,
                                hipStream_t stream) {
  if (plan.rows_per_wg != 16 * RB || NW % plan.heads_per_wg != 0 ||
      p.num_kv_heads % plan.heads_per_wg != 0)
    return hipErrorInvalidValue;
  const dim3 grid(plan.num_splits * plan.row_groups, p.num_kv_heads / plan.heads_per_wg, batch);
  // 4-wave workgroups reserve unused LDS so that two, not three, stay resident
  // per compute unit: 8 waves per CU, as with 8-wave workgroups.  At 12 resident
  // waves the Qwen3-235B decode step took 726 us instead of 632.
  constexpr int kStatic = RB == 1 ? mfma_static_lds<D, NW>() : mfma_rows_static_lds<D, NW, RB>();
  constexpr size_t kReserve = NW == 4 && kStatic < kMfmaLdsPerNarrowWg
                                  ? static_cast<size_t>(kMfmaLdsPerNarrowWg - kStatic)
                                  : 0;
  if constexpr (RB == 1)
    attn_mfma_kernel<T, KV, D, PS, NW><<<grid, dim3(NW * 64), kReserve, stream>>>(p);
  else
    attn_mfma_rows_kernel<T, KV, D, PS, NW, RB><<<grid, dim3(NW * 64), kReserve, stream>>>(p);
  return hipGetLastError();
}

// 16-bit caches: 8 or 4 waves per workgroup; 8-bit codes: 8.  One or two
// blocks of 16 rows per wave (rows_per_wg 16 or 32).
template <typename T, typename KV, int D, int PS, int NW>
hipError_t launch_attn_mfma_dpn(const AttnParams& p, const AttnPlan& plan, int batch,
                                hipStream_t stream) {
  if (plan.rows_per_wg == 32) return launch_attn_mfma_dpw<T, KV, D, PS, NW, 2>(p, plan, batch, stream);
  return launch_attn_mfma_dpw<T, KV, D, PS, NW, 1>(p, plan, batch, stream);
}

template <typename T, typename KV, int D, int PS>
hipError_t launch_attn_mfma_dp(const AttnParams& p, const AttnPlan& plan, int batch,
                               hipStream_t stream) {
  if (plan.waves == kMfmaWaves)
    return launch_attn_mfma_dpn<T, KV, D, PS, kMfmaWaves>(p, plan, batch, stream);
  if constexpr (!KvTraits<KV>::quant) {
    if (plan.waves == kMfmaWavesNarrow)
      return launch_attn_mfma_dpn<T, KV, D, PS, kMfmaWavesNarrow>(p, plan, batch, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T, int D, int PS>
hipError_t launch_attn_prefill_dp(const AttnParams& p, const AttnPlan& plan, int batch,
                                  hipStream_t stream) {
  constexpr int kWaves = prefill_waves(D);
  if (plan.waves != kWaves || plan.rows_per_wg != 16 * kPrefillRowBlocks * kWaves ||
      plan.heads_per_wg != 1)
    return hipErrorInvalidValue;
  const dim3 grid(plan.num_splits * plan.row_groups, p.num_kv_heads, batch);
  // the kernels' workgroup order is computed in 32-bit arithmetic
  if (static_cast<uint64_t>(grid.x) * grid.y * grid.z > 0xFFFFFFFFull)
    return hipErrorInvalidConfiguration;
  if constexpr (kWaves == kPrefillTeamWaves) {
    static_assert(kPrefillRowBlocks == 2, "the two-team kernel holds two row blocks per wave");
    attn_prefill_pp_kernel<T, D, PS><<<grid, dim3(kWaves * 64), 0, stream>>>(p);
  } else {
    attn_prefill_kernel<T, D, PS, kWaves, kPrefillRowBlocks>
        <<<grid, dim3(kWaves * 64), 0, stream>>>(p);
  }
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
    if (head_dim == 32) return launch_attn_mfma_dp<T, KvSame, 32, 16>(p, plan, batch, stream);
    if (head_dim == 64) return launch_attn_mfma_dp<T, KvSame, 64, 16>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_mfma_dp<T, KvSame, 128, 16>(p, plan, batch, stream);
  } else if (page_size == 32) {
    if (head_dim == 32) return launch_attn_mfma_dp<T, KvSame, 32, 32>(p, plan, batch, stream);
    if (head_dim == 64) return launch_attn_mfma_dp<T, KvSame, 64, 32>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_mfma_dp<T, KvSame, 128, 32>(p, plan, batch, stream);
  }
  return hipErrorInvalidValue;
}

// 8-bit K/V codes, shared-tile prefill: the single-team kernel at both head
// dims (its K tile passes through registers to be decoded, which the two-team
// kernel's direct-to-LDS K loads cannot do).
template <typename T, typename KV, int D, int PS>
hipError_t launch_attn_prefill_q_dp(const AttnParams& p, const AttnPlan& plan, int batch,
                                    hipStream_t stream) {
  if (plan.waves != kPrefillWaves || plan.rows_per_wg != 16 * kPrefillRowBlocks * kPrefillWaves ||
      plan.heads_per_wg != 1)
    return hipErrorInvalidValue;
  const dim3 grid(plan.num_splits * plan.row_groups, p.num_kv_heads, batch);
  attn_prefill_kernel<T, D, PS, kPrefillWaves, kPrefillRowBlocks, KV>
      <<<grid, dim3(kPrefillWaves * 64), 0, stream>>>(p);
  return hipGetLastError();
}

// 8-bit K/V codes: the MFMA kernel, or the shared-tile prefill kernel.
template <typename T, typename KV>
hipError_t launch_attn_mfma_q_kv(const AttnParams& p, const AttnPlan& plan, int head_dim,
                                 int page_size, int batch, hipStream_t stream) {
  if (plan.prefill) {
    if (page_size == 16) {
      if (head_dim == 64) return launch_attn_prefill_q_dp<T, KV, 64, 16>(p, plan, batch, stream);
      if (head_dim == 128) return launch_attn_prefill_q_dp<T, KV, 128, 16>(p, plan, batch, stream);
    } else if (page_size == 32) {
      if (head_dim == 64) return launch_attn_prefill_q_dp<T, KV, 64, 32>(p, plan, batch, stream);
      if (head_dim == 128) return launch_attn_prefill_q_dp<T, KV, 128, 32>(p, plan, batch, stream);
    }
    return hipErrorInvalidValue;
  }
  if (page_size == 16) {
    if (head_dim == 64) return launch_attn_mfma_dp<T, KV, 64, 16>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_mfma_dp<T, KV, 128, 16>(p, plan, batch, stream);
  } else if (page_size == 32) {
    if (head_dim == 64) return launch_attn_mfma_dp<T, KV, 64, 32>(p, plan, batch, stream);
    if (head_dim == 128) return launch_attn_mfma_dp<T, KV, 128, 32>(p, plan, batch, stream);
  }
  return hipErrorInvalidValue;
}

template <typename T>
hipError_t launch_attn_mfma_q_t(const AttnParams& p, const AttnPlan& plan, int kv_dtype,
                                int head_dim, int page_size, int batch, hipStream_t stream) {
  if (kv_dtype == kI8)
    return launch_attn_mfma_q_kv<T, KvI8>(p, plan, head_dim, page_size, batch, stream);
  if (kv_dtype == kFp8E4M3)
    return launch_attn_mfma_q_kv<T, KvFp8>(p, plan, head_dim, page_size, batch, stream);
  return hipErrorInvalidValue;
}

}  // namespace pa
