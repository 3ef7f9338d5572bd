// Log-sum-exp merge of split-KV partials, in float32 for every storage type
// (rocMLIR "Fix split-kv attention masking and sweep RMS", Technical Details,
// host reference: the combine stage runs in f32 and casts back once).
//
// One wave per row: lanes reduce max and sum of the split LSEs, then walk the
// head dimension.  Rows whose every split is empty (all LSE = -inf) get
// output 0 and LSE -inf instead of a 0/0.
#include "device_common.h"
#include "pa_internal.h"

namespace pa {

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = __builtin_fmaxf(x, shfl_xor(x, m));
  return x;
}

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x += shfl_xor(x, m);
  return x;
}

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ part_out,
                                                      const float* __restrict__ part_lse,
                                                      T* __restrict__ out, float* __restrict__ lse,
                                                      int rows, int num_splits, int dv) {
  const int lane = threadIdx.x & 63;
  const int row = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // whole wave leaves together
  const float* lr = part_lse + static_cast<int64_t>(row) * num_splits;
  const float* orow = part_out + static_cast<int64_t>(row) * num_splits * dv;
  T* dst = out + static_cast<int64_t>(row) * dv;

  float mx = kNegInf;
  for (int s = lane; s < num_splits; s += 64) mx = __builtin_fmaxf(mx, lr[s]);
  mx = wave_max(mx);
  if (mx == kNegInf) {
    for (int d = lane; d < dv; d += 64) dst[d] = from_float<T>(0.f);
    if (lane == 0 && lse != nullptr) lse[row] = kNegInf;
    return;
  }
  float wsum = 0.f;
  for (int s = lane; s < num_splits; s += 64) wsum += expf(lr[s] - mx);
  wsum = wave_sum(wsum);
  for (int d = lane; d < dv; d += 64) {
    float a = 0.f;
    for (int s = 0; s < num_splits; ++s) a += expf(lr[s] - mx) * orow[s * dv + d];
    dst[d] = from_float<T>(a / wsum);
  }
  if (lane == 0 && lse != nullptr) lse[row] = mx + logf(wsum);
}

hipError_t launch_combine(int dtype, int rows, int num_splits, int head_dim_v,
                          const float* part_out, const float* part_lse, void* out, float* lse,
                          hipStream_t stream) {
  const dim3 grid((rows + 3) / 4), block(256);
  switch (dtype) {
    case kF32:
      combine_kernel<float><<<grid, block, 0, stream>>>(part_out, part_lse,
                                                         static_cast<float*>(out), lse, rows,
                                                         num_splits, head_dim_v);
      break;
    case kF16:
      combine_kernel<f16_t><<<grid, block, 0, stream>>>(part_out, part_lse,
                                                         static_cast<f16_t*>(out), lse, rows,
                                                         num_splits, head_dim_v);
      break;
    case kBF16:
      combine_kernel<bf16_t><<<grid, block, 0, stream>>>(part_out, part_lse,
                                                          static_cast<bf16_t*>(out), lse, rows,
                                                          num_splits, head_dim_v);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pa
