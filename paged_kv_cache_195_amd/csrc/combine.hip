// Log-sum-exp merge of split-KV partials, in float32 for every storage type
// (rocMLIR "Fix split-kv attention masking and sweep RMS", Technical Details,
// host reference: the combine stage runs in f32 and casts back once).
//
// combine_row_kernel (S <= 256, Dv a multiple of 4 and at most 1024,
// 16-byte aligned partials -- every call the attention path makes): one
// workgroup per row.  Each thread reads the partials in 16-byte chunks, a
// chunk of the head dimension for every (256 / (Dv/4))-th split, issuing its
// first four loads at entry; meanwhile every wave reduces the S LSEs to their
// max M and the weights exp(lse_s - M) on its own (kept in its LDS row), so
// no workgroup barrier precedes the weighted sum; the split groups are then
// summed through LDS.
// combine_kernel (any other shape): one wave per row, lanes reduce max and
// sum of the split LSEs, then walk the head dimension.
// Rows whose every split is empty (all LSE = -inf) get output 0 and LSE -inf
// instead of a 0/0.
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
    for (int s = 0; s < num_splits; ++s)
      a += expf(lr[s] - mx) * orow[static_cast<int64_t>(s) * dv + d];
    dst[d] = from_float<T>(a / wsum);
  }
  if (lane == 0 && lse != nullptr) lse[row] = mx + logf(wsum);
}

constexpr int kCombineThreads = 256;

template <typename T>
__global__ __launch_bounds__(kCombineThreads) void combine_row_kernel(
    const float* __restrict__ part_out, const float* __restrict__ part_lse,
    T* __restrict__ out, float* __restrict__ lse, int num_splits, int dv) {
  typedef float f32x4_t __attribute__((ext_vector_type(4)));
  constexpr int kWaves = kCombineThreads / 64;
  constexpr int kLseSlots = kCombineThreads / 64;  // LSEs per lane (S <= 256)
  constexpr int kPrefetch = 4;                     // partial chunks loaded up front
  __shared__ float w_s[kWaves][kCombineThreads];   // each wave's own copy of the weights
  __shared__ f32x4_t acc_s[kCombineThreads];
  const int t = threadIdx.x;
  const int lane = t & 63, wave = t >> 6;
  const int64_t row = blockIdx.x;
  const float* lr = part_lse + row * num_splits;
  const float* orow = part_out + row * num_splits * dv;
  T* dst = out + row * dv;

  // thread (sg, c): chunk c (4 floats) of splits sg, sg + groups, ...; the
  // first kPrefetch of them are loaded before the weights are known, so their
  // latency overlaps the LSE reductions
  const int nc = dv >> 2;
  const int groups = kCombineThreads / nc;
  const int c = t % nc, sg = t / nc;
  const bool active = sg < groups;
  f32x4_t pv[kPrefetch];
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    const int sp = sg + k * groups;
    pv[k] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    if (active && sp < num_splits)
      pv[k] = *reinterpret_cast<const f32x4_t*>(orow + static_cast<int64_t>(sp) * dv + 4 * c);
  }

  // every wave reduces all S LSEs itself (lane holds splits lane + 64 j), so
  // no workgroup barrier is needed before the weighted sum
  float l[kLseSlots];
  float lm = kNegInf;
#pragma unroll
  for (int j = 0; j < kLseSlots; ++j) {
    const int sp = lane + 64 * j;
    l[j] = sp < num_splits ? lr[sp] : kNegInf;
    lm = __builtin_fmaxf(lm, l[j]);
  }
  const float mx = wave_max(lm);
  if (mx == kNegInf) {  // the same in every wave: every split is empty
    for (int d = t; d < dv; d += kCombineThreads) dst[d] = from_float<T>(0.f);
    if (t == 0 && lse != nullptr) lse[row] = kNegInf;
    return;
  }
  float ws = 0.f;
#pragma unroll
  for (int j = 0; j < kLseSlots; ++j) {
    const float w = l[j] == kNegInf ? 0.f : expf(l[j] - mx);
    w_s[wave][lane + 64 * j] = w;
    ws += w;
  }
  const float wsum = wave_sum(ws);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

  f32x4_t a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < kPrefetch; ++k) {
    const int sp = sg + k * groups;
    const float w = active && sp < num_splits ? w_s[wave][sp] : 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = __builtin_fmaf(w, pv[k][i], a[i]);
  }
  if (active) {
    for (int sp = sg + kPrefetch * groups; sp < num_splits; sp += groups) {
      const f32x4_t v = *reinterpret_cast<const f32x4_t*>(orow + static_cast<int64_t>(sp) * dv + 4 * c);
      const float w = w_s[wave][sp];
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = __builtin_fmaf(w, v[i], a[i]);
    }
  }
  if (groups > 1) {
    acc_s[t] = a;
    __syncthreads();
    if (t < nc) {
      a = acc_s[t];
      for (int k = 1; k < groups; ++k) {
        const f32x4_t q = acc_s[k * nc + t];
#pragma unroll
        for (int i = 0; i < 4; ++i) a[i] += q[i];
      }
    }
  }
  if (t < nc) {
#pragma unroll
    for (int i = 0; i < 4; ++i) dst[4 * t + i] = from_float<T>(a[i] / wsum);
  }
  if (t == 0 && lse != nullptr) lse[row] = mx + logf(wsum);
}

template <typename T>
hipError_t launch_combine_t(int rows, int num_splits, int dv, const float* part_out,
                            const float* part_lse, T* out, float* lse, hipStream_t stream) {
  const bool row_kernel = num_splits <= kCombineThreads && dv % 4 == 0 &&
                          dv / 4 <= kCombineThreads &&
                          (reinterpret_cast<uintptr_t>(part_out) & 15u) == 0;
  if (row_kernel)
    combine_row_kernel<T><<<dim3(rows), dim3(kCombineThreads), 0, stream>>>(
        part_out, part_lse, out, lse, num_splits, dv);
  else
    combine_kernel<T><<<dim3((rows + 3) / 4), dim3(256), 0, stream>>>(part_out, part_lse, out,
                                                                      lse, rows, num_splits, dv);
  return hipGetLastError();
}

hipError_t launch_combine(int dtype, int rows, int num_splits, int head_dim_v,
                          const float* part_out, const float* part_lse, void* out, float* lse,
                          hipStream_t stream) {
  switch (dtype) {
    case kF32:
      return launch_combine_t(rows, num_splits, head_dim_v, part_out, part_lse,
                              static_cast<float*>(out), lse, stream);
    case kF16:
      return launch_combine_t(rows, num_splits, head_dim_v, part_out, part_lse,
                              static_cast<f16_t*>(out), lse, stream);
    case kBF16:
      return launch_combine_t(rows, num_splits, head_dim_v, part_out, part_lse,
                              static_cast<bf16_t*>(out), lse, stream);
    default:
      return hipErrorInvalidValue;
  }
}

}  // namespace pa
