// Device helpers shared by the kernels: element types, 16-byte chunk
// arithmetic and wavefront (64-lane) reductions for gfx950.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pa {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

// Storage-only bfloat16 (the top 16 bits of an IEEE float).
struct bf16_t {
  uint16_t bits;
};
using f16_t = _Float16;

constexpr float kNegInf = -__builtin_huge_valf();
constexpr float kLn2 = 0.693147180559945309417f;

// ---------------------------------------------------------------- 16-byte chunks
// A lane moves K/V in 16-byte chunks (one global_load_dwordx4).

// Word i of a chunk, by value.  The copy into a scalar matters: this clang
// compiles __builtin_bit_cast(T, v[i]) on an ext_vector element as element 0
// whatever i is, so every bit cast below goes through word().
__device__ __forceinline__ uint32_t word(const u32x4& v, int i) {
  const uint32_t w = v[i];
  return w;
}

template <typename T>
struct Chunk {
  static constexpr int kElems = 16 / sizeof(T);
};

// sum_e a[e] * b[e] over one chunk, accumulated in float32.  16-bit types use
// the packed dot instructions (v_dot2_f32_f16 / v_dot2_f32_bf16): products of
// two 16-bit values are exact in float32.
template <typename T>
__device__ __forceinline__ float chunk_dot(const u32x4& a, const u32x4& b, float acc);

template <>
__device__ __forceinline__ float chunk_dot<float>(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_fmaf(__builtin_bit_cast(float, word(a, i)),
                          __builtin_bit_cast(float, word(b, i)), acc);
  return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<f16_t>(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, word(a, i)),
                                 __builtin_bit_cast(f16x2_t, word(b, i)), acc, false);
  return acc;
}

template <>
__device__ __forceinline__ float chunk_dot<bf16_t>(const u32x4& a, const u32x4& b, float acc) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
    acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, word(a, i)),
                                          __builtin_bit_cast(bf16x2_t, word(b, i)), acc, false);
  return acc;
}

// Widen one chunk to float32 (exact for every element type).
template <typename T>
__device__ __forceinline__ void chunk_to_float(const u32x4& c, float* f);

template <>
__device__ __forceinline__ void chunk_to_float<float>(const u32x4& c, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) f[i] = __builtin_bit_cast(float, word(c, i));
}

template <>
__device__ __forceinline__ void chunk_to_float<f16_t>(const u32x4& c, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, word(c, i));
    f[2 * i] = static_cast<float>(h[0]);
    f[2 * i + 1] = static_cast<float>(h[1]);
  }
}

template <>
__device__ __forceinline__ void chunk_to_float<bf16_t>(const u32x4& c, float* f) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t w = word(c, i);
    f[2 * i] = __builtin_bit_cast(float, w << 16);
    f[2 * i + 1] = __builtin_bit_cast(float, w & 0xffff0000u);
  }
}

// Round a float32 to the storage type (round to nearest, ties to even).
template <typename T>
__device__ __forceinline__ T from_float(float x);

template <>
__device__ __forceinline__ float from_float<float>(float x) { return x; }

template <>
__device__ __forceinline__ f16_t from_float<f16_t>(float x) { return static_cast<f16_t>(x); }

// bf16: gfx950's conversion instruction (v_cvt_pk_bf16_f32) rounds to nearest
// even and quiets NaN in one instruction, where the integer form took six.
template <>
__device__ __forceinline__ bf16_t from_float<bf16_t>(float x) {
  bf16_t r;
  r.bits = __builtin_bit_cast(uint16_t, static_cast<__bf16>(x));
  return r;
}

// ---------------------------------------------------------------- lane exchange
// DPP moves inside a row of 16 lanes; every source lane is inside the row, so
// no lane reads an undefined value.
template <int kCtrl>
__device__ __forceinline__ float dpp_mov(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xf, 0xf, false));
}

constexpr int kDppQuadXor1 = 0xb1;      // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4e;      // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;

__device__ __forceinline__ float swizzle_xor16(float x) {
  // ds_swizzle bit-mask mode: and 0x1f, or 0, xor 0x10 (within 32 lanes).
  return __builtin_bit_cast(float, __builtin_amdgcn_ds_swizzle(__builtin_bit_cast(int, x), 0x401f));
}

__device__ __forceinline__ float shfl_xor(float x, int mask) {
  const int lane = __lane_id();
  return __builtin_bit_cast(
      float, __builtin_amdgcn_ds_bpermute((lane ^ mask) << 2, __builtin_bit_cast(int, x)));
}

// Sum over aligned groups of N consecutive lanes; every lane of a group gets
// the same bits (each step adds two values in commutative pairs).
template <int N>
__device__ __forceinline__ float group_sum(float x) {
  static_assert(N == 1 || N == 2 || N == 4 || N == 8 || N == 16 || N == 32 || N == 64, "N");
  if constexpr (N >= 2) x += dpp_mov<kDppQuadXor1>(x);
  if constexpr (N >= 4) x += dpp_mov<kDppQuadXor2>(x);
  if constexpr (N >= 8) x += dpp_mov<kDppRowHalfMirror>(x);
  if constexpr (N >= 16) x += dpp_mov<kDppRowMirror>(x);
  if constexpr (N >= 32) x += swizzle_xor16(x);
  if constexpr (N >= 64) x += shfl_xor(x, 32);
  return x;
}

// Reductions over the lanes that share (lane mod N): masks N, 2N, ..., 32.
template <int N>
__device__ __forceinline__ float strided_max(float x) {
#pragma unroll
  for (int m = N; m < 64; m <<= 1) x = __builtin_fmaxf(x, shfl_xor(x, m));
  return x;
}

template <int N>
__device__ __forceinline__ float strided_sum(float x) {
#pragma unroll
  for (int m = N; m < 64; m <<= 1) x += shfl_xor(x, m);
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Keys [0, limit) that query row i of a sequence may see under causal
// masking.  pos0 is the key position of row 0: seq_len - Sq (bottom-right
// alignment) or the sequence's prefix offset.  64-bit arithmetic, so any int32
// offset is safe; the limit is clamped to [0, seq_len].
__device__ __forceinline__ int causal_key_limit(int seq_len, int64_t pos0, int i) {
  const int64_t l = pos0 + i + 1;
  return l < 0 ? 0 : (l > seq_len ? seq_len : static_cast<int>(l));
}

// Key position of row 0 of sequence b (see causal_key_limit).
__device__ __forceinline__ int64_t causal_row0(const int32_t* prefix_offset, int b, int seq_len,
                                               int seq_q) {
  return prefix_offset != nullptr ? static_cast<int64_t>(prefix_offset[b])
                                  : static_cast<int64_t>(seq_len) - seq_q;
}

}  // namespace pa
