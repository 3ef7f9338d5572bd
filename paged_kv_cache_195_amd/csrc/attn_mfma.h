// Split-KV paged attention on the matrix cores (gfx950 MFMA), for 16-bit and
// 8-bit caches: every decode, whatever the group size, and prefill with fewer
// than 64 query rows per kv head (the shared-tile prefill kernel takes more).
//
// A wave owns 16 query rows of one kv head (a row is a (query position, head
// of the group) pair) and streams its kv head's pages in 16-token tiles:
//
//   S^T[16 tokens x 16 rows] = K_tile[16 x D] . Q^T[D x 16]
//       D/32 v_mfma_f32_16x16x32 steps; K is the A operand (lane l: token
//       l%16, 8 dims), Q^T the B operand, loaded once.
//   O[16 rows x D] += P[16 x 16 tokens] . V_tile[16 x D]
//       D/16 v_mfma_f32_16x16x16 blocks.  The S^T accumulator layout (lane l
//       holds row l%16, tokens 4*(l/16)..+3) is exactly the A-operand layout
//       of this product, so P needs no data movement.  V is read back from
//       LDS with ds_read_b64_tr_b16, which returns four consecutive tokens of
//       one dimension per lane: the B-operand layout.
//
// K and V tiles are loaded from HBM as whole rows (each wave load covers
// 512/D full rows of D*2 bytes, the pattern that streams fastest) and staged
// in the wave's own LDS rows; the operand layouts are read from there.  Inside
// a row, 16-byte chunk c sits at position c ^ (2 r mod chunks), an XOR swizzle
// that keeps the row writes, the K operand reads and the transposing V reads
// free of bank conflicts.
//
// P is split into a high and a low 16-bit part (P = P_hi + P_lo, both fed to
// the MFMA), so the weights keep about 16 significant bits instead of the 8
// of a single bfloat16 rounding.
//
// Softmax state per row: ref (reference max of scaled scores, -inf before the
// first valid key), msub (ref, or 0 while ref is -inf, so -inf - (-inf) never
// forms), l (sum of weights, per lane over its tokens) and the O accumulator,
// relative to msub.  ref is raised only when a tile's max exceeds it by more
// than kSlack (log2 units) -- a wave-uniform branch -- so the rescale of O is
// rare.  Guards and split ranges follow rocMLIR "Fix split-kv attention
// masking and sweep RMS" (Technical Details): fully masked splits contribute
// nothing and a zero row sum stores (0, -inf).  V rows of tokens past the
// sequence length are zeroed in LDS, so NaN in a last page's tail never meets
// a zero weight in the MFMA.
//
// Quantized caches (8-bit codes, one float32 scale per (page, kv head)): each
// lane loads 16 codes of a row and decodes them exactly to the 16-bit operand
// type (int8: one SDWA convert to float per code, then the top halves or a
// round-toward-zero pack, exact since a code has at most 8 significant bits;
// fp8 E4M3: one gfx950 scaled conversion per two codes, straight to the
// operand type, which decodes the OCP format).  The staged rows then feed the same MFMA steps.  The K scale
// multiplies the tile's scores; the V scale multiplies the tile's P.V product
// before it is added to O (with bf16 operands it folds into the weights
// instead), so a scale of any sign or size costs no precision.
#pragma once

#include "device_common.h"
#include "pa_internal.h"
#include "page_table.h"

// Tiles in flight ahead of the compute, per wave, for 8-bit caches (a
// compile-time tuning constant; 16-bit caches run one tile ahead).
#ifndef PA_QUANT_AHEAD
#define PA_QUANT_AHEAD 3
#endif

namespace pa {

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2_v __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef __attribute__((address_space(3))) char lds_char;

// Element kind of the K/V caches: the operand type itself, or 8-bit codes.
struct KvSame {};
struct KvI8 {};
struct KvFp8 {};

template <typename KV>
struct KvTraits {
  static constexpr bool quant = true;
};
template <>
struct KvTraits<KvSame> {
  static constexpr bool quant = false;
};

// Four codes of one 32-bit word as floats (exact).
__device__ __forceinline__ void decode4(KvI8, uint32_t w, float* f) {
  f[0] = static_cast<float>(static_cast<int8_t>(w & 0xffu));
  f[1] = static_cast<float>(static_cast<int8_t>((w >> 8) & 0xffu));
  f[2] = static_cast<float>(static_cast<int8_t>((w >> 16) & 0xffu));
  f[3] = static_cast<float>(static_cast<int8_t>(w >> 24));
}
__device__ __forceinline__ void decode4(KvFp8, uint32_t w, float* f) {
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(w), true);
  f[0] = lo[0];
  f[1] = lo[1];
  f[2] = hi[0];
  f[3] = hi[1];
}

template <typename T>
struct Mfma;

template <>
struct Mfma<bf16_t> {
  // acc += A[16x32] . B[32x16]; operands are 8 packed bf16 (one u32x4)
  static __device__ __forceinline__ f32x4 k32(const u32x4& a, const u32x4& b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), acc, 0, 0, 0);
  }
  // acc += A[16x16] . B[16x16]; operands are 4 packed bf16
  static __device__ __forceinline__ f32x4 k16(s16x4 a, s16x4 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
  }
  // Two finite weights a, b (of either sign) as packed high and low parts:
  // hi = the top 16 bits of each (exact as floats), lo = bf16(p - hi) rounded
  // to nearest even, so hi + lo keeps about 16 significant bits.
  static __device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const uint32_t ua = __builtin_bit_cast(uint32_t, a), ub = __builtin_bit_cast(uint32_t, b);
    hi = __builtin_amdgcn_perm(ub, ua, 0x07060302u);
    const f32x2 rest = {a - __builtin_bit_cast(float, ua & 0xffff0000u),
                        b - __builtin_bit_cast(float, ub & 0xffff0000u)};
    lo = __builtin_bit_cast(uint32_t, __builtin_convertvector(rest, bf16x2_v));
  }
  static constexpr uint32_t kOnes = 0x3f803f80u;  // two packed 1.0
  // Two floats with at most 8 significant bits as packed bf16: their top
  // halves (exact).
  static __device__ __forceinline__ uint32_t pack_exact(float a, float b) {
    return __builtin_amdgcn_perm(__builtin_bit_cast(uint32_t, b), __builtin_bit_cast(uint32_t, a),
                                 0x07060302u);
  }
};

template <>
struct Mfma<f16_t> {
  static __device__ __forceinline__ f32x4 k32(const u32x4& a, const u32x4& b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), acc, 0, 0, 0);
  }
  static __device__ __forceinline__ f32x4 k16(s16x4 a, s16x4 b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4_t, a),
                                                 __builtin_bit_cast(f16x4_t, b), acc, 0, 0, 0);
  }
  // hi = each weight rounded toward zero to f16, lo = the rest, also
  // rounded toward zero (weights are at most 2^8, well inside f16 range).
  static __device__ __forceinline__ void split2(float a, float b, uint32_t& hi, uint32_t& lo) {
    const f16x2_t h = __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(a, b));
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a - static_cast<float>(h[0]),
                                                                 b - static_cast<float>(h[1])));
  }
  static constexpr uint32_t kOnes = 0x3c003c00u;  // two packed 1.0
  // Two floats that f16 represents exactly (8-bit code values) as packed f16.
  static __device__ __forceinline__ uint32_t pack_exact(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
  }
};

// Two fp8 E4M3 codes (the low or the high half of a word) as a packed pair of
// the operand type, in one gfx950 scaled conversion with scale 1 (exact; all
// 256 codes were checked against the format on the GPU).
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8_pair(bf16_t, uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(w, 1.0f, kHigh));
}
template <bool kHigh>
__device__ __forceinline__ uint32_t fp8_pair(f16_t, uint32_t w) {
  return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, kHigh));
}

// 16 codes (one 16-byte load) as two 16-byte chunks of 8 operand values.
template <typename T, typename KV>
__device__ __forceinline__ void widen16(const u32x4& w, u32x4& lo, u32x4& hi) {
  uint32_t packed[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if constexpr (__is_same(KV, KvFp8)) {
      packed[2 * i] = fp8_pair<false>(T{}, word(w, i));
      packed[2 * i + 1] = fp8_pair<true>(T{}, word(w, i));
    } else {
      float f[4];
      decode4(KV{}, word(w, i), f);
      packed[2 * i] = Mfma<T>::pack_exact(f[0], f[1]);
      packed[2 * i + 1] = Mfma<T>::pack_exact(f[2], f[3]);
    }
  }
  lo = u32x4{packed[0], packed[1], packed[2], packed[3]};
  hi = u32x4{packed[4], packed[5], packed[6], packed[7]};
}

// The end of the matrix-core decode kernels: merges the partial softmax states
// of the waves that share a kv head, then writes the rows (out and lse, or the
// split partials).  Wave w left at smem + w * kPerWave: o [kRows][D] (f32,
// unnormalised), then ref [kRows] (running maximum, base 2) and l [kRows] (row
// sum).  Waves hg * WPH .. hg * WPH + WPH - 1 serve the workgroup's kv head hg.
// Call after a workgroup barrier that follows those writes.
//
// Two passes.  First one thread per (kv head, row) forms each wave's weight
// 2^(ref_w - max) and the row's total sum, writes the row's lse, and leaves the
// weights in the l slots and the total in the first wave's ref slot.  Then
// one thread per output element sums the weighted o values of the waves.  The
// weights are formed once per row, not once per element, and the wave count
// is a compile-time constant, so each pass issues all its LDS reads of an
// element at once (one round trip); with a run-time wave count every wave's
// reads were a separate round trip.
template <typename T, int D, int kRows, int NW, int kPerWave, int WPH>
__device__ __forceinline__ void merge_wave_states_n(const AttnParams& p, char* smem, int kpw,
                                                    int rg, int b, int split) {
  const int S = p.num_splits;
  const int G = p.group;
  const int Sq = p.seq_q;
  const int Hq = p.num_q_heads;
  auto wave_f = [&](int w) __attribute__((always_inline)) {
    return reinterpret_cast<float*>(smem + w * kPerWave);
  };
  auto row_id = [&](int hg, int r_lin) __attribute__((always_inline)) {
    const int i = r_lin / G;
    return (b * Sq + i) * Hq + (blockIdx.y * kpw + hg) * G + (r_lin - i * G);
  };
  for (int t = threadIdx.x; t < kpw * kRows; t += NW * 64) {
    const int hg = t / kRows;
    const int r = t - hg * kRows;
    const int r_lin = rg * kRows + r;
    if (r_lin >= p.rows_per_kvh) continue;
    float wr[WPH], wl[WPH];
#pragma unroll
    for (int k = 0; k < WPH; ++k) {
      wr[k] = wave_f(hg * WPH + k)[kRows * D + r];
      wl[k] = wave_f(hg * WPH + k)[kRows * D + kRows + r];
    }
    float mx = kNegInf;
#pragma unroll
    for (int k = 0; k < WPH; ++k) mx = __builtin_fmaxf(mx, wr[k]);
    const float wsub = mx == kNegInf ? 0.f : mx;
    float tot = 0.f;
#pragma unroll
    for (int k = 0; k < WPH; ++k) {
      // a wave with no valid key for this row has ref = -inf and l = 0, o = 0
      const float f = wr[k] == kNegInf ? 0.f : fast_exp2(wr[k] - wsub);
      tot += f * wl[k];
      wave_f(hg * WPH + k)[kRows * D + kRows + r] = f;
    }
    wave_f(hg * WPH)[kRows * D + r] = tot;
    const float lse = tot > 0.f ? (mx + log2f(tot)) * kLn2 : kNegInf;
    const int rid = row_id(hg, r_lin);
    if (S == 1) {
      if (p.lse != nullptr) p.lse[rid] = lse;
    } else {
      p.part_lse[static_cast<int64_t>(rid) * S + split] = lse;
    }
  }
  __syncthreads();
  // four consecutive elements of a row per thread: one 16-byte LDS read per
  // wave, and one 8-byte store when the output allows it
  const bool out8 = (reinterpret_cast<uintptr_t>(p.out) & 7u) == 0;
  for (int idx = threadIdx.x; idx < kpw * kRows * (D / 4); idx += NW * 64) {
    const int e0 = 4 * idx;
    const int hg = e0 / (kRows * D);
    const int r = (e0 / D) % kRows;
    const int d0 = e0 % D;
    const int r_lin = rg * kRows + r;
    if (r_lin >= p.rows_per_kvh) continue;
    const float tot = wave_f(hg * WPH)[kRows * D + r];
    float f[WPH];
    f32x4 o[WPH];
#pragma unroll
    for (int k = 0; k < WPH; ++k) {
      f[k] = wave_f(hg * WPH + k)[kRows * D + kRows + r];
      o[k] = *reinterpret_cast<const f32x4*>(wave_f(hg * WPH + k) + r * D + d0);
    }
    f32x4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < WPH; ++k)
#pragma unroll
      for (int c = 0; c < 4; ++c) a[c] += f[k] * o[k][c];
    f32x4 out;
#pragma unroll
    for (int c = 0; c < 4; ++c) out[c] = tot > 0.f ? a[c] / tot : 0.f;
    const int rid = row_id(hg, r_lin);
    if (S == 1) {
      T* dst = static_cast<T*>(p.out) + static_cast<int64_t>(rid) * D + d0;
      if (out8) {
        uint32_t w[2];
#pragma unroll
        for (int c = 0; c < 2; ++c)
          w[c] = static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_float<T>(out[2 * c]))) |
                 (static_cast<uint32_t>(__builtin_bit_cast(uint16_t, from_float<T>(out[2 * c + 1])))
                  << 16);
        *reinterpret_cast<uint2*>(dst) = make_uint2(w[0], w[1]);
      } else {
#pragma unroll
        for (int c = 0; c < 4; ++c) dst[c] = from_float<T>(out[c]);
      }
    } else {
      *reinterpret_cast<f32x4*>(p.part_out + (static_cast<int64_t>(rid) * S + split) * D + d0) = out;
    }
  }
}

// kpw kv heads per workgroup, NW / kpw waves per head (1, 2, 4 or 8).
template <typename T, int D, int kRows, int NW, int kPerWave>
__device__ __forceinline__ void merge_wave_states(const AttnParams& p, char* smem, int kpw, int rg,
                                                  int b, int split) {
  const int wph = NW / kpw;
  if (wph == 1) {
    merge_wave_states_n<T, D, kRows, NW, kPerWave, 1>(p, smem, kpw, rg, b, split);
  } else if (wph == 2) {
    merge_wave_states_n<T, D, kRows, NW, kPerWave, 2>(p, smem, kpw, rg, b, split);
  } else if (wph == 4 || NW == 4) {
    merge_wave_states_n<T, D, kRows, NW, kPerWave, (NW < 4 ? NW : 4)>(p, smem, kpw, rg, b, split);
  } else {
    merge_wave_states_n<T, D, kRows, NW, kPerWave, NW>(p, smem, kpw, rg, b, split);
  }
}

// T: bf16_t or f16_t (q, out and the MFMA operands); KV: KvSame (caches of
// T) or KvI8 / KvFp8 (8-bit codes with p.k_scale / p.v_scale); D: head dim
// (= Dv, a multiple of 32; >= 64 for codes); PS: tokens per page (a multiple
// of 16); NW: waves per workgroup.  p.heads_per_wg kv heads per workgroup,
// NW / heads_per_wg waves per head; each workgroup covers 16 rows per kv head
// (row group rg = blockIdx.x / S).
// Static LDS of one workgroup: per wave, a K and a V tile of 16 staged rows,
// reused for the final merge.
template <int D, int NW>
constexpr int mfma_static_lds() {
  return NW * ((2 * 16 * D * 2) > (16 * D * 4 + 2 * 16 * 4) ? (2 * 16 * D * 2)
                                                            : (16 * D * 4 + 2 * 16 * 4));
}

template <typename T, typename KV, int D, int PS, int NW>
__global__ __launch_bounds__(NW * 64) void attn_mfma_kernel(const AttnParams p) {
  static_assert(D % 32 == 0 && PS % 16 == 0, "tile shape");
  constexpr bool kQuant = KvTraits<KV>::quant;
  constexpr int kKSteps = D / 32;         // 16x16x32 steps for q.k
  constexpr int kNBlocks = D / 16;        // 16-dim output blocks
  constexpr int kTiles = PS / 16;         // 16-token tiles per page
  constexpr int kRowBytes = D * 2;        // a staged row (operand type)
  constexpr int kCacheRowBytes = kQuant ? D : D * 2;  // a row in the cache
  constexpr float kSlack = 8.f;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int g = lane >> 4;   // 16-lane group
  const int li = lane & 15;  // index inside the group

  const int S = p.num_splits;
  const int split = blockIdx.x % S;
  const int rg = blockIdx.x / S;
  const int kpw = p.heads_per_wg;
  const int wph = NW / kpw;
  const int kg = wave / wph;
  const int sub = wave - kg * wph;
  const int kvh = blockIdx.y * kpw + kg;
  const int b = blockIdx.z;
  const int Hkv = p.num_kv_heads;
  const int G = p.group;
  const int Sq = p.seq_q;
  const int Hq = p.num_q_heads;

  const int seq_len = p.seq_lens[b];
  const int n_pages = (seq_len + PS - 1) / PS;
  const int64_t pos0 = causal_row0(p.prefix_offset, b, seq_len, Sq);

  // ---- this lane's row (row li of the 16) and the key limits of the group
  auto row_limit = [&](int r_lin) __attribute__((always_inline)) {
    return p.causal ? causal_key_limit(seq_len, pos0, r_lin / G) : seq_len;
  };
  const int my_r = rg * 16 + li;
  const bool my_valid = my_r < p.rows_per_kvh;
  // rows 0..15 of this group: limits are the same for every kv head
  int max_lim = 0, min_lim = 0x7fffffff;
  for (int r = 0; r < 16; ++r) {
    const int r_lin = rg * 16 + r;
    if (r_lin >= p.rows_per_kvh) break;
    const int l = row_limit(r_lin);
    max_lim = l > max_lim ? l : max_lim;
    min_lim = l < min_lim ? l : min_lim;
  }
  const int my_lim = my_valid ? row_limit(my_r) : max_lim;

  // Q^T as the B operand: lane l holds q[row li][32 s + 8 g .. +8]
  u32x4 qb[kKSteps];
  {
    const int i = my_r / G;
    const int h = kvh * G + (my_r - i * G);
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qb[s] = u32x4{0u, 0u, 0u, 0u};
    if (my_valid) {  // padding rows past the last row never touch q
      const T* qrow =
          static_cast<const T*>(p.q) + (static_cast<int64_t>(b * Sq + i) * Hq + h) * D;
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) qb[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * g);
    }
  }
  const float c = __builtin_fmaxf(__builtin_fabsf(p.scale_log2), 1.17549435e-38f);
  if (p.scale_log2 < 0.f) {
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) qb[s] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  // ---- split range (ceil-divided, clamped, cut at the last visible page)
  const int per = (n_pages + S - 1) / S;
  const int first = min(split * per, n_pages);
  int end = min(first + per, n_pages);
  end = min(end, (max_lim + PS - 1) / PS);

  PageTable pt;
  pt.row = p.block_table + static_cast<int64_t>(b) * p.bt_stride;
  pt.page_bytes = static_cast<int64_t>(PS) * Hkv * kCacheRowBytes;
  pt.n_pages = n_pages;

  // Whole-row loads: wave load j covers rows j * kRowsPerLoad .. +kRowsPerLoad
  // of the tile; lane l takes 16-byte chunk lc of row lr.
  constexpr int kChunks = D / 8;                      // 16-byte chunks per staged row
  constexpr int kCacheChunks = kCacheRowBytes / 16;   // 16-byte chunks per cache row
  constexpr int kRowsPerLoad = 64 / kCacheChunks;     // rows per wave load
  constexpr int kLoads = 16 / kRowsPerLoad;           // wave loads per tile
  static_assert(kRowsPerLoad <= 16 && 16 % kRowsPerLoad == 0, "whole rows per tile");
  const int lr = lane / kCacheChunks;
  const int lc = lane % kCacheChunks;
  const uint32_t lane_off = static_cast<uint32_t>((lr * Hkv + kvh) * kCacheRowBytes + 16 * lc);
  const uint32_t load_step = static_cast<uint32_t>(kRowsPerLoad * Hkv * kCacheRowBytes);
  const uint32_t tile_step = static_cast<uint32_t>(16 * Hkv * kCacheRowBytes);
  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);

  // LDS: per wave, a K tile and a V tile of 16 swizzled rows; reused for the
  // final merge
  constexpr int kTileLds = 2 * 16 * kRowBytes;
  constexpr int kMergeLds = 16 * D * 4 + 2 * 16 * 4;
  constexpr int kPerWave = kTileLds > kMergeLds ? kTileLds : kMergeLds;
  static_assert(NW * kPerWave == mfma_static_lds<D, NW>(), "LDS size");
  __shared__ __attribute__((aligned(16))) char smem[NW * kPerWave];
  char* my_lds = smem + wave * kPerWave;
  lds_char* my_lds3 = (lds_char*)(smem) + wave * kPerWave;
  char* lds_k = my_lds;
  char* lds_v = my_lds + 16 * kRowBytes;
  lds_char* lds_v3 = my_lds3 + 16 * kRowBytes;
  // byte offset in a tile of 16-byte chunk c of row r
  auto swz = [](int r, int c) __attribute__((always_inline)) { return r * kRowBytes + 16 * (c ^ ((2 * r) & (kChunks - 1))); };

  float ref = kNegInf, msub = 0.f, lsum = 0.f;
  f32x4 o[kNBlocks];
#pragma unroll
  for (int nb = 0; nb < kNBlocks; ++nb) o[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_tile = [&](int64_t base, int t, u32x4* kk, u32x4* vv) __attribute__((always_inline)) {
    const uint32_t off = lane_off + t * tile_step;
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      kk[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(kbase + base + off + j * load_step));
#pragma unroll
    for (int j = 0; j < kLoads; ++j)
      vv[j] = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(vbase + base + off + j * load_step));
  };

  auto consume_tile = [&](int tok0, const u32x4* kk, u32x4* vv, float ks, float vs)
                          __attribute__((always_inline)) {
    // stage K and V rows; V rows of tokens past the sequence become zero
    const bool tail = tok0 + 16 > min_lim;  // wave-uniform
#pragma unroll
    for (int j = 0; j < kLoads; ++j) {
      const int r = j * kRowsPerLoad + lr;
      u32x4 vrow = vv[j];
      if (tail && tok0 + r >= seq_len) vrow = u32x4{0u, 0u, 0u, 0u};
      if constexpr (kQuant) {
        u32x4 lo, hi;
        widen16<T, KV>(kk[j], lo, hi);
        *reinterpret_cast<u32x4*>(lds_k + swz(r, 2 * lc)) = lo;
        *reinterpret_cast<u32x4*>(lds_k + swz(r, 2 * lc + 1)) = hi;
        widen16<T, KV>(vrow, lo, hi);
        *reinterpret_cast<u32x4*>(lds_v + swz(r, 2 * lc)) = lo;
        *reinterpret_cast<u32x4*>(lds_v + swz(r, 2 * lc + 1)) = hi;
      } else {
        *reinterpret_cast<u32x4*>(lds_k + swz(r, lc)) = kk[j];
        *reinterpret_cast<u32x4*>(lds_v + swz(r, lc)) = vrow;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // S^T: lane holds S[row li][token tok0 + 4 g + e]
    f32x4 sacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const u32x4 ka = *reinterpret_cast<const u32x4*>(lds_k + swz(li, 4 * s + g));
      sacc = Mfma<T>::k32(ka, qb[s], sacc);
    }
    float x[4] = {sacc[0], sacc[1], sacc[2], sacc[3]};
    if constexpr (kQuant) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] *= ks;
    }
    if (tail) {
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = tok0 + 4 * g + e < my_lim ? x[e] : kNegInf;
    }

    float tmax = __builtin_fmaxf(__builtin_fmaxf(x[0], x[1]), __builtin_fmaxf(x[2], x[3]));
    const bool raise = tmax * c > ref + kSlack;
    if (__builtin_amdgcn_ballot_w64(raise) != 0) {  // wave-uniform
      float rmax = __builtin_fmaxf(tmax, shfl_xor(tmax, 16));
      rmax = __builtin_fmaxf(rmax, shfl_xor(rmax, 32));  // max of row li over the tile
      const float nref = __builtin_fmaxf(ref, rmax * c);
      const float nsub = nref == kNegInf ? 0.f : nref;
      const float alpha = fast_exp2(msub - nsub);
      ref = nref;
      msub = nsub;
      lsum *= alpha;
      // O rows 4 g + e need the factor of those rows, held by lanes 4 g + e
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float ae = __builtin_bit_cast(
            float, __builtin_amdgcn_ds_bpermute((4 * g + e) << 2, __builtin_bit_cast(int, alpha)));
#pragma unroll
        for (int nb = 0; nb < kNBlocks; ++nb) o[nb][e] *= ae;
      }
    }

    // weights, split into high and low 16-bit parts.  For 8-bit caches with
    // bf16 operands the V scale folds into the weights (bf16 keeps float's
    // exponent range and the split keeps the sign); f16 weights could overflow,
    // so there the scale multiplies each tile's P.V product instead.
    constexpr bool kFoldV = kQuant && __is_same(T, bf16_t);
    float pe[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pe[e] = fast_exp2(__builtin_fmaf(x[e], c, -msub));  // x = -inf gives 0
      lsum += pe[e];
      if constexpr (kFoldV) pe[e] *= vs;
    }
    uint32_t h01, l01, h23, l23;
    Mfma<T>::split2(pe[0], pe[1], h01, l01);
    Mfma<T>::split2(pe[2], pe[3], h23, l23);
    const s16x4 phi = __builtin_bit_cast(s16x4, uint64_t(h01) | (uint64_t(h23) << 32));
    const s16x4 plo = __builtin_bit_cast(s16x4, uint64_t(l01) | (uint64_t(l23) << 32));

    // B operand for block nb: tokens 4 g .. 4 g + 3 of dimension 16 nb + li;
    // source lane li points at row 4 g + li / 4, dimensions 16 nb + 4 (li % 4) ..
    const int tr_row = 4 * g + (li >> 2);
#pragma unroll
    for (int nb = 0; nb < kNBlocks; ++nb) {
      const int chunk = 2 * nb + ((li & 3) >> 1);
      const s16x4 vb = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (lds_s16x4*)(lds_v3 + swz(tr_row, chunk) + 8 * (li & 1)));
      if constexpr (kQuant && !kFoldV) {
        f32x4 t = Mfma<T>::k16(phi, vb, f32x4{0.f, 0.f, 0.f, 0.f});
        t = Mfma<T>::k16(plo, vb, t);
#pragma unroll
        for (int e = 0; e < 4; ++e) o[nb][e] = __builtin_fmaf(vs, t[e], o[nb][e]);
      } else {
        o[nb] = Mfma<T>::k16(phi, vb, o[nb]);
        o[nb] = Mfma<T>::k16(plo, vb, o[nb]);
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  };

  // Scales of a page: [page][kv head], read as wave-uniform scalars.
  auto page_scales = [&](uint32_t pid, float& ks, float& vs) __attribute__((always_inline)) {
    if constexpr (kQuant) {
      const int64_t si = static_cast<int64_t>(pid) * Hkv + kvh;
      ks = p.k_scale[si];
      vs = p.v_scale[si];
    }
  };
  if constexpr (!kQuant) {
    // ---- stream, 16-bit caches: the wave takes pages first + sub,
    // first + sub + wph, ...; each page is kTiles tiles; the next tile's
    // loads are issued before the current tile is computed.
    int slot = first + sub;
    if (slot < end) {
      int64_t base = pt.base(slot);
      u32x4 kc[kLoads], vc[kLoads];
      int t = 0;
      load_tile(base, 0, kc, vc);
      while (true) {
        const int tok0 = slot * PS + 16 * t;
        int nslot = slot, nt = t + 1;
        if (nt == kTiles) {
          nslot = slot + wph;
          nt = 0;
        }
        const bool more = nslot < end;
        int64_t nbase = base;
        u32x4 kn[kLoads], vn[kLoads];
        if (more) {
          if (nslot != slot) nbase = pt.base(nslot);
          load_tile(nbase, nt, kn, vn);
        }
        consume_tile(tok0, kc, vc, 1.f, 1.f);
        if (!more) break;
#pragma unroll
        for (int s = 0; s < kLoads; ++s) {
          kc[s] = kn[s];
          vc[s] = vn[s];
        }
        slot = nslot;
        t = nt;
        base = nbase;
      }
    }
  } else {
    // ---- stream, 8-bit caches: the same tile order (tile k is tile
    // k % kTiles of the page in slot first + sub + (k / kTiles) * wph), with
    // loads kAhead tiles ahead of the compute through a ring of kAhead + 1
    // register buffers indexed by compile-time stages.  An 8-bit tile holds
    // half the bytes of a 16-bit one, so more of them stay in flight (one
    // ahead: 452 us, three ahead: 356 us on the Llama-3-8B decode shape).
    constexpr int kAhead = PA_QUANT_AHEAD;
    constexpr int kRing = kAhead + 1;
    const int my_first = first + sub;
    const int my_pages = my_first < end ? (end - my_first + wph - 1) / wph : 0;
    const int n_tiles = my_pages * kTiles;
    u32x4 kr[kRing][kLoads], vr[kRing][kLoads];
    float rks[kRing], rvs[kRing];
    int64_t cur_base = 0;
    float cur_ks = 1.f, cur_vs = 1.f;
    // issue the loads of tile k into one ring stage
    auto issue = [&](int k, u32x4* kk, u32x4* vv, float& ks, float& vs)
                     __attribute__((always_inline)) {
      const int pg = k / kTiles;
      const int t = k - pg * kTiles;
      if (t == 0) {
        const uint32_t pid = pt.id(my_first + pg * wph);
        cur_base = pt.base_of(pid);
        page_scales(pid, cur_ks, cur_vs);
      }
      ks = cur_ks;
      vs = cur_vs;
      load_tile(cur_base, t, kk, vv);
    };
#pragma unroll
    for (int st = 0; st < kAhead; ++st)
      if (st < n_tiles) issue(st, kr[st], vr[st], rks[st], rvs[st]);
    for (int k0 = 0; k0 < n_tiles; k0 += kRing) {
#pragma unroll
      for (int st = 0; st < kRing; ++st) {
        const int k = k0 + st;
        if (k < n_tiles) {  // wave-uniform
          const int ns = (st + kAhead) % kRing;
          if (k + kAhead < n_tiles) issue(k + kAhead, kr[ns], vr[ns], rks[ns], rvs[ns]);
          const int pg = k / kTiles;
          const int tok0 = (my_first + pg * wph) * PS + 16 * (k - pg * kTiles);
          consume_tile(tok0, kr[st], vr[st], rks[st], rvs[st]);
        }
      }
    }
  }

  // ---- finish this wave: row sums over the four token groups
  lsum += shfl_xor(lsum, 16);
  lsum += shfl_xor(lsum, 32);

  // ---- merge the waves of each kv head through LDS, then write
  __syncthreads();  // every wave is done with its V tiles
  float* mo = reinterpret_cast<float*>(my_lds);  // [16 rows][D]
  float* mref = mo + 16 * D;                     // [16]
  float* ml = mref + 16;                         // [16]
#pragma unroll
  for (int nb = 0; nb < kNBlocks; ++nb)
#pragma unroll
    for (int e = 0; e < 4; ++e) mo[(4 * g + e) * D + 16 * nb + li] = o[nb][e];
  if (g == 0) {
    mref[li] = ref;
    ml[li] = lsum;
  }
  __syncthreads();

  merge_wave_states<T, D, 16, NW, kPerWave>(p, smem, kpw, rg, b, split);
}

}  // namespace pa
