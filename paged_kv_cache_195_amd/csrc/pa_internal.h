// Internal interface between the C-ABI host code and the kernel launchers.
// Host and device code both include this file; it holds no device code.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stddef.h>
#include <stdint.h>

#include "fast_div.h"
#include "pa.h"

namespace pa {

// Everything one attention launch needs.  Pointers are device memory.
struct AttnParams {
  const void* q;               // [B, Sq, Hq, D]
  const void* k;               // [num_pages, page_size, Hkv, D]
  const void* v;               // [num_pages, page_size, Hkv, Dv]
  const int32_t* block_table;  // row b at block_table + b * bt_stride
  const int32_t* seq_lens;     // [B]
  const int32_t* prefix_offset;  // [B] key position of each sequence's row 0, or nullptr
  const float* k_scale;        // [num_pages, Hkv] for 8-bit caches, else nullptr
  const float* v_scale;        // [num_pages, Hkv] for 8-bit caches, else nullptr
  void* out;                   // [B, Sq, Hq, Dv]           (num_splits == 1)
  float* lse;                  // [B, Sq, Hq] or nullptr     (num_splits == 1)
  float* part_out;             // [B*Sq*Hq, S, Dv]           (num_splits > 1)
  float* part_lse;             // [B*Sq*Hq, S]               (num_splits > 1)
  int64_t bt_stride;
  int32_t table_width;         // W: slots of each block-table row (>= every sequence's page count)
  int32_t seq_q;
  int32_t num_q_heads;
  int32_t num_kv_heads;
  int32_t group;               // Hq / Hkv
  DivMagic group_div;          // division by group as a multiply-high (fast_div.h)
  int32_t rows_per_kvh;        // Sq * group: query rows that share one kv head
  int32_t num_splits;          // S >= 1
  int32_t causal;              // 1 also when prefix_offset is set (prefix-causal is causal)
  int32_t heads_per_wg;        // kv heads one workgroup serves (divides Hkv and its wave count)
  float scale_log2;            // scale * log2(e): scores are kept in base 2
};

// Launch shape chosen on the host.
struct AttnPlan {
  bool mfma;         // matrix-core kernel (16-bit and 8-bit caches)
  bool prefill;      // a shared-tile kernel (kPrefillMinRows rows per kv head and more)
  int rows_per_wg;   // MR: query rows (position, head) per kv head in one workgroup
  int row_groups;    // ceil(rows_per_kvh / MR)
  int num_splits;    // S
  int waves;         // waves per workgroup
  int heads_per_wg;  // kv heads per workgroup
};

// Launch shape of the vector-ALU kernel for each (element bytes, D, page
// size, MR).  Kernels whose working set fits 128 VGPRs (at most 4 KiB of K
// per page and kv head, MR <= 4) run 16 waves (one 1024-thread workgroup
// fills a compute unit) and rely on occupancy for loads in flight; larger
// ones run 8 waves.  Measured on the Llama-3-8B decode shape (bf16, when that
// shape still ran on this kernel), a deeper per-wave register ring
// (pages_ahead > 0) gained nothing over occupancy and pushed the larger
// kernels into spills, so every configuration streams one page at a time.
struct ValuConfig {
  int waves;
  int pages_ahead;
};

constexpr ValuConfig valu_config(int elem_bytes, int head_dim, int page_size, int rows_per_wg) {
  return (page_size * head_dim * elem_bytes / 1024 <= 4 && rows_per_wg <= 4) ? ValuConfig{16, 0}
                                                                              : ValuConfig{8, 0};
}
// Most rows per workgroup of the vector-ALU kernel: 8, but 4 for f32 at D = 128
// with 32-token pages, whose 8-row form needs more than 256 VGPRs (a page of K
// and V is 128 registers per lane there) and spilled 193 of them; two 4-row
// groups read the pages twice instead.
constexpr int valu_max_rows(int elem_bytes, int head_dim, int page_size) {
  return (elem_bytes == 4 && head_dim == 128 && page_size == 32) ? 4 : 8;
}

// The matrix-core kernel: 16 rows per kv head and workgroup, 8 waves.  It
// serves every 16-bit and 8-bit cache (the shared-tile prefill kernel aside):
// even at 1, 2 or 4 query rows per kv head, where most of its 16-row tile is
// padding, it streams faster than the vector-ALU kernel (bf16 decode, B=256,
// Skv 4096, 8 kv heads: 620 against 650-685 us at G = 4, 622 against 639 us
// at G = 1), which is left to f32 caches.
//
// Waves per workgroup: 8, or 4 for 16-bit caches whose kv-head count is not a
// multiple of 8.  The fastest layout gives each kv head of a page one wave and
// lets one workgroup cover all kv heads of its pages (Qwen3-235B decode,
// Hkv = 4: 632 against 638 us; Hkv = 4, G = 4: 623 against 633 us); at
// Hkv = 8 eight waves win (Llama-3-8B decode 621 against 627 us).  8-bit
// caches keep 8 (the int8 step ran 352 against 371 us with 4).  Both widths
// run 8 resident waves per compute unit: more resident waves stream slower.
constexpr int kMfmaWaves = 8;
constexpr int kMfmaWavesNarrow = 4;
// LDS a 4-wave workgroup holds (static plus reserved): more than a third of a
// compute unit's 160 KiB, so at most two are resident.
constexpr int kMfmaLdsPerNarrowWg = 56 * 1024;
// The shared-tile prefill kernels: kPrefillRowBlocks blocks of 16 rows per
// wave, one kv head per workgroup; D = 64 takes the single-team kernel with
// kPrefillWaves waves, D = 128 the two-team kernel with kPrefillTeamWaves.
constexpr int kPrefillWaves = 4;
constexpr int kPrefillTeamWaves = 8;
constexpr int kPrefillRowBlocks = 2;
constexpr int prefill_waves(int head_dim) {
  return head_dim == 128 ? kPrefillTeamWaves : kPrefillWaves;
}
// Query rows per kv head from which the shared-tile kernels take over from
// the 16-row matrix-core kernel, which reads a kv head's pages once per 16
// rows.  16-bit caches as soon as a kv head has more than one 16-row block
// (graph-replayed bf16, B=256, L=4096: GQA 24/1 168 -> 140 us, GQA 32/1 167
// -> 140 us, GQA 40/2 324 -> 265 us; 5 new queries at GQA 32/8 21.7 -> 18.2
// us); 8-bit codes from 64 (their decoding makes the shared tile's mostly
// idle rows cost more: GQA 32/1 int8 107 us on the 16-row kernel, 149 us
// shared).
constexpr int kPrefillMinRows = 17;
// Decode with 17 to 32 rows per kv head runs two 16-row blocks per wave on the
// matrix-core kernel instead (attn_mfma_rows.h), the shared-tile kernels from
// 33, when the batch holds at least kDecodeRowsMinUnits (sequence, kv head)
// pairs; smaller batches, which split each sequence many ways, run faster on
// the shared-tile kernels.
constexpr int kDecodeMinSharedRows = 33;
constexpr int kDecodeRowsMinUnits = 128;
constexpr int kPrefillMinRowsQuant = 64;

enum DType { kF32 = 0, kF16 = 1, kBF16 = 2, kI8 = 3, kFp8E4M3 = 4 };

// Grid = (S * row_groups, Hkv, B); returns a hipError_t.
hipError_t launch_attn_valu_f32(const AttnParams& p, const AttnPlan& plan, int head_dim,
                                int page_size, int batch, hipStream_t stream);


hipError_t launch_attn_mfma_f16(const AttnParams& p, const AttnPlan& plan, int head_dim,
                                int page_size, int batch, hipStream_t stream);
hipError_t launch_attn_mfma_bf16(const AttnParams& p, const AttnPlan& plan, int head_dim,
                                 int page_size, int batch, hipStream_t stream);

// Page-id range check: writes result[1 + b] = seq_lens[b] when sequence b's
// length lies in [0, width * page_size] and its first ceil(len / page_size)
// ids lie in [0, num_pages), else 0; then result[0] = the smallest failing b,
// or -1.  Two launches on `stream`.
hipError_t launch_page_check(const int32_t* block_table, int64_t bt_stride,
                             const int32_t* seq_lens, int batch, int width, int page_size,
                             int64_t num_pages, int32_t* result, hipStream_t stream);

// The MFMA kernel over 8-bit K/V codes (kv_dtype PA_I8 or PA_FP8_E4M3), q and
// out of the named type; D in {64, 128}.
hipError_t launch_attn_mfma_q_f16(const AttnParams& p, const AttnPlan& plan, int kv_dtype,
                                  int head_dim, int page_size, int batch, hipStream_t stream);
hipError_t launch_attn_mfma_q_bf16(const AttnParams& p, const AttnPlan& plan, int kv_dtype,
                                   int head_dim, int page_size, int batch, hipStream_t stream);

// Validation, planning and launches of one pa_decode / pa_prefill call (with
// the optional inputs of pa_options, which may be null); the split partials go
// to `workspace`.  Returns a pa_status.
int run_attention(const pa_shape* s, const pa_options* opt, bool decode, const void* q,
                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                  const int32_t* seq_lens, float scale, int causal, int num_splits, void* out,
                  float* lse, void* workspace, size_t workspace_bytes, void* stream);

hipError_t launch_combine(int dtype, int rows, int num_splits, int head_dim_v,
                          const float* part_out, const float* part_lse, void* out, float* lse,
                          hipStream_t stream);

}  // namespace pa
