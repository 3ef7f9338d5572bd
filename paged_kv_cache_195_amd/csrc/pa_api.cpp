// Host side of the C ABI declared in include/pa.h: argument validation,
// split planning, workspace layout and kernel dispatch.  Nothing here touches
// the GPU until every check has passed; nothing is allocated.
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "pa.h"
#include "pa_internal.h"

namespace {

// The automatic split count aims at one workgroup per compute unit of an
// MI355X (256 CUs).  A split keeps at least kMinAutoPagesPerSplit pages of the
// table width: with fewer, the per-split start-up and the partials' write and
// combine cost more than the extra workgroups gain (bf16 decode, B=8, 63-slot
// table, lengths 17..1000: S=8 23.7 us, S=16 24.8 us, S=32 30.4 us).
constexpr int64_t kTargetWorkgroups = 256;
constexpr int kMaxSplits = 256;
constexpr int kMaxAutoSplits = 64;
constexpr int64_t kMinAutoPagesPerSplit = 8;
constexpr size_t kAlign = 256;

bool aligned16(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 15u) == 0; }
bool aligned4(const void* ptr) { return (reinterpret_cast<uintptr_t>(ptr) & 3u) == 0; }

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Rows per workgroup: the smallest power of two >= the rows that share a kv
// head, at most 8.
int rows_per_wg(int64_t rows_per_kvh) {
  int mr = 1;
  while (mr < rows_per_kvh && mr < 8) mr *= 2;
  return mr;
}

// Shape checks common to decode and prefill.  Returns PA_OK or an error.
int check_shape(const pa_shape* s, bool decode) {
  if (s == nullptr) return PA_EINVAL;
  if (s->dtype != PA_F32 && s->dtype != PA_F16 && s->dtype != PA_BF16) return PA_EINVAL;
  if (s->kv_dtype != 0 && s->kv_dtype != PA_I8 && s->kv_dtype != PA_FP8_E4M3) return PA_EINVAL;
  if (s->batch <= 0 || s->seq_q <= 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 ||
      s->head_dim_qk <= 0 || s->head_dim_v <= 0 || s->page_size <= 0 || s->num_pages <= 0 ||
      s->max_pages_per_seq <= 0)
    return PA_EINVAL;
  if (decode && s->seq_q != 1) return PA_EINVAL;
  if (s->num_q_heads % s->num_kv_heads != 0) return PA_EINVAL;
  if (s->block_table_stride < s->max_pages_per_seq) return PA_EINVAL;
  // W * page_size tokens must fit in int32 (sequence positions are int32).
  if (static_cast<int64_t>(s->max_pages_per_seq) * s->page_size > INT32_MAX) return PA_EINVAL;
  // Flat row indices B * Sq * Hq and element offsets inside q/out fit int32 / int64.
  const int64_t rows = static_cast<int64_t>(s->batch) * s->seq_q * s->num_q_heads;
  if (rows > INT32_MAX) return PA_EINVAL;
  // The byte size of one cache tensor must be representable.
  const int64_t elem = s->kv_dtype != 0 ? 1 : (s->dtype == PA_F32 ? 4 : 2);
  const int64_t page_bytes =
      static_cast<int64_t>(s->page_size) * s->num_kv_heads * s->head_dim_qk * elem;
  if (page_bytes > INT32_MAX) return PA_EINVAL;
  if (s->num_pages > INT64_MAX / page_bytes) return PA_EINVAL;
  // The last row's end, (B - 1) * stride + W, must be representable; tested
  // by division so the check itself cannot overflow.
  if (s->batch > 1 &&
      s->block_table_stride > (INT64_MAX - s->max_pages_per_seq) / (s->batch - 1))
    return PA_EINVAL;
  // Envelope of the compiled kernels (grid y = Hkv and z = B are 16-bit).
  if (s->batch > 65535 || s->num_kv_heads > 65535) return PA_EUNSUPPORTED;
  if (s->head_dim_qk != s->head_dim_v) return PA_EUNSUPPORTED;
  if ((s->head_dim_qk != 32 && s->head_dim_qk != 64 && s->head_dim_qk != 128) ||
      (s->page_size != 16 && s->page_size != 32))
    return PA_EUNSUPPORTED;
  // 8-bit caches: 16-bit queries, whole 16-byte code chunks per row lane
  if (s->kv_dtype != 0 && (s->dtype == PA_F32 || s->head_dim_qk == 32)) return PA_EUNSUPPORTED;
  return PA_OK;
}

pa::AttnPlan plan_for(const pa_shape* s, int num_splits) {
  pa::AttnPlan plan;
  const int group = s->num_q_heads / s->num_kv_heads;
  const int64_t rows_per_kvh = static_cast<int64_t>(s->seq_q) * group;
  const int elem = s->dtype == PA_F32 ? 4 : 2;
  const bool quant = s->kv_dtype != 0;
  // 16-bit and 8-bit caches take the matrix-core kernels (8-bit codes are
  // dequantized exactly to the operand type); f32 caches the vector-ALU one.
  // The shared-tile prefill kernels read 16-bit caches and, in the
  // single-team kernel, 8-bit codes.
  plan.mfma = quant || s->dtype != PA_F32;
  // Decode (one query row per sequence) with up to 32 rows per kv head stays
  // on the matrix-core kernel, two row blocks per wave from 17 rows, when the
  // batch has at least kDecodeRowsMinUnits (sequence, kv head) pairs (bf16,
  // L=4096: GQA 24/1 B=256 140 -> 95 us, B=128 67 -> 60 us, but B=64 36 ->
  // 39 us, against the shared-tile kernel); several query rows per sequence
  // take the shared-tile kernel from 17 rows (5 new queries at GQA 32/8: 18.2
  // against 21.3 us).
  const bool wide = static_cast<int64_t>(s->batch) * s->num_kv_heads >= pa::kDecodeRowsMinUnits;
  const int64_t min_rows =
      quant ? pa::kPrefillMinRowsQuant
            : (s->seq_q == 1 && wide ? pa::kDecodeMinSharedRows : pa::kPrefillMinRows);
  plan.prefill = plan.mfma && rows_per_kvh >= min_rows &&
                 (s->head_dim_qk == 64 || s->head_dim_qk == 128);
  if (plan.prefill) {
    plan.waves = quant ? pa::kPrefillWaves : pa::prefill_waves(s->head_dim_qk);
    plan.rows_per_wg = 16 * pa::kPrefillRowBlocks * plan.waves;
  } else if (plan.mfma) {
    // two 16-row blocks per wave when a kv head has more than 16 rows and the
    // batch is wide: its pages are then read once per 32 rows instead of once
    // per 16 (int8 GQA 32/1, B=256: 107 -> 71 us; at B=8, split 32 ways, one
    // block per wave stays faster: 15.8 against 22.9 us)
    plan.rows_per_wg = rows_per_kvh > 16 && wide ? 32 : 16;
    // 8 waves with two row blocks per wave whatever the kv-head count: the
    // 4-wave form holds 273 registers, one wave per SIMD (GQA 32/1, B=256:
    // 99.4 against 92.7 us with 8)
    plan.waves = (!quant && s->num_kv_heads % 8 != 0 && plan.rows_per_wg == 16)
                     ? pa::kMfmaWavesNarrow
                     : pa::kMfmaWaves;
  } else {
    plan.rows_per_wg = rows_per_wg(rows_per_kvh);
    const int max_rows = pa::valu_max_rows(elem, s->head_dim_qk, s->page_size);
    if (plan.rows_per_wg > max_rows) plan.rows_per_wg = max_rows;
    plan.waves = pa::valu_config(elem, s->head_dim_qk, s->page_size, plan.rows_per_wg).waves;
  }
  plan.row_groups = static_cast<int>((rows_per_kvh + plan.rows_per_wg - 1) / plan.rows_per_wg);
  // kv heads per workgroup: the largest divisor of Hkv that also divides the
  // wave count, at most 8 (a workgroup then reads most of each page it touches)
  plan.heads_per_wg = 1;
  for (int k = 8; k >= 1 && !plan.prefill; k /= 2) {
    if (plan.waves % k == 0 && s->num_kv_heads % k == 0) {
      plan.heads_per_wg = k;
      break;
    }
  }
  if (num_splits > 0) {
    plan.num_splits = num_splits;
  } else {
    auto units_for = [&](int kpw) {
      return static_cast<int64_t>(s->batch) * (s->num_kv_heads / kpw) * plan.row_groups;
    };
    const int64_t by_width =
        (s->max_pages_per_seq + kMinAutoPagesPerSplit - 1) / kMinAutoPagesPerSplit;
    auto splits_for = [&](int kpw) {
      const int64_t units = units_for(kpw);
      int64_t want = (kTargetWorkgroups + units - 1) / units;
      if (want > by_width) want = by_width;
      if (want > kMaxAutoSplits) want = kMaxAutoSplits;
      return want < 1 ? 1 : static_cast<int>(want);
    };
    // Below one workgroup per compute unit, fewer kv heads per matrix-core
    // workgroup (more waves on each head's pages) come first, down to two,
    // then splits: at equal workgroup counts fewer splits are faster (graph-
    // replayed bf16 decode, GQA 32/8: B=8, L=4096, S=32 x 8 heads 30.8 us,
    // S=8 x 2 heads 27.3 us; B=16 50.4 -> 46.9 us; GQA 64/8, B=4, L=8192
    // 37.3 -> 29.2 us)
    while (plan.mfma && !plan.prefill && plan.heads_per_wg > 2 &&
           units_for(plan.heads_per_wg) < kTargetWorkgroups)
      plan.heads_per_wg /= 2;
    plan.num_splits = splits_for(plan.heads_per_wg);
    // small batches, where the table width caps the splits: one kv head per
    // workgroup if the grid is still short (B=1, L=4096, GQA 32/8: 34 -> 25 us)
    while (plan.mfma && !plan.prefill && plan.heads_per_wg > 1 &&
           units_for(plan.heads_per_wg) * plan.num_splits < kTargetWorkgroups) {
      plan.heads_per_wg /= 2;
      plan.num_splits = splits_for(plan.heads_per_wg);
    }
    // From two kv heads per workgroup to one where that removes the combine
    // (S = 1 then fills the GPU: B=32, L=4096, GQA 32/8 86.4 -> 84.2 us) or
    // where the splits already have the fewest table slots allowed (the
    // ragged B=8 batch, S=8 -> 4: 11.8 -> 11.0 us); elsewhere one head per
    // workgroup doubles the splits and is 3-5% slower.
    if (plan.mfma && !plan.prefill && plan.heads_per_wg == 2 && plan.num_splits > 1 &&
        (units_for(1) >= kTargetWorkgroups || plan.num_splits == by_width)) {
      plan.heads_per_wg = 1;
      plan.num_splits = splits_for(1);
    }
  }
  return plan;
}

size_t workspace_for(const pa_shape* s, int splits) {
  if (splits <= 1) return 0;
  const size_t rows = static_cast<size_t>(s->batch) * s->seq_q * s->num_q_heads;
  const size_t part = rows * static_cast<size_t>(splits) * s->head_dim_v * sizeof(float);
  return align_up(part) + rows * static_cast<size_t>(splits) * sizeof(float);
}

int check_splits(int num_splits) {
  return (num_splits < 0 || num_splits > kMaxSplits) ? PA_EINVAL : PA_OK;
}

}  // namespace

namespace pa {

int run_attention(const pa_shape* s, const pa_options* opt, bool decode, const void* q,
                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                  const int32_t* seq_lens, float scale, int causal, int num_splits, void* out,
                  float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  int st = check_shape(s, decode);
  if (st != PA_OK) return st;
  st = check_splits(num_splits);
  if (st != PA_OK) return st;
  if (q == nullptr || k_cache == nullptr || v_cache == nullptr || block_table == nullptr ||
      seq_lens == nullptr || out == nullptr)
    return PA_EINVAL;
  if (!isfinite(scale)) return PA_EINVAL;
  // q, k_cache and v_cache are read in 16-byte chunks.
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache)) return PA_EINVAL;
  const int32_t* prefix_offset = opt != nullptr ? opt->prefix_offset : nullptr;
  int32_t* page_check = opt != nullptr ? opt->page_check : nullptr;
  const float* k_scale = opt != nullptr ? opt->k_scale : nullptr;
  const float* v_scale = opt != nullptr ? opt->v_scale : nullptr;
  if (!aligned4(prefix_offset) || !aligned4(page_check) || !aligned4(seq_lens) ||
      !aligned4(block_table) || !aligned4(k_scale) || !aligned4(v_scale))
    return PA_EINVAL;
  // scales come with 8-bit caches and only with them
  const bool quant = s->kv_dtype != 0;
  if (quant != (k_scale != nullptr) || quant != (v_scale != nullptr)) return PA_EINVAL;

  const pa::AttnPlan plan = plan_for(s, num_splits);
  const size_t need = workspace_for(s, plan.num_splits);
  if (need > 0 && (workspace == nullptr || workspace_bytes < need)) return PA_EWORKSPACE;

  const int group = s->num_q_heads / s->num_kv_heads;
  pa::AttnParams p;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.block_table = block_table;
  p.seq_lens = page_check != nullptr ? page_check + 1 : seq_lens;
  p.prefix_offset = prefix_offset;
  p.k_scale = k_scale;
  p.v_scale = v_scale;
  p.out = out;
  p.lse = lse;
  p.part_out = nullptr;
  p.part_lse = nullptr;
  if (plan.num_splits > 1) {
    const size_t rows = static_cast<size_t>(s->batch) * s->seq_q * s->num_q_heads;
    p.part_out = static_cast<float*>(workspace);
    p.part_lse = reinterpret_cast<float*>(
        static_cast<char*>(workspace) +
        align_up(rows * static_cast<size_t>(plan.num_splits) * s->head_dim_v * sizeof(float)));
  }
  p.bt_stride = s->block_table_stride;
  p.table_width = s->max_pages_per_seq;
  p.seq_q = s->seq_q;
  p.num_q_heads = s->num_q_heads;
  p.num_kv_heads = s->num_kv_heads;
  p.group = group;
  p.group_div = pa::div_magic(static_cast<uint32_t>(group));
  p.rows_per_kvh = s->seq_q * group;
  p.num_splits = plan.num_splits;
  p.causal = (causal != 0 || prefix_offset != nullptr) ? 1 : 0;
  p.heads_per_wg = plan.heads_per_wg;
  p.scale_log2 = scale * 1.4426950408889634f;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  hipError_t err;
  if (page_check != nullptr) {
    err = pa::launch_page_check(block_table, s->block_table_stride, seq_lens, s->batch,
                                s->max_pages_per_seq, s->page_size, s->num_pages, page_check, hs);
    if (err != hipSuccess) return PA_EHIP;
  }
  if (quant) {
    err = s->dtype == PA_F16
              ? pa::launch_attn_mfma_q_f16(p, plan, s->kv_dtype, s->head_dim_qk, s->page_size,
                                           s->batch, hs)
              : pa::launch_attn_mfma_q_bf16(p, plan, s->kv_dtype, s->head_dim_qk, s->page_size,
                                            s->batch, hs);
  } else if (plan.mfma) {
    err = s->dtype == PA_F16
              ? pa::launch_attn_mfma_f16(p, plan, s->head_dim_qk, s->page_size, s->batch, hs)
              : pa::launch_attn_mfma_bf16(p, plan, s->head_dim_qk, s->page_size, s->batch, hs);
  } else {
    err = pa::launch_attn_valu_f32(p, plan, s->head_dim_qk, s->page_size, s->batch, hs);
  }
  if (err != hipSuccess) return PA_EHIP;
  if (plan.num_splits > 1) {
    const int rows = s->batch * s->seq_q * s->num_q_heads;
    err = pa::launch_combine(s->dtype, rows, plan.num_splits, s->head_dim_v, p.part_out,
                             p.part_lse, out, lse, hs);
    if (err != hipSuccess) return PA_EHIP;
  }
  return PA_OK;
}

}  // namespace pa

extern "C" {

int pa_decode(const pa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
              const int32_t* block_table, const int32_t* seq_lens, float scale, int causal,
              int num_splits, void* out, float* lse, void* workspace, size_t workspace_bytes,
              void* stream) {
  return pa::run_attention(shape, nullptr, true, q, k_cache, v_cache, block_table, seq_lens, scale,
                       causal, num_splits, out, lse, workspace, workspace_bytes, stream);
}

int pa_prefill(const pa_shape* shape, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* block_table, const int32_t* seq_lens, float scale, int causal,
               int num_splits, void* out, float* lse, void* workspace, size_t workspace_bytes,
               void* stream) {
  return pa::run_attention(shape, nullptr, false, q, k_cache, v_cache, block_table, seq_lens, scale,
                       causal, num_splits, out, lse, workspace, workspace_bytes, stream);
}

int pa_decode_ex(const pa_shape* shape, const pa_options* options, const void* q,
                 const void* k_cache, const void* v_cache, const int32_t* block_table,
                 const int32_t* seq_lens, float scale, int causal, int num_splits, void* out,
                 float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return pa::run_attention(shape, options, true, q, k_cache, v_cache, block_table, seq_lens, scale,
                       causal, num_splits, out, lse, workspace, workspace_bytes, stream);
}

int pa_prefill_ex(const pa_shape* shape, const pa_options* options, const void* q,
                  const void* k_cache, const void* v_cache, const int32_t* block_table,
                  const int32_t* seq_lens, float scale, int causal, int num_splits, void* out,
                  float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return pa::run_attention(shape, options, false, q, k_cache, v_cache, block_table, seq_lens, scale,
                       causal, num_splits, out, lse, workspace, workspace_bytes, stream);
}

int pa_combine(int32_t dtype, int32_t rows, int32_t num_splits, int32_t head_dim_v,
               const float* part_out, const float* part_lse, void* out, float* lse,
               void* stream) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) return PA_EINVAL;
  if (rows <= 0 || num_splits <= 0 || head_dim_v <= 0) return PA_EINVAL;
  if (part_out == nullptr || part_lse == nullptr || out == nullptr) return PA_EINVAL;
  const uintptr_t out_align = dtype == PA_F32 ? 3u : 1u;
  if (!aligned4(part_out) || !aligned4(part_lse) || !aligned4(lse) ||
      (reinterpret_cast<uintptr_t>(out) & out_align) != 0)
    return PA_EINVAL;
  const hipError_t err = pa::launch_combine(dtype, rows, num_splits, head_dim_v, part_out,
                                            part_lse, out, lse, static_cast<hipStream_t>(stream));
  return err == hipSuccess ? PA_OK : PA_EHIP;
}

size_t pa_workspace_bytes(const pa_shape* shape, int num_splits) {
  if (check_shape(shape, false) != PA_OK || check_splits(num_splits) != PA_OK) return 0;
  return workspace_for(shape, plan_for(shape, num_splits).num_splits);
}

int pa_resolve_num_splits(const pa_shape* shape, int num_splits) {
  int st = check_shape(shape, false);
  if (st != PA_OK) return st;
  st = check_splits(num_splits);
  if (st != PA_OK) return st;
  return plan_for(shape, num_splits).num_splits;
}

int pa_describe_plan(const pa_shape* shape, int num_splits, pa_plan_info* info) {
  if (info == nullptr) return PA_EINVAL;
  int st = check_shape(shape, false);
  if (st != PA_OK) return st;
  st = check_splits(num_splits);
  if (st != PA_OK) return st;
  const pa::AttnPlan plan = plan_for(shape, num_splits);
  int kernel = PA_KERNEL_VALU;
  if (plan.prefill)
    kernel = plan.waves == pa::kPrefillTeamWaves ? PA_KERNEL_SHARED_TILE_TEAMS
                                                 : PA_KERNEL_SHARED_TILE;
  else if (plan.mfma)
    kernel = plan.rows_per_wg == 32 ? PA_KERNEL_MFMA_TWO_BLOCKS : PA_KERNEL_MFMA;
  info->kernel = kernel;
  info->num_splits = plan.num_splits;
  info->rows_per_workgroup = plan.rows_per_wg;
  info->row_groups = plan.row_groups;
  info->waves = plan.waves;
  info->kv_heads_per_workgroup = plan.heads_per_wg;
  return PA_OK;
}

const char* pa_strerror(int status) {
  switch (status) {
    case PA_OK: return "success";
    case PA_EINVAL: return "invalid argument";
    case PA_EUNSUPPORTED: return "shape or dtype outside the compiled envelope";
    case PA_EWORKSPACE: return "workspace missing or too small";
    case PA_EHIP: return "HIP runtime error at launch";
    case PA_ESCRATCH:
      return "split partials larger than the library's static scratch (PA_NOALLOC_SCRATCH_BYTES)";
    default: return "unknown status";
  }
}

}  // extern "C"
