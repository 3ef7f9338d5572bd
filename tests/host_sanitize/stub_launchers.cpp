// Stand-ins for the kernel launchers of libpa.so, for a host-only build of the
// C-ABI layer (pa_api.cpp) under AddressSanitizer and UndefinedBehaviorSanitizer.
// Each stub checks the launch description it receives for internal consistency
// and records it; none touches a pointer.  Test infrastructure only.
#include <stdio.h>
#include <stdlib.h>

#include "pa_internal.h"
#include "stub_record.h"

StubRecord g_stub;

namespace {

void fail(const char* what) {
  fprintf(stderr, "stub check failed: %s\n", what);
  abort();
}

hipError_t record_attention(const pa::AttnParams& p, const pa::AttnPlan& plan, int kind,
                            int head_dim, int page_size, int batch) {
  if (plan.num_splits < 1 || plan.num_splits > 256) fail("split count out of range");
  if (p.num_splits != plan.num_splits) fail("params and plan disagree on the split count");
  if (plan.rows_per_wg <= 0 || plan.row_groups <= 0) fail("empty row groups");
  if (static_cast<int64_t>(plan.rows_per_wg) * plan.row_groups < p.rows_per_kvh)
    fail("row groups do not cover the rows of a kv head");
  if (plan.heads_per_wg <= 0 || p.num_kv_heads % plan.heads_per_wg != 0)
    fail("kv heads per workgroup do not divide Hkv");
  if (plan.waves != 4 && plan.waves != 8 && plan.waves != 16) fail("wave count");
  if (p.group * p.num_kv_heads != p.num_q_heads) fail("group size");
  if ((plan.num_splits > 1) != (p.part_out != nullptr && p.part_lse != nullptr))
    fail("partials present exactly when splitting");
  if (head_dim <= 0 || page_size <= 0 || batch <= 0) fail("launch sizes");
  g_stub.calls += 1;
  g_stub.kind = kind;
  g_stub.num_splits = plan.num_splits;
  g_stub.rows_per_wg = plan.rows_per_wg;
  g_stub.waves = plan.waves;
  g_stub.heads_per_wg = plan.heads_per_wg;
  g_stub.causal = p.causal;
  return g_stub.fail_launch ? hipErrorInvalidValue : hipSuccess;
}

}  // namespace

namespace pa {

hipError_t launch_attn_valu_f32(const AttnParams& p, const AttnPlan& plan, int head_dim,
                                int page_size, int batch, hipStream_t) {
  return record_attention(p, plan, 0, head_dim, page_size, batch);
}
hipError_t launch_attn_mfma_f16(const AttnParams& p, const AttnPlan& plan, int head_dim,
                                int page_size, int batch, hipStream_t) {
  return record_attention(p, plan, 1, head_dim, page_size, batch);
}
hipError_t launch_attn_mfma_bf16(const AttnParams& p, const AttnPlan& plan, int head_dim,
                                 int page_size, int batch, hipStream_t) {
  return record_attention(p, plan, 2, head_dim, page_size, batch);
}
hipError_t launch_attn_mfma_q_f16(const AttnParams& p, const AttnPlan& plan, int kv_dtype,
                                  int head_dim, int page_size, int batch, hipStream_t) {
  if (kv_dtype != PA_I8 && kv_dtype != PA_FP8_E4M3) fail("8-bit kind");
  return record_attention(p, plan, 3, head_dim, page_size, batch);
}
hipError_t launch_attn_mfma_q_bf16(const AttnParams& p, const AttnPlan& plan, int kv_dtype,
                                   int head_dim, int page_size, int batch, hipStream_t) {
  if (kv_dtype != PA_I8 && kv_dtype != PA_FP8_E4M3) fail("8-bit kind");
  return record_attention(p, plan, 4, head_dim, page_size, batch);
}
hipError_t launch_page_check(const int32_t*, int64_t bt_stride, const int32_t*, int batch,
                             int width, int page_size, int64_t num_pages, int32_t*, hipStream_t) {
  if (bt_stride < width || batch <= 0 || width <= 0 || page_size <= 0 || num_pages <= 0)
    fail("page-check sizes");
  g_stub.page_checks += 1;
  return hipSuccess;
}
hipError_t launch_combine(int dtype, int rows, int num_splits, int head_dim_v, const float*,
                          const float*, void*, float*, hipStream_t) {
  if (dtype != PA_F32 && dtype != PA_F16 && dtype != PA_BF16) fail("combine dtype");
  if (rows <= 0 || num_splits <= 0 || head_dim_v <= 0) fail("combine sizes");
  g_stub.combines += 1;
  return g_stub.fail_launch ? hipErrorInvalidValue : hipSuccess;
}

}  // namespace pa
