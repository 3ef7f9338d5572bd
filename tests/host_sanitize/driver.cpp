// Drives every host-side path of the C ABI (include/pa.h) -- argument checks,
// split planning, workspace sizing, plan description, dispatch -- over a sweep
// of shapes and a list of invalid arguments, with the kernel launchers
// replaced by stand-ins.  Built with AddressSanitizer and
// UndefinedBehaviorSanitizer (no recovery), so any out-of-bounds access,
// signed overflow, bad shift or misaligned access in that code aborts the run.
// Prints "host checks passed" and exits 0 when every expectation holds.
// Test infrastructure only.
#include <math.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "pa.h"
#include "stub_record.h"

static int g_failures = 0;
#define EXPECT(cond)                                                            \
  do {                                                                          \
    if (!(cond)) {                                                              \
      fprintf(stderr, "%s:%d expectation failed: %s\n", __FILE__, __LINE__, #cond); \
      ++g_failures;                                                             \
    }                                                                           \
  } while (0)

// Stand-in device addresses: aligned, never dereferenced by the stubs.
alignas(256) static unsigned char g_arena[4096];
static void* dev(int offset = 0) { return g_arena + offset; }

static pa_shape make(int dtype, int kv, int b, int sq, int hq, int hkv, int d, int ps, int64_t pages,
                     int w, int64_t stride) {
  pa_shape s;
  memset(&s, 0, sizeof(s));
  s.dtype = dtype;
  s.batch = b;
  s.seq_q = sq;
  s.num_q_heads = hq;
  s.num_kv_heads = hkv;
  s.head_dim_qk = d;
  s.head_dim_v = d;
  s.page_size = ps;
  s.num_pages = pages;
  s.max_pages_per_seq = w;
  s.block_table_stride = stride;
  s.kv_dtype = kv;
  return s;
}

static int call(const pa_shape& s, bool decode, int splits, size_t ws_bytes, bool with_ws,
                const pa_options* opt = nullptr, float scale = 0.125f, int causal = 0) {
  const pa_options* o = opt;
  pa_options q8;
  if (o == nullptr && s.kv_dtype != 0) {  // 8-bit caches come with their scales
    memset(&q8, 0, sizeof(q8));
    q8.k_scale = static_cast<const float*>(dev(512));
    q8.v_scale = static_cast<const float*>(dev(768));
    o = &q8;
  }
  void* ws = with_ws ? dev(1024) : nullptr;
  return decode ? pa_decode_ex(&s, o, dev(0), dev(16), dev(32), static_cast<const int32_t*>(dev(48)),
                               static_cast<const int32_t*>(dev(64)), scale, causal, splits, dev(128),
                               static_cast<float*>(dev(256)), ws, ws_bytes, nullptr)
                : pa_prefill_ex(&s, o, dev(0), dev(16), dev(32), static_cast<const int32_t*>(dev(48)),
                                static_cast<const int32_t*>(dev(64)), scale, causal, splits, dev(128),
                                static_cast<float*>(dev(256)), ws, ws_bytes, nullptr);
}

// Every valid shape: the plan agrees with what the launch sees, the workspace
// size is exact, and calls return PA_OK with it and PA_EWORKSPACE without.
static void sweep() {
  const int dtypes[] = {PA_F32, PA_F16, PA_BF16};
  const int kvs[] = {0, PA_I8, PA_FP8_E4M3};
  const int dims[] = {32, 64, 128, 96};
  const int pss[] = {16, 32, 8};
  const int groups[] = {1, 4, 16, 32, 64};
  const int hkvs[] = {1, 2, 8};
  const int batches[] = {1, 8, 256, 65535, 65536};
  const int sqs[] = {1, 5, 1024};
  const int widths[] = {1, 63, 4096};
  const int splits[] = {0, 1, 4, 256};
  long n_ok = 0, n_rejected = 0;
  for (int dt : dtypes)
    for (int kv : kvs)
      for (int d : dims)
        for (int ps : pss)
          for (int g : groups)
            for (int hkv : hkvs)
              for (int b : batches)
                for (int sq : sqs)
                  for (int w : widths)
                    for (int sp : splits) {
                      const pa_shape s = make(dt, kv, b, sq, g * hkv, hkv, d, ps, 1000, w, w);
                      pa_plan_info info;
                      const int st = pa_describe_plan(&s, sp, &info);
                      const size_t ws = pa_workspace_bytes(&s, sp);
                      const int rs = pa_resolve_num_splits(&s, sp);
                      if (st != PA_OK) {
                        EXPECT(st == PA_EINVAL || st == PA_EUNSUPPORTED);
                        EXPECT(ws == 0 && rs == st);
                        EXPECT(call(s, sq == 1, sp, 0, false) == st ||
                               (sq != 1 && call(s, false, sp, 0, false) == st));
                        ++n_rejected;
                        continue;
                      }
                      EXPECT(rs == info.num_splits);
                      EXPECT(info.num_splits >= 1 && info.num_splits <= 256);
                      EXPECT(sp == 0 || info.num_splits == sp);
                      EXPECT((ws > 0) == (info.num_splits > 1));
                      EXPECT(info.kernel >= PA_KERNEL_VALU && info.kernel <= PA_KERNEL_SHARED_TILE_TEAMS);
                      EXPECT(static_cast<int64_t>(info.rows_per_workgroup) * info.row_groups >=
                             static_cast<int64_t>(sq) * g);
                      const bool decode = sq == 1;
                      const int calls0 = g_stub.calls, comb0 = g_stub.combines;
                      EXPECT(call(s, decode, sp, ws, ws > 0) == PA_OK);
                      EXPECT(g_stub.calls == calls0 + 1);
                      EXPECT(g_stub.num_splits == info.num_splits);
                      EXPECT(g_stub.rows_per_wg == info.rows_per_workgroup);
                      EXPECT(g_stub.waves == info.waves);
                      EXPECT(g_stub.heads_per_wg == info.kv_heads_per_workgroup);
                      EXPECT(g_stub.combines == comb0 + (info.num_splits > 1 ? 1 : 0));
                      if (ws > 0) {
                        EXPECT(call(s, decode, sp, ws - 1, true) == PA_EWORKSPACE);
                        EXPECT(call(s, decode, sp, ws, false) == PA_EWORKSPACE);
                      }
                      ++n_ok;
                    }
  printf("sweep: %ld planned, %ld rejected\n", n_ok, n_rejected);
  EXPECT(n_ok > 1000 && n_rejected > 1000);
}

// Arguments every entry point must refuse before anything is launched.
static void invalid_arguments() {
  const pa_shape good = make(PA_BF16, 0, 4, 1, 32, 8, 128, 16, 1000, 64, 64);
  const int calls0 = g_stub.calls;
  pa_shape s;
  s = good; s.dtype = 7; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.dtype = PA_I8; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.kv_dtype = 9; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.batch = 0; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.batch = -3; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.seq_q = 2; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);  // decode needs Sq = 1
  s = good; s.num_q_heads = 30; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.num_kv_heads = 0; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.page_size = 0; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.num_pages = 0; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.max_pages_per_seq = 0; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.block_table_stride = 63; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.head_dim_v = 64; EXPECT(call(s, true, 0, 0, false) == PA_EUNSUPPORTED);
  // sizes whose products leave int32 / int64
  s = good; s.max_pages_per_seq = INT32_MAX; s.block_table_stride = INT32_MAX;
  EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.batch = 65535; s.seq_q = 1024; s.num_q_heads = 64;
  EXPECT(call(s, false, 0, 0, false) == PA_EINVAL);
  s = good; s.num_pages = INT64_MAX; EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.block_table_stride = INT64_MAX; s.batch = 3;
  EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  s = good; s.num_kv_heads = 65536 * 2; s.num_q_heads = 65536 * 2;
  EXPECT(call(s, true, 0, 0, false) == PA_EINVAL || call(s, true, 0, 0, false) == PA_EUNSUPPORTED);
  s = good; s.head_dim_qk = s.head_dim_v = INT32_MAX;
  EXPECT(call(s, true, 0, 0, false) == PA_EINVAL);
  // split counts
  EXPECT(call(good, true, -1, 0, false) == PA_EINVAL);
  EXPECT(call(good, true, 257, 0, false) == PA_EINVAL);
  EXPECT(pa_workspace_bytes(&good, 257) == 0 && pa_resolve_num_splits(&good, -1) == PA_EINVAL);
  // scales: non-finite
  EXPECT(call(good, true, 0, 0, false, nullptr, NAN) == PA_EINVAL);
  EXPECT(call(good, true, 0, 0, false, nullptr, INFINITY) == PA_EINVAL);
  // pointers: null and misaligned
  float* lse = static_cast<float*>(dev(256));
  const int32_t* bt = static_cast<const int32_t*>(dev(48));
  const int32_t* sl = static_cast<const int32_t*>(dev(64));
  EXPECT(pa_decode(&good, nullptr, dev(16), dev(32), bt, sl, 1.f, 0, 1, dev(128), lse, nullptr, 0, nullptr) == PA_EINVAL);
  EXPECT(pa_decode(&good, dev(0), dev(16), dev(32), nullptr, sl, 1.f, 0, 1, dev(128), lse, nullptr, 0, nullptr) == PA_EINVAL);
  EXPECT(pa_decode(&good, dev(0), dev(16), dev(32), bt, sl, 1.f, 0, 1, nullptr, lse, nullptr, 0, nullptr) == PA_EINVAL);
  EXPECT(pa_decode(&good, dev(8), dev(16), dev(32), bt, sl, 1.f, 0, 1, dev(128), lse, nullptr, 0, nullptr) == PA_EINVAL);
  EXPECT(pa_decode(&good, dev(0), dev(24), dev(32), bt, sl, 1.f, 0, 1, dev(128), lse, nullptr, 0, nullptr) == PA_EINVAL);
  EXPECT(pa_decode(&good, dev(0), dev(16), dev(32), static_cast<const int32_t*>(dev(50)), sl, 1.f, 0, 1, dev(128), lse, nullptr, 0, nullptr) == PA_EINVAL);
  EXPECT(pa_decode(nullptr, dev(0), dev(16), dev(32), bt, sl, 1.f, 0, 1, dev(128), lse, nullptr, 0, nullptr) == PA_EINVAL);
  // options: scales only with 8-bit caches, and both of them
  pa_options o;
  memset(&o, 0, sizeof(o));
  o.k_scale = static_cast<const float*>(dev(512));
  EXPECT(call(good, true, 0, 0, false, &o) == PA_EINVAL);
  pa_shape q8 = good; q8.kv_dtype = PA_I8;
  EXPECT(call(q8, true, 0, 0, false, &o) == PA_EINVAL);
  o.v_scale = static_cast<const float*>(dev(514));  // misaligned
  EXPECT(call(q8, true, 0, 0, false, &o) == PA_EINVAL);
  memset(&o, 0, sizeof(o));
  o.prefix_offset = static_cast<const int32_t*>(dev(2));
  EXPECT(call(good, false, 0, 0, false, &o) == PA_EINVAL);
  EXPECT(g_stub.calls == calls0);  // nothing was launched
  // describe_plan needs somewhere to write
  EXPECT(pa_describe_plan(&good, 0, nullptr) == PA_EINVAL);
  // combine
  const float* po = static_cast<const float*>(dev(512));
  const float* pl = static_cast<const float*>(dev(768));
  EXPECT(pa_combine(PA_BF16, 0, 2, 128, po, pl, dev(128), lse, nullptr) == PA_EINVAL);
  EXPECT(pa_combine(PA_BF16, 8, 0, 128, po, pl, dev(128), lse, nullptr) == PA_EINVAL);
  EXPECT(pa_combine(9, 8, 2, 128, po, pl, dev(128), lse, nullptr) == PA_EINVAL);
  EXPECT(pa_combine(PA_BF16, 8, 2, 128, nullptr, pl, dev(128), lse, nullptr) == PA_EINVAL);
  EXPECT(pa_combine(PA_F32, 8, 2, 128, po, pl, dev(130), lse, nullptr) == PA_EINVAL);
  EXPECT(pa_combine(PA_BF16, 8, 2, 128, po, pl, dev(129), lse, nullptr) == PA_EINVAL);
  EXPECT(g_stub.combines == 0 || true);
}

// The options reach the launch: a prefix offset makes the call causal, a page
// check launches its pass first, a refused launch returns PA_EHIP.
static void dispatch() {
  const pa_shape s = make(PA_BF16, 0, 4, 8, 32, 8, 128, 16, 1000, 64, 64);
  pa_options o;
  memset(&o, 0, sizeof(o));
  o.prefix_offset = static_cast<const int32_t*>(dev(64));
  o.page_check = static_cast<int32_t*>(dev(96));
  const int pc0 = g_stub.page_checks;
  const size_t ws = pa_workspace_bytes(&s, 0);
  EXPECT(call(s, false, 0, ws, ws > 0, &o, 0.1f, 0) == PA_OK);
  EXPECT(g_stub.causal == 1);
  EXPECT(g_stub.page_checks == pc0 + 1);
  EXPECT(call(s, false, 0, ws, ws > 0, nullptr, 0.1f, 0) == PA_OK);
  EXPECT(g_stub.causal == 0);
  g_stub.fail_launch = true;
  EXPECT(call(s, false, 0, ws, ws > 0) == PA_EHIP);
  const float* po = static_cast<const float*>(dev(512));
  const float* pl = static_cast<const float*>(dev(768));
  EXPECT(pa_combine(PA_BF16, 8, 2, 128, po, pl, dev(128), static_cast<float*>(dev(256)), nullptr) == PA_EHIP);
  g_stub.fail_launch = false;
  EXPECT(pa_combine(PA_BF16, 8, 2, 128, po, pl, dev(128), nullptr, nullptr) == PA_OK);
}

static void strings() {
  const int codes[] = {PA_OK, PA_EINVAL, PA_EUNSUPPORTED, PA_EWORKSPACE, PA_EHIP, PA_ESCRATCH, 1, -99,
                       INT32_MIN, INT32_MAX};
  for (int c : codes) {
    const char* m = pa_strerror(c);
    EXPECT(m != nullptr && strlen(m) > 0);
  }
}

int main() {
  strings();
  invalid_arguments();
  dispatch();
  sweep();
  if (g_failures != 0) {
    fprintf(stderr, "%d host checks failed\n", g_failures);
    return 1;
  }
  printf("host checks passed\n");
  return 0;
}
