// What the stand-in launchers saw last (host-only sanitizer build).
#pragma once

struct StubRecord {
  int calls = 0;          // attention launches
  int combines = 0;
  int page_checks = 0;
  int kind = -1;          // 0 valu f32, 1 mfma f16, 2 mfma bf16, 3 / 4 8-bit f16 / bf16
  int num_splits = 0;
  int rows_per_wg = 0;
  int waves = 0;
  int heads_per_wg = 0;
  int causal = 0;
  bool fail_launch = false;  // make the next launches report a HIP error
};

extern StubRecord g_stub;
