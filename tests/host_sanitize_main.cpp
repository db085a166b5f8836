// host_sanitize_main.cpp -- drives the library's host-side code (argument checks, workspace
// plans, launch plans, status strings) under AddressSanitizer and UndefinedBehaviorSanitizer
// on the CPU.  Every call below is rejected or answered before any HIP call, so no GPU is
// needed.  Built and run by tests/test_host_sanitize.py; prints one line per checked value.
#include <stdint.h>
#include <stdio.h>

#include "spec_verify.h"
#include "sv_probe.h"

int main() {
  const int32_t shapes[][3] = {{1, 0, 1}, {1, 4, 32}, {64, 4, 128256}, {256, 7, 152064}, {128, 6, 128256},
                               {3, 64, 2200000}, {1 << 20, 64, 1 << 20}, {0, 4, 32}, {4, -1, 32}, {4, 4, 0}};
  const float temps[] = {0.0f, 1.0f, 0.7f, -1.0f, 1.0f / 0.0f};
  const int32_t ks[] = {0, 1, 50, 256, 257, 40000, -3};
  unsigned long long acc = 0;
  for (auto &s : shapes)
    for (int dt = -1; dt <= 2; ++dt)
      for (float T : temps)
        for (int32_t k : ks) {
          acc += sv_workspace_bytes(s[0], s[1], s[2], (sv_dtype)dt, T, k);
          acc += sv_workspace_zero_bytes(s[0], s[1], s[2], (sv_dtype)dt, T, k);
          acc += sv_overlap_workspace_bytes(s[0], s[1], s[2], (sv_dtype)dt, T, k);
          acc += sv_tree_workspace_bytes(s[0], s[1] + 1, s[2], 4, (sv_dtype)dt, T, k);
          acc += sv_typical_workspace_bytes(s[0], s[1], s[2], (sv_dtype)dt, T, k);
          const char *p = sv_launch_plan(s[0], s[1], s[2], (sv_dtype)dt, T, k);
          for (; p && *p; ++p) acc += (unsigned char)*p;
          const char *q = sv_tree_launch_plan(s[0], s[1] + 1, s[2], 3, (sv_dtype)dt, T, k);
          for (; q && *q; ++q) acc += (unsigned char)*q;
        }
  // argument errors: each returns before any device work
  int32_t a[4];
  float u[4];
  char ws[512];
  void *W = (void *)(((uintptr_t)ws + 255) & ~(uintptr_t)255);
  printf("null %d\n", (int)spec_verify(nullptr, nullptr, SV_BF16, a, u, u, 1, 1, 8, 1.0f, 0, a, a, nullptr, W, 256, nullptr));
  printf("shape %d\n", (int)spec_verify(a, a, SV_BF16, a, u, u, 0, 1, 8, 1.0f, 0, a, a, nullptr, W, 256, nullptr));
  printf("dtype %d\n", (int)spec_verify(a, a, (sv_dtype)7, a, u, u, 1, 1, 8, 1.0f, 0, a, a, nullptr, W, 256, nullptr));
  printf("temp %d\n", (int)spec_verify(a, a, SV_F32, a, u, u, 1, 1, 8, -2.0f, 0, a, a, nullptr, W, 256, nullptr));
  printf("workspace %d\n", (int)spec_verify(a, a, SV_F32, a, u, u, 1, 1, 8, 1.0f, 0, a, a, nullptr, W, 0, nullptr));
  printf("align %d\n", (int)spec_verify((char *)a + 1, a, SV_F32, a, u, u, 1, 1, 8, 1.0f, 0, a, a, nullptr, W, 256, nullptr));
  printf("sample %d\n", (int)spec_sample(nullptr, SV_F32, u, 1, 8, 1.0f, 0, a, a, W, 256, nullptr));
  printf("typical %d\n", (int)spec_typical_verify(a, SV_F32, a, 1, 1, 8, 1.0f, 0, -1.0, 0.3, a, a, W, 256, nullptr));
  printf("probe %d\n", (int)sv_read_probe(a, 100, (uint32_t *)a, nullptr));
  for (int st = 0; st <= 9; ++st) {
    const char *m = sv_status_string((sv_status)st);
    for (; *m; ++m) acc += (unsigned char)*m;
  }
  printf("epoch %u\n", sv_tag_epoch());
  printf("checksum %llu\n", acc);
  return 0;
}
