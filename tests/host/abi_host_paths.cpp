// Drives every host-only path of the C ABI (argument validation, launch
// planning, plan descriptions into short buffers, plan overrides, host
// scalars): built with AddressSanitizer by tests/test_host_asan.py and run
// without a GPU. No call here reaches a kernel launch: each either plans,
// describes, sizes, or fails validation first.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>
#include <string>
#include <vector>

#include "fql.h"

static int failures = 0;
#define EXPECT(cond)                                                  \
  do {                                                                \
    if (!(cond)) {                                                    \
      std::fprintf(stderr, "expectation failed: %s (line %d)\n", #cond, __LINE__); \
      ++failures;                                                     \
    }                                                                 \
  } while (0)

int main() {
  EXPECT(fql_version() > 0);
  char reason[8];  // deliberately short: messages are truncated, never overrun
  fql_is_supported(0, reason, sizeof(reason));
  EXPECT(std::strlen(reason) < sizeof(reason));
  for (int fmt = 0; fmt <= 6; ++fmt)
    for (int64_t K : {16, 100, 128, 4096})
      fql_can_implement(fmt, 4096, K, 16, reason, sizeof(reason));

  const int64_t Ms[] = {1, 2, 7, 8, 16, 17, 31, 32, 33, 64, 100, 128, 129, 256, 1000, 2048, 8192};
  const int64_t Ns[] = {16, 100, 400, 4096, 6144, 28672, 51200};
  const int64_t Ks[] = {16, 272, 1040, 4096, 14336, 25600};
  char desc[300];
  char tiny[5];
  for (int64_t M : Ms)
    for (int64_t N : Ns)
      for (int64_t K : Ks) {
        size_t bytes = 0;
        EXPECT(fql_linear_nvfp4_workspace_bytes(M, N, K, &bytes) == 0);
        for (int aligned = 0; aligned < 4; ++aligned) {
          EXPECT(fql_linear_nvfp4_describe(M, N, K, aligned, desc, sizeof(desc)) == 0);
          fql_linear_nvfp4_describe(M, N, K, aligned, tiny, sizeof(tiny));
          EXPECT(std::strlen(tiny) < sizeof(tiny));
        }
        if (K % 128 == 0 && N % 16 == 0) {
          fql_linear_mxfp4_workspace_bytes(M, N, K, &bytes);
          fql_linear_mxfp4_describe(M, N, K, desc, sizeof(desc));
          fql_linear_mxfp8_describe(M, N, K, tiny, sizeof(tiny));
          fql_linear_fp8_describe(M, N, K, desc, sizeof(desc));
          fql_linear_fp8_block_describe(M, N, K, tiny, sizeof(tiny));
        }
      }

  // plan overrides: valid, partial, malformed, very long, cleared
  const std::string long_spec(10000, 'x');
  const char* specs[] = {"kind=3,mt=4,nt=1,st=3,wm=1,cw=8,splits=2,xg=3", "kind=0,waves=4,ntw=2,rc=8",
                         "kind=4,waves=8,nt=1,st=3,pa=1,il=0", "=,=,,==", "kind=", "mt=999",
                         long_spec.c_str(), ""};
  for (const char* s : specs) {
    fql_set_plan_override(0, s);
    for (int64_t M : {1, 32, 128, 4096}) fql_linear_nvfp4_describe(M, 6144, 4096, 1, desc, sizeof(desc));
  }
  fql_set_plan_override(0, nullptr);
  for (const char* s : {"2,4,8,4,4,1", "1,4,4,2,4", "garbage", "0"}) {
    fql_set_plan_override(1, s);
    fql_set_plan_override(2, s);
    fql_linear_mxfp4_describe(4096, 14336, 4096, desc, sizeof(desc));
    fql_linear_mxfp4_describe(1, 14336, 4096, desc, sizeof(desc));
  }
  fql_set_plan_override(1, nullptr);
  fql_set_plan_override(2, nullptr);
  EXPECT(fql_set_plan_override(7, nullptr) < 0);

  // host scalars, including invalid inputs
  const float specials[] = {0.0f, -1.0f, 1.0f, 1e-30f, 3.0e38f, std::numeric_limits<float>::infinity(),
                            std::numeric_limits<float>::quiet_NaN(), std::numeric_limits<float>::denorm_min()};
  for (float a : specials) {
    float g = 0.0f, s = 0.0f, alpha = 0.0f;
    fql_nvfp4_global_scale(a, &g);
    fql_fp8_scale(a, &s);
    for (float b : specials) {
      fql_nvfp4_alpha(a, b, &alpha);
      fql_fp8_output_scale(a, b, &alpha);
    }
  }
  EXPECT(fql_nvfp4_global_scale(1.0f, nullptr) < 0);

  // linear calls rejected before any launch: null pointers, bad shapes, strides,
  // scales, Hadamard blocks and workspaces
  alignas(16) static uint16_t x[64], y[64];
  alignas(16) static uint8_t w[4096], ws[4096];
  EXPECT(fql_linear_nvfp4(nullptr, 1, 16, 16, 1.0f, 0, w, 16, 1.0f, nullptr, y, 16, ws, sizeof(ws), nullptr) < 0);
  EXPECT(fql_linear_nvfp4(x, 1, 15, 16, 1.0f, 0, w, 16, 1.0f, nullptr, y, 16, ws, sizeof(ws), nullptr) < 0);
  EXPECT(fql_linear_nvfp4(x, 1, 16, 8, 1.0f, 0, w, 16, 1.0f, nullptr, y, 16, ws, sizeof(ws), nullptr) < 0);
  EXPECT(fql_linear_nvfp4(x, 1, 16, 16, -1.0f, 0, w, 16, 1.0f, nullptr, y, 16, ws, sizeof(ws), nullptr) < 0);
  EXPECT(fql_linear_nvfp4(x, 1, 16, 16, 1.0f, 24, w, 16, 1.0f, nullptr, y, 16, ws, sizeof(ws), nullptr) < 0);
  EXPECT(fql_linear_nvfp4(x, 1, 16, 16, 1.0f, 0, w, 16, 1.0f, nullptr, y, 8, ws, sizeof(ws), nullptr) < 0);
  EXPECT(fql_linear_nvfp4(x, 1, 16, 16, 1.0f, 0, w, 16, 1.0f, nullptr, y, 16, ws, 0, nullptr) < 0);
  EXPECT(fql_linear_nvfp4(x, 0, 16, 16, 1.0f, 0, w, 16, 1.0f, nullptr, y, 16, ws, sizeof(ws), nullptr) < 0);
  EXPECT(fql_linear_nvfp4_noalloc(x, int64_t(1) << 40, 16, 16, 1.0f, 0, w, 16, 1.0f, nullptr, y, 16, nullptr) < 0);
  EXPECT(fql_linear_mxfp4(x, 1, 100, 100, w, 16, 1.0f, nullptr, y, 16, ws, sizeof(ws), nullptr) < 0);
  const char* err = fql_last_error();
  EXPECT(err != nullptr && std::strlen(err) > 0);

  if (failures) std::fprintf(stderr, "%d expectation(s) failed\n", failures);
  std::printf("host paths done\n");
  return failures ? 1 : 0;
}
