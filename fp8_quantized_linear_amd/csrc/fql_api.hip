// C ABI of the gfx950 NVFP4 linear library: argument validation, dispatch,
// error reporting. Every entry point validates on the host (cheap checks
// only), enqueues kernels on the caller's stream and returns a status code.
// The availability / format-constraint split follows the write-ups' kernel
// lifecycle: is_supported decides availability with a reason string,
// can_implement checks format constraints, and the hot call only asserts.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>

#include "../../include/fql.h"
#include "fql_internal.h"

// ---- launch-plan overrides and per-thread plan caches ------------------------

namespace fql {
namespace {

std::mutex g_override_mutex;
std::string g_override[3];
bool g_override_read = false;
std::atomic<uint32_t> g_override_generation{1};

void read_env_overrides_locked() {
  if (g_override_read) return;
  static const char* const names[3] = {"FQL_PLAN", "FQL_SC_PLAN", "FQL_SC_GEMV"};
  for (int i = 0; i < 3; ++i) {
    const char* e = std::getenv(names[i]);
    g_override[i] = e ? e : "";
  }
  g_override_read = true;
}

// Direct-mapped cache of plans keyed by shape, a tag (alignment or format)
// and the override generation.
template <typename Plan>
struct PlanCache {
  struct Entry {
    int64_t M = -1, N = -1, K = -1;
    int tag = -1;
    uint32_t gen = 0;
    Plan plan{};
  };
  static constexpr int kEntries = 64;
  Entry e[kEntries];
  template <typename Make>
  const Plan& get(int64_t M, int64_t N, int64_t K, int tag, Make make) {
    const uint32_t gen = plan_generation();
    const uint64_t h = (uint64_t)M * 0x9E3779B97F4A7C15ull ^ (uint64_t)N * 0xC2B2AE3D27D4EB4Full ^
                       (uint64_t)K * 0x165667B19E3779F9ull ^ (uint64_t)tag;
    Entry& x = e[(h >> 32) % kEntries];
    if (x.M != M || x.N != N || x.K != K || x.tag != tag || x.gen != gen) {
      x.plan = make();
      x.M = M; x.N = N; x.K = K; x.tag = tag; x.gen = gen;
    }
    return x.plan;
  }
};

}  // namespace

std::string plan_override(int which) {
  std::lock_guard<std::mutex> lock(g_override_mutex);
  read_env_overrides_locked();
  return which >= 0 && which < 3 ? g_override[which] : std::string();
}

void set_plan_override(int which, const char* spec) {
  std::lock_guard<std::mutex> lock(g_override_mutex);
  read_env_overrides_locked();
  if (which < 0 || which >= 3) return;
  g_override[which] = spec ? spec : "";
  g_override_generation.fetch_add(1, std::memory_order_acq_rel);
}

uint32_t plan_generation() { return g_override_generation.load(std::memory_order_acquire); }

GemmPlan cached_plan_gemm_nvfp4(int64_t M, int64_t N, int64_t K, bool aligned, bool rotated) {
  thread_local PlanCache<GemmPlan> cache;
  return cache.get(M, N, K, (aligned ? 1 : 0) | (rotated ? 2 : 0),
                   [&] { return plan_gemm_nvfp4(M, N, K, aligned, rotated); });
}

ScPlan cached_plan_sc_gemm(int fmt, int64_t M, int64_t N, int64_t K) {
  thread_local PlanCache<ScPlan> cache;
  return cache.get(M, N, K, fmt, [&] { return plan_sc_gemm(fmt, M, N, K); });
}

}  // namespace fql

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int ok() {
  g_last_error.clear();
  return FQL_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(FQL_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return ok();
}

void write_reason(char* reason, size_t len, const std::string& s) {
  if (reason && len > 0) {
    std::snprintf(reason, len, "%s", s.c_str());
  }
}

bool valid_hadamard(int hb) { return hb == 0 || hb == 16 || hb == 32 || hb == 64 || hb == 128; }

// Shared NVFP4 shape checks; returns FQL_OK or an error with a message.
int check_nvfp4_shape(int64_t rows, int64_t K, int64_t ld, int hb, const char* rows_name) {
  if (rows < 1) return fail(FQL_ERR_INVALID, "%s must be >= 1 (got %lld)", rows_name, (long long)rows);
  if (K < 16 || K % 16 != 0)
    return fail(FQL_ERR_INVALID, "K must be a positive multiple of 16 (got %lld)", (long long)K);
  if (ld < K) return fail(FQL_ERR_INVALID, "row stride %lld is smaller than K %lld", (long long)ld, (long long)K);
  if (!valid_hadamard(hb))
    return fail(FQL_ERR_INVALID, "hadamard_block must be 0, 16, 32, 64 or 128 (got %d)", hb);
  if (hb > 0 && K % hb != 0)
    return fail(FQL_ERR_INVALID, "K %lld is not a multiple of hadamard_block %d", (long long)K, hb);
  if (K > (int64_t)1 << 24 || rows > (int64_t)1 << 24)
    return fail(FQL_ERR_INVALID, "dimension too large");
  return FQL_OK;
}

bool aligned16(const void* p, int64_t ld, int64_t elem_bytes) {
  return (reinterpret_cast<uintptr_t>(p) % 16 == 0) && ((ld * elem_bytes) % 16 == 0);
}

int check_scale(float g, const char* name) {
  if (!std::isfinite(g) || !(g > 0.0f))
    return fail(FQL_ERR_INVALID, "%s must be finite and > 0 (got %g)", name, (double)g);
  return FQL_OK;
}

}  // namespace

extern "C" {

int fql_version(void) { return 100; }

const char* fql_last_error(void) { return g_last_error.c_str(); }

int fql_is_supported(int device, char* reason, size_t reason_len) {
  int count = 0;
  hipError_t e = hipGetDeviceCount(&count);
  if (e != hipSuccess || count == 0) {
    write_reason(reason, reason_len, "no HIP device available");
    ok();
    return 0;
  }
  if (device < 0 || device >= count) {
    write_reason(reason, reason_len, "device index out of range");
    ok();
    return 0;
  }
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, device);
  if (e != hipSuccess) return hip_status(e, "hipGetDeviceProperties");
  if (std::strncmp(prop.gcnArchName, "gfx950", 6) != 0) {
    write_reason(reason, reason_len,
                 std::string("requires a gfx950 (MI355X) device, found ") + prop.gcnArchName);
    ok();
    return 0;
  }
  write_reason(reason, reason_len, "");
  ok();
  return 1;
}

int fql_can_implement(int format, int64_t N, int64_t K, int hadamard_block, char* reason,
                      size_t reason_len) {
  std::string why;
  if (format == FQL_FMT_NVFP4) {
    if (N < 1) why = "N must be >= 1";
    else if (K < 16 || K % 16 != 0) why = "K must be a positive multiple of 16 (the NVFP4 block)";
    else if (!valid_hadamard(hadamard_block)) why = "hadamard_block must be 0, 16, 32, 64 or 128";
    else if (hadamard_block > 0 && K % hadamard_block != 0) why = "K must be a multiple of hadamard_block";
  } else if (format == FQL_FMT_MXFP4 || format == FQL_FMT_MXFP8 || format == FQL_FMT_FP8) {
    if (N < 1) why = "N must be >= 1";
    else if (K < 32 || K % 32 != 0) why = "K must be a positive multiple of 32 (the MX block)";
    else if (hadamard_block != 0) why = "this format takes no rotation (hadamard_block must be 0)";
  } else if (format == FQL_FMT_FP8_BLOCK) {
    if (N < 128 || N % 128 != 0) why = "N must be a positive multiple of 128 (weight group 128 x 128)";
    else if (K < 128 || K % 128 != 0) why = "K must be a positive multiple of 128 (activation group 1 x 128)";
    else if (hadamard_block != 0) why = "this format takes no rotation (hadamard_block must be 0)";
  } else {
    why = "unknown format";
  }
  if (why.empty() && (N > (int64_t)1 << 24 || K > (int64_t)1 << 24)) why = "dimension too large";
  write_reason(reason, reason_len, why);
  ok();
  return why.empty() ? 1 : 0;
}

int fql_amax_bf16(const void* x, int64_t M, int64_t K, int64_t ldx, int hadamard_block,
                  float* amax_out, void* stream) {
  if (int r = check_nvfp4_shape(M, K, ldx, hadamard_block, "M")) return r;
  if (!x || !amax_out) return fail(FQL_ERR_INVALID, "null pointer");
  const uint16_t* xp = static_cast<const uint16_t*>(x);
  return hip_status(fql::launch_amax_bf16(xp, M, K, ldx, hadamard_block, aligned16(x, ldx, 2),
                                          amax_out, static_cast<hipStream_t>(stream)),
                    "amax_bf16 launch");
}

int fql_amax_f32(const float* w, int64_t N, int64_t K, int64_t ldw, int hadamard_block,
                 float* amax_out, void* stream) {
  if (int r = check_nvfp4_shape(N, K, ldw, hadamard_block, "N")) return r;
  if (!w || !amax_out) return fail(FQL_ERR_INVALID, "null pointer");
  return hip_status(fql::launch_amax_f32(w, N, K, ldw, hadamard_block, aligned16(w, ldw, 4),
                                         amax_out, static_cast<hipStream_t>(stream)),
                    "amax_f32 launch");
}

int fql_quant_nvfp4(const void* x, int64_t M, int64_t K, int64_t ldx, float global_scale,
                    int hadamard_block, uint8_t* codes, uint8_t* scales, void* stream) {
  if (int r = check_nvfp4_shape(M, K, ldx, hadamard_block, "M")) return r;
  if (int r = check_scale(global_scale, "global_scale")) return r;
  if (!x || !codes || !scales) return fail(FQL_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(codes) % 8 != 0)
    return fail(FQL_ERR_INVALID, "codes must be 8-byte aligned");
  return hip_status(
      fql::launch_quant_nvfp4_bf16(static_cast<const uint16_t*>(x), M, K, ldx, global_scale,
                                   hadamard_block, aligned16(x, ldx, 2), codes, scales,
                                   static_cast<hipStream_t>(stream)),
      "quant_nvfp4 launch");
}

int fql_quant_nvfp4_f32(const float* w, int64_t N, int64_t K, int64_t ldw, float global_scale,
                        int hadamard_block, uint8_t* codes, uint8_t* scales, void* stream) {
  if (int r = check_nvfp4_shape(N, K, ldw, hadamard_block, "N")) return r;
  if (int r = check_scale(global_scale, "global_scale")) return r;
  if (!w || !codes || !scales) return fail(FQL_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(codes) % 8 != 0)
    return fail(FQL_ERR_INVALID, "codes must be 8-byte aligned");
  return hip_status(fql::launch_quant_nvfp4_f32(w, N, K, ldw, global_scale, hadamard_block,
                                                aligned16(w, ldw, 4), codes, scales,
                                                static_cast<hipStream_t>(stream)),
                    "quant_nvfp4_f32 launch");
}

int fql_packed_nvfp4_bytes(int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(FQL_ERR_INVALID, "null pointer");
  if (N < 1 || K < 16 || K % 16 != 0)
    return fail(FQL_ERR_INVALID, "need N >= 1 and K a positive multiple of 16");
  *bytes = (size_t)fql::packed_dims(N, K).total_bytes();
  return ok();
}

int fql_pack_weight_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                          void* packed, size_t packed_bytes, void* stream) {
  if (int r = check_nvfp4_shape(N, K, K, 0, "N")) return r;
  if (!codes || !scales || !packed) return fail(FQL_ERR_INVALID, "null pointer");
  const size_t need = (size_t)fql::packed_dims(N, K).total_bytes();
  if (packed_bytes < need)
    return fail(FQL_ERR_INVALID, "packed buffer holds %zu bytes, %zu needed", packed_bytes, need);
  if (reinterpret_cast<uintptr_t>(packed) % 16 != 0)
    return fail(FQL_ERR_INVALID, "packed buffer must be 16-byte aligned");
  return hip_status(fql::launch_pack_nvfp4(codes, scales, N, K, static_cast<uint8_t*>(packed),
                                           static_cast<hipStream_t>(stream)),
                    "pack launch");
}

int fql_unpack_weight_nvfp4(const void* packed, int64_t N, int64_t K, uint8_t* codes,
                            uint8_t* scales, void* stream) {
  if (int r = check_nvfp4_shape(N, K, K, 0, "N")) return r;
  if (!codes || !scales || !packed) return fail(FQL_ERR_INVALID, "null pointer");
  return hip_status(fql::launch_unpack_nvfp4(static_cast<const uint8_t*>(packed), N, K, codes,
                                             scales, static_cast<hipStream_t>(stream)),
                    "unpack launch");
}

int fql_linear_nvfp4_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(FQL_ERR_INVALID, "null pointer");
  if (M < 1 || N < 1 || K < 16 || K % 16 != 0)
    return fail(FQL_ERR_INVALID, "need M, N >= 1 and K a positive multiple of 16");
  // either plan a call of this shape may take: aligned or unaligned rows (the
  // transform and dynamic-scale calls take the unaligned one); the rotation
  // changes no plan's workspace
  const int64_t a = fql::cached_plan_gemm_nvfp4(M, N, K, true, false).total_bytes;
  const int64_t u = fql::cached_plan_gemm_nvfp4(M, N, K, false, false).total_bytes;
  *bytes = (size_t)std::max(a, u);
  return ok();
}

int fql_linear_nvfp4_describe(int64_t M, int64_t N, int64_t K, int aligned, char* buf,
                              size_t buf_len) {
  if (M < 1 || N < 1 || K < 16 || K % 16 != 0)
    return fail(FQL_ERR_INVALID, "need M, N >= 1 and K a positive multiple of 16");
  // a transform call plans as unaligned rows; its quantizer is the transform kernel
  const bool transform = (aligned & 2) != 0;
  const bool rotated = (aligned & 4) != 0;
  std::string d = fql::describe_plan(
      fql::plan_gemm_nvfp4(M, N, K, !transform && (aligned & 1) != 0, rotated && !transform));
  if (transform) {
    for (const char* q : {"quant_nvfp4_apack_kernel", "quant_nvfp4_xhat_kernel"}) {
      const size_t at = d.find(q);
      if (at != std::string::npos) d.replace(at, std::strlen(q), "transform_quant_kernel");
    }
  }
  write_reason(buf, buf_len, d);
  return ok();
}

}  // extern "C"

namespace {

// Checks shared by the NVFP4 linear entry points (shape, scales, pointers).
int check_linear_nvfp4(const void* x, int64_t M, int64_t K, int64_t ldx, float g, int hb,
                       const void* w_packed, int64_t N, const void* y, int64_t ldy) {
  if (int r = check_nvfp4_shape(M, K, ldx, hb, "M")) return r;
  if (int r = check_scale(g, "input_global_scale")) return r;
  if (N < 1 || N > (int64_t)1 << 24) return fail(FQL_ERR_INVALID, "N out of range");
  if (ldy < N) return fail(FQL_ERR_INVALID, "ldy %lld is smaller than N %lld", (long long)ldy, (long long)N);
  if (!x || !w_packed || !y) return fail(FQL_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(w_packed) % 16 != 0)
    return fail(FQL_ERR_INVALID, "packed weight must be 16-byte aligned");
  return FQL_OK;
}

int check_workspace(const void* workspace, size_t workspace_bytes, int64_t need) {
  if (!workspace) return fail(FQL_ERR_INVALID, "null workspace");
  if (reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(FQL_ERR_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < (size_t)need)
    return fail(FQL_ERR_WORKSPACE, "workspace holds %zu bytes, %lld needed", workspace_bytes,
                (long long)need);
  return FQL_OK;
}

// fql_linear_nvfp4 with alpha either a host value or (alpha_dev non-null) a
// device scalar.
int linear_nvfp4_plain(const void* x, int64_t M, int64_t K, int64_t ldx, float g, int hb,
                       const void* w_packed, int64_t N, float alpha, const float* alpha_dev,
                       const void* bias, void* y, int64_t ldy, void* workspace,
                       size_t workspace_bytes, void* stream) {
  if (int r = check_linear_nvfp4(x, M, K, ldx, g, hb, w_packed, N, y, ldy)) return r;
  if (alpha_dev == nullptr && !std::isfinite(alpha)) return fail(FQL_ERR_INVALID, "alpha must be finite");
  if (alpha_dev != nullptr && reinterpret_cast<uintptr_t>(alpha_dev) % 4 != 0)
    return fail(FQL_ERR_INVALID, "alpha_dev must be 4-byte aligned");
  const bool xal = aligned16(x, ldx, 2);
  const fql::GemmPlan plan = fql::cached_plan_gemm_nvfp4(M, N, K, xal, hb > 0);
  if (int r = check_workspace(workspace, workspace_bytes, plan.total_bytes)) return r;
  fql::LinearExtras ex{};
  ex.alpha_dev = alpha_dev;
  hipError_t e = fql::launch_linear_nvfp4(
      plan, static_cast<const uint16_t*>(x), M, K, ldx, g, hb, xal,
      static_cast<const uint8_t*>(w_packed), N, alpha, static_cast<const uint16_t*>(bias),
      static_cast<uint16_t*>(y), ldy, static_cast<uint8_t*>(workspace),
      static_cast<hipStream_t>(stream), alpha_dev != nullptr ? &ex : nullptr);
  return hip_status(e, "linear launch");
}

}  // namespace

extern "C" {

int fql_linear_nvfp4(const void* x, int64_t M, int64_t K, int64_t ldx, float input_global_scale,
                     int hadamard_block, const void* w_packed, int64_t N, float alpha,
                     const void* bias, void* y, int64_t ldy, void* workspace,
                     size_t workspace_bytes, void* stream) {
  return linear_nvfp4_plain(x, M, K, ldx, input_global_scale, hadamard_block, w_packed, N, alpha,
                            nullptr, bias, y, ldy, workspace, workspace_bytes, stream);
}

int fql_linear_nvfp4_dev_alpha(const void* x, int64_t M, int64_t K, int64_t ldx,
                               float input_global_scale, int hadamard_block, const void* w_packed,
                               int64_t N, const float* alpha_dev, const void* bias, void* y,
                               int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  if (!alpha_dev) return fail(FQL_ERR_INVALID, "null alpha_dev");
  return linear_nvfp4_plain(x, M, K, ldx, input_global_scale, hadamard_block, w_packed, N, 0.0f,
                            alpha_dev, bias, y, ldy, workspace, workspace_bytes, stream);
}

int fql_linear_nvfp4_quantize(const void* x, int64_t M, int64_t K, int64_t ldx,
                              float input_global_scale, int hadamard_block, int64_t N,
                              void* workspace, size_t workspace_bytes, void* stream) {
  if (int r = check_nvfp4_shape(M, K, ldx, hadamard_block, "M")) return r;
  if (int r = check_scale(input_global_scale, "input_global_scale")) return r;
  if (N < 1 || N > (int64_t)1 << 24) return fail(FQL_ERR_INVALID, "N out of range");
  if (!x) return fail(FQL_ERR_INVALID, "null pointer");
  const bool xal = aligned16(x, ldx, 2);
  const fql::GemmPlan plan = fql::cached_plan_gemm_nvfp4(M, N, K, xal, hadamard_block > 0);
  if (!fql::has_quant_pass(plan))
    return fail(FQL_ERR_UNSUPPORTED, "this call's plan quantizes inside the GEMM (%s)",
                fql::describe_plan(plan).c_str());
  if (int r = check_workspace(workspace, workspace_bytes, plan.total_bytes)) return r;
  return hip_status(fql::launch_linear_quant(plan, static_cast<const uint16_t*>(x), M, K, ldx,
                                             input_global_scale, hadamard_block, xal,
                                             static_cast<uint8_t*>(workspace),
                                             static_cast<hipStream_t>(stream)),
                    "quantize launch");
}

int fql_linear_nvfp4_gemm(int64_t M, int64_t K, int x_aligned, const void* w_packed, int64_t N,
                          float alpha, const void* bias, void* y, int64_t ldy, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (M < 1 || M > (int64_t)1 << 24 || K < 16 || K % 16 != 0 || K > (int64_t)1 << 24)
    return fail(FQL_ERR_INVALID, "need 1 <= M <= 2^24 and K a positive multiple of 16");
  if (N < 1 || N > (int64_t)1 << 24) return fail(FQL_ERR_INVALID, "N out of range");
  if (!std::isfinite(alpha)) return fail(FQL_ERR_INVALID, "alpha must be finite");
  if (ldy < N) return fail(FQL_ERR_INVALID, "ldy %lld is smaller than N %lld", (long long)ldy, (long long)N);
  if (!w_packed || !y) return fail(FQL_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(w_packed) % 16 != 0)
    return fail(FQL_ERR_INVALID, "packed weight must be 16-byte aligned");
  // the rotation never changes a plan with a quantizer pass
  const fql::GemmPlan plan = fql::cached_plan_gemm_nvfp4(M, N, K, x_aligned != 0, false);
  if (plan.kind == 0)
    return fail(FQL_ERR_UNSUPPORTED, "this call's plan quantizes inside the GEMM (%s)",
                fql::describe_plan(plan).c_str());
  if (int r = check_workspace(workspace, workspace_bytes, plan.total_bytes)) return r;
  return hip_status(fql::launch_linear_gemm(plan, static_cast<const uint8_t*>(w_packed), M, N, alpha,
                                            static_cast<const uint16_t*>(bias),
                                            static_cast<uint16_t*>(y), ldy,
                                            static_cast<uint8_t*>(workspace),
                                            static_cast<hipStream_t>(stream)),
                    "gemm launch");
}

// ---- host-side scalars of the layer -------------------------------------------

int fql_nvfp4_global_scale(float amax, float* global_scale) {
  if (!global_scale) return fail(FQL_ERR_INVALID, "null pointer");
  if (!std::isfinite(amax) || amax < 0.0f)
    return fail(FQL_ERR_INVALID, "amax must be finite and >= 0 (got %g)", (double)amax);
  if (amax == 0.0f) {
    *global_scale = 1.0f;
  } else {
    const float g = 2688.0f / amax;  // fl32(448 * 6 / amax), a correctly rounded division
    const float cap = 0x1p118f;      // keeps g / (smallest E4M3 scale 2^-9) finite
    *global_scale = g < cap ? g : cap;
  }
  return ok();
}

int fql_nvfp4_alpha(float input_global_scale, float weight_global_scale, float* alpha) {
  if (!alpha) return fail(FQL_ERR_INVALID, "null pointer");
  if (int r = check_scale(input_global_scale, "input_global_scale")) return r;
  if (int r = check_scale(weight_global_scale, "weight_global_scale")) return r;
  *alpha = (float)((1.0 / (double)input_global_scale) * (1.0 / (double)weight_global_scale));
  return ok();
}

int fql_fp8_scale(float amax, float* scale) {
  if (!scale) return fail(FQL_ERR_INVALID, "null pointer");
  if (!std::isfinite(amax) || amax < 0.0f)
    return fail(FQL_ERR_INVALID, "amax must be finite and >= 0 (got %g)", (double)amax);
  const float s = (float)((double)amax / 448.0);
  *scale = s > 0.0f ? s : 1.0f;  // an all-zero tensor (or one whose amax / 448 underflows) takes 1
  return ok();
}

int fql_fp8_output_scale(float input_scale, float weight_scale, float* alpha) {
  if (!alpha) return fail(FQL_ERR_INVALID, "null pointer");
  if (int r = check_scale(input_scale, "input_scale")) return r;
  if (int r = check_scale(weight_scale, "weight_scale")) return r;
  *alpha = (float)((double)input_scale * (double)weight_scale);
  return ok();
}

int fql_set_plan_override(int which, const char* spec) {
  if (which != FQL_PLAN_NVFP4 && which != FQL_PLAN_SC_GEMM && which != FQL_PLAN_SC_GEMV)
    return fail(FQL_ERR_INVALID, "unknown plan override %d", which);
  static_assert(FQL_PLAN_NVFP4 == fql::kOverrideNvfp4 && FQL_PLAN_SC_GEMM == fql::kOverrideScGemm &&
                    FQL_PLAN_SC_GEMV == fql::kOverrideScGemv,
                "override numbering");
  fql::set_plan_override(which, spec);
  return ok();
}

// ---- general block-diagonal transform, dynamic global scale ------------------

}  // extern "C"

namespace {

int check_transform(const void* T, int b, int64_t K) {
  if (b != 16 && b != 32 && b != 64 && b != 128)
    return fail(FQL_ERR_INVALID, "transform block must be 16, 32, 64 or 128 (got %d)", b);
  if (K % b != 0)
    return fail(FQL_ERR_INVALID, "K %lld is not a multiple of the transform block %d", (long long)K, b);
  if (!T) return fail(FQL_ERR_INVALID, "null transform matrix");
  if (reinterpret_cast<uintptr_t>(T) % 16 != 0)
    return fail(FQL_ERR_INVALID, "transform matrix must be 16-byte aligned");
  return FQL_OK;
}

// amax of the (optionally transformed or rotated) activation into the
// partial-maximum slots of scal, then amax, g (and alpha when with_alpha) on
// the device (layout: fql::kAmaxSlots partial maxima, amax, g, alpha).
hipError_t launch_dynamic_prologue(const void* x, int64_t M, int64_t K, int64_t ldx,
                                   const void* T, int b, float* scal, float g_w, bool with_alpha,
                                   hipStream_t st) {
  hipError_t e;
  if (T) {
    fql::TransformArgs a{};
    a.mode = 2;
    a.x = static_cast<const uint16_t*>(x); a.M = M; a.K = K; a.ldx = ldx;
    a.aligned = fql::transform_aligned(x, ldx, b);
    a.T = static_cast<const uint16_t*>(T); a.b = b;
    a.rows_out = M; a.amax = reinterpret_cast<uint32_t*>(scal);
    e = fql::launch_transform_nvfp4(a, st);
  } else {
    e = fql::launch_amax_bf16(static_cast<const uint16_t*>(x), M, K, ldx, b, aligned16(x, ldx, 2),
                              scal, st, fql::kAmaxSlots);
  }
  if (e != hipSuccess) return e;
  return fql::launch_dynamic_scale(scal, g_w, with_alpha, st);
}

}  // namespace

extern "C" {

int fql_transform_bf16(const void* x, int64_t M, int64_t K, int64_t ldx, const void* T, int b,
                       float* v, int64_t ldv, void* stream) {
  if (int r = check_nvfp4_shape(M, K, ldx, 0, "M")) return r;
  if (int r = check_transform(T, b, K)) return r;
  if (!x || !v) return fail(FQL_ERR_INVALID, "null pointer");
  if (ldv < K || ldv % 4 != 0 || reinterpret_cast<uintptr_t>(v) % 16 != 0)
    return fail(FQL_ERR_INVALID, "v must be 16-byte aligned with ldv >= K, ldv % 4 == 0");
  fql::TransformArgs a{};
  a.mode = 3;
  a.x = static_cast<const uint16_t*>(x); a.M = M; a.K = K; a.ldx = ldx;
  a.aligned = fql::transform_aligned(x, ldx, b);
  a.T = static_cast<const uint16_t*>(T); a.b = b;
  a.rows_out = M; a.v = v; a.ldv = ldv;
  return hip_status(fql::launch_transform_nvfp4(a, static_cast<hipStream_t>(stream)), "transform launch");
}

int fql_quant_nvfp4_transform(const void* x, int64_t M, int64_t K, int64_t ldx, float global_scale,
                              const void* T, int b, uint8_t* codes, uint8_t* scales, void* stream) {
  if (int r = check_nvfp4_shape(M, K, ldx, 0, "M")) return r;
  if (int r = check_transform(T, b, K)) return r;
  if (int r = check_scale(global_scale, "global_scale")) return r;
  if (!x || !codes || !scales) return fail(FQL_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(codes) % 8 != 0)
    return fail(FQL_ERR_INVALID, "codes must be 8-byte aligned");
  fql::TransformArgs a{};
  a.mode = 0;
  a.x = static_cast<const uint16_t*>(x); a.M = M; a.K = K; a.ldx = ldx;
  a.aligned = fql::transform_aligned(x, ldx, b);
  a.T = static_cast<const uint16_t*>(T); a.b = b; a.g = global_scale;
  a.codes = codes; a.scales = scales; a.rows_out = M;
  return hip_status(fql::launch_transform_nvfp4(a, static_cast<hipStream_t>(stream)), "transform quant launch");
}

int fql_quant_nvfp4_dynamic(const void* x, int64_t M, int64_t K, int64_t ldx, const void* T, int b,
                            float* scalars, uint8_t* codes, uint8_t* scales, void* stream) {
  if (int r = check_nvfp4_shape(M, K, ldx, T ? 0 : b, "M")) return r;
  if (T) {
    if (int r = check_transform(T, b, K)) return r;
  }
  if (!x || !codes || !scales || !scalars) return fail(FQL_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(codes) % 8 != 0 || reinterpret_cast<uintptr_t>(scalars) % 4 != 0)
    return fail(FQL_ERR_INVALID, "codes must be 8-byte and scalars 4-byte aligned");
  static_assert(FQL_DYNAMIC_SCALARS >= fql::kDynScalarWords, "scalar buffer size");
  hipStream_t st = static_cast<hipStream_t>(stream);
  float* g_dev = scalars + fql::kAmaxSlots + 1;
  hipError_t e = launch_dynamic_prologue(x, M, K, ldx, T, b, scalars, 0.0f, false, st);
  if (e != hipSuccess) return hip_status(e, "dynamic scale launch");
  if (T) {
    fql::TransformArgs a{};
    a.mode = 0;
    a.x = static_cast<const uint16_t*>(x); a.M = M; a.K = K; a.ldx = ldx;
    a.aligned = fql::transform_aligned(x, ldx, b);
    a.T = static_cast<const uint16_t*>(T); a.b = b; a.g = 1.0f; a.g_dev = g_dev;
    a.codes = codes; a.scales = scales; a.rows_out = M;
    e = fql::launch_transform_nvfp4(a, st);
  } else {
    e = fql::launch_quant_nvfp4_bf16(static_cast<const uint16_t*>(x), M, K, ldx, 1.0f, b,
                                     aligned16(x, ldx, 2), codes, scales, st, g_dev);
  }
  return hip_status(e, "dynamic quant launch");
}

}  // extern "C"

namespace {

int linear_nvfp4_extras(const void* x, int64_t M, int64_t K, int64_t ldx, float g, const void* T,
                        int b, const void* w_packed, int64_t N, float alpha, float g_w,
                        bool dynamic, const void* bias, void* y, int64_t ldy, void* workspace,
                        size_t workspace_bytes, void* stream) {
  if (int r = check_nvfp4_shape(M, K, ldx, T ? 0 : b, "M")) return r;
  if (T) {
    if (int r = check_transform(T, b, K)) return r;
  }
  if (dynamic) {
    if (int r = check_scale(g_w, "weight_global_scale")) return r;
  } else {
    if (int r = check_scale(g, "input_global_scale")) return r;
    if (!std::isfinite(alpha)) return fail(FQL_ERR_INVALID, "alpha must be finite");
  }
  if (N < 1 || N > (int64_t)1 << 24) return fail(FQL_ERR_INVALID, "N out of range");
  if (ldy < N) return fail(FQL_ERR_INVALID, "ldy %lld is smaller than N %lld", (long long)ldy, (long long)N);
  if (!x || !w_packed || !y || !workspace) return fail(FQL_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(w_packed) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(FQL_ERR_INVALID, "packed weight must be 16-byte and workspace 256-byte aligned");
  // a plan whose quantizer pass writes the GEMM's operand (x_hat or the packed
  // activation), since the fused small-M kernel quantizes with a host-side scale
  const fql::GemmPlan plan = fql::cached_plan_gemm_nvfp4(M, N, K, false, false);
  if (workspace_bytes < (size_t)plan.total_bytes)
    return fail(FQL_ERR_WORKSPACE, "workspace holds %zu bytes, %lld needed", workspace_bytes,
                (long long)plan.total_bytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* scal = reinterpret_cast<float*>(ws + fql::kWorkspaceScalarOffset);
  fql::LinearExtras ex{};
  ex.T = static_cast<const uint16_t*>(T);
  ex.t_aligned = T ? fql::transform_aligned(x, ldx, b) : false;
  if (dynamic) {
    static_assert(fql::kDynScalarWords * 4 <= fql::kWorkspaceScalarBytes, "workspace scalar region");
    hipError_t e = launch_dynamic_prologue(x, M, K, ldx, T, b, scal, g_w, true, st);
    if (e != hipSuccess) return hip_status(e, "dynamic scale launch");
    ex.g_dev = scal + fql::kAmaxSlots + 1;
    ex.alpha_dev = scal + fql::kAmaxSlots + 2;
    g = 1.0f;
    alpha = 1.0f;
  }
  hipError_t e = fql::launch_linear_nvfp4(
      plan, static_cast<const uint16_t*>(x), M, K, ldx, g, b, aligned16(x, ldx, 2),
      static_cast<const uint8_t*>(w_packed), N, alpha, static_cast<const uint16_t*>(bias),
      static_cast<uint16_t*>(y), ldy, ws, st, &ex);
  return hip_status(e, "linear launch");
}

}  // namespace

extern "C" {

int fql_linear_nvfp4_transform(const void* x, int64_t M, int64_t K, int64_t ldx,
                               float input_global_scale, const void* T, int b,
                               const void* w_packed, int64_t N, float alpha, const void* bias,
                               void* y, int64_t ldy, void* workspace, size_t workspace_bytes,
                               void* stream) {
  if (!T) return fail(FQL_ERR_INVALID, "null transform matrix");
  return linear_nvfp4_extras(x, M, K, ldx, input_global_scale, T, b, w_packed, N, alpha, 0.0f,
                             false, bias, y, ldy, workspace, workspace_bytes, stream);
}

int fql_linear_nvfp4_dynamic(const void* x, int64_t M, int64_t K, int64_t ldx, const void* T,
                             int b, const void* w_packed, int64_t N, float weight_global_scale,
                             const void* bias, void* y, int64_t ldy, void* workspace,
                             size_t workspace_bytes, void* stream) {
  return linear_nvfp4_extras(x, M, K, ldx, 0.0f, T, b, w_packed, N, 0.0f, weight_global_scale,
                             true, bias, y, ldy, workspace, workspace_bytes, stream);
}

// ---- scaled-MFMA formats: MXFP4, MXFP8, per-tensor FP8, block FP8 -------------

}  // extern "C"

namespace {

const char* sc_name(int fmt) {
  return fmt == fql::SC_MXFP4 ? "MXFP4" : fmt == fql::SC_MXFP8 ? "MXFP8" : fmt == fql::SC_FP8 ? "FP8" : "block FP8";
}

// K granularity: 32 (MX block; per-tensor FP8 follows the same operand
// granularity) or 128 (block FP8 group).
int64_t sc_kmult(int fmt) { return fmt == fql::SC_FP8_BLOCK ? 128 : 32; }

int check_sc_shape(int fmt, int64_t rows, int64_t K, int64_t ld, const char* rows_name, bool weight) {
  if (rows < 1) return fail(FQL_ERR_INVALID, "%s must be >= 1 (got %lld)", rows_name, (long long)rows);
  const int64_t km = sc_kmult(fmt);
  if (K < km || K % km != 0)
    return fail(FQL_ERR_INVALID, "%s needs K a positive multiple of %lld (got %lld)", sc_name(fmt),
                (long long)km, (long long)K);
  if (weight && fmt == fql::SC_FP8_BLOCK && rows % 128 != 0)
    return fail(FQL_ERR_INVALID, "block FP8 needs N a multiple of 128 (got %lld)", (long long)rows);
  if (ld < K) return fail(FQL_ERR_INVALID, "row stride %lld is smaller than K %lld", (long long)ld, (long long)K);
  if (K > (int64_t)1 << 24 || rows > (int64_t)1 << 24) return fail(FQL_ERR_INVALID, "dimension too large");
  if (rows * (fql::round_up(K, 128) / 32) > ((int64_t)1 << 31) - 4096)
    return fail(FQL_ERR_INVALID, "too many 32-element blocks");
  return FQL_OK;
}

int sc_quant(int fmt, bool f32_input, bool weight_tiles, const void* x, int64_t rows, int64_t K,
             int64_t ld, float scale, uint8_t* codes, void* scales, void* stream) {
  if (int r = check_sc_shape(fmt, rows, K, ld, weight_tiles ? "N" : "M", weight_tiles)) return r;
  if (!x || !codes || (fmt != fql::SC_FP8 && !scales)) return fail(FQL_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(codes) % 4 != 0 ||
      (fmt == fql::SC_FP8_BLOCK && reinterpret_cast<uintptr_t>(scales) % 4 != 0))
    return fail(FQL_ERR_INVALID, "codes (and float scales) must be 4-byte aligned");
  float inv = 0.0f;
  if (fmt == fql::SC_FP8) {
    if (int r = check_scale(scale, "scale")) return r;
    inv = std::fmin(1.0f / scale, 3.4028234663852886e38f);  // fl32(1/s), finite
  }
  return hip_status(fql::launch_sc_quant(fmt, f32_input, weight_tiles, x, rows, K, ld, inv, codes,
                                         scales, static_cast<hipStream_t>(stream)),
                    "quant launch");
}

int sc_packed_bytes(int fmt, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(FQL_ERR_INVALID, "null pointer");
  if (int r = check_sc_shape(fmt, N, K, K, "N", true)) return r;
  *bytes = (size_t)fql::sc_dims(fmt, N, K, true).total_bytes();
  return ok();
}

int sc_pack(int fmt, const uint8_t* codes, const void* scales, int64_t N, int64_t K, void* packed,
            size_t packed_bytes, void* stream) {
  if (int r = check_sc_shape(fmt, N, K, K, "N", true)) return r;
  if (!codes || !packed || (fmt != fql::SC_FP8 && !scales)) return fail(FQL_ERR_INVALID, "null pointer");
  const size_t need = (size_t)fql::sc_dims(fmt, N, K, true).total_bytes();
  if (packed_bytes < need)
    return fail(FQL_ERR_INVALID, "packed buffer holds %zu bytes, %zu needed", packed_bytes, need);
  if (reinterpret_cast<uintptr_t>(packed) % 16 != 0 || reinterpret_cast<uintptr_t>(codes) % 16 != 0)
    return fail(FQL_ERR_INVALID, "codes and the packed buffer must be 16-byte aligned");
  if (fmt == fql::SC_FP8_BLOCK && reinterpret_cast<uintptr_t>(scales) % 4 != 0)
    return fail(FQL_ERR_INVALID, "scales must be 4-byte aligned");
  return hip_status(fql::launch_sc_pack(fmt, codes, scales, N, K, static_cast<uint8_t*>(packed),
                                        static_cast<hipStream_t>(stream)),
                    "pack launch");
}

int sc_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, size_t* bytes) {
  if (!bytes) return fail(FQL_ERR_INVALID, "null pointer");
  if (int r = check_sc_shape(fmt, N, K, K, "N", true)) return r;
  if (M < 1) return fail(FQL_ERR_INVALID, "M must be >= 1");
  *bytes = (size_t)fql::cached_plan_sc_gemm(fmt, M, N, K).total_bytes;
  return ok();
}

int sc_describe(int fmt, int64_t M, int64_t N, int64_t K, char* buf, size_t len) {
  if (int r = check_sc_shape(fmt, N, K, K, "N", true)) return r;
  if (M < 1) return fail(FQL_ERR_INVALID, "M must be >= 1");
  write_reason(buf, len, fql::describe_sc_plan(fql::plan_sc_gemm(fmt, M, N, K)));
  return ok();
}

int sc_linear(int fmt, const void* x, int64_t M, int64_t K, int64_t ldx, float input_scale,
              const void* w_packed, int64_t N, float alpha, const void* bias, void* y, int64_t ldy,
              void* workspace, size_t workspace_bytes, void* stream,
              const float* alpha_dev = nullptr) {
  if (int r = check_sc_shape(fmt, M, K, ldx, "M", false)) return r;
  if (int r = check_sc_shape(fmt, N, K, K, "N", true)) return r;
  if (!std::isfinite(alpha)) return fail(FQL_ERR_INVALID, "alpha must be finite");
  float inv = 0.0f;
  if (fmt == fql::SC_FP8) {
    if (int r = check_scale(input_scale, "input_scale")) return r;
    inv = std::fmin(1.0f / input_scale, 3.4028234663852886e38f);
  }
  if (ldy < N) return fail(FQL_ERR_INVALID, "ldy %lld is smaller than N %lld", (long long)ldy, (long long)N);
  if (!x || !w_packed || !y || !workspace) return fail(FQL_ERR_INVALID, "null pointer");
  if (reinterpret_cast<uintptr_t>(w_packed) % 16 != 0 ||
      reinterpret_cast<uintptr_t>(workspace) % 256 != 0)
    return fail(FQL_ERR_INVALID, "packed weight must be 16-byte and workspace 256-byte aligned");
  const fql::ScPlan plan = fql::cached_plan_sc_gemm(fmt, M, N, K);
  if (workspace_bytes < (size_t)plan.total_bytes)
    return fail(FQL_ERR_WORKSPACE, "workspace holds %zu bytes, %lld needed", workspace_bytes,
                (long long)plan.total_bytes);
  if (plan.splits > 1 && plan.groups > plan.counter_bytes / 4)
    return fail(FQL_ERR_INVALID, "too many output tiles for the arrival counters");
  if (plan.Mp * (plan.groups > 0 ? fql::round_up(K, 128) / 32 : 0) > ((int64_t)1 << 31) - 4096)
    return fail(FQL_ERR_INVALID, "activation too large");
  hipError_t e = fql::launch_sc_linear(
      plan, static_cast<const uint16_t*>(x), M, K, ldx, aligned16(x, ldx, 2), inv,
      static_cast<const uint8_t*>(w_packed), N, alpha, alpha_dev, static_cast<const uint16_t*>(bias),
      static_cast<uint16_t*>(y), ldy, static_cast<uint8_t*>(workspace), static_cast<hipStream_t>(stream));
  return hip_status(e, "linear launch");
}

}  // namespace

extern "C" {

// MXFP4
int fql_quant_mxfp4(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                    uint8_t* scales, void* stream) {
  return sc_quant(fql::SC_MXFP4, false, false, x, M, K, ldx, 0.0f, codes, scales, stream);
}
int fql_quant_mxfp4_f32(const float* w, int64_t N, int64_t K, int64_t ldw, uint8_t* codes,
                        uint8_t* scales, void* stream) {
  return sc_quant(fql::SC_MXFP4, true, false, w, N, K, ldw, 0.0f, codes, scales, stream);
}
int fql_packed_mxfp4_bytes(int64_t N, int64_t K, size_t* bytes) {
  return sc_packed_bytes(fql::SC_MXFP4, N, K, bytes);
}
int fql_pack_weight_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                          void* packed, size_t packed_bytes, void* stream) {
  return sc_pack(fql::SC_MXFP4, codes, scales, N, K, packed, packed_bytes, stream);
}
int fql_linear_mxfp4_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  return sc_workspace_bytes(fql::SC_MXFP4, M, N, K, bytes);
}
int fql_linear_mxfp4_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len) {
  return sc_describe(fql::SC_MXFP4, M, N, K, buf, buf_len);
}
int fql_linear_mxfp4(const void* x, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                     int64_t N, float alpha, const void* bias, void* y, int64_t ldy,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return sc_linear(fql::SC_MXFP4, x, M, K, ldx, 1.0f, w_packed, N, alpha, bias, y, ldy, workspace,
                   workspace_bytes, stream);
}

// MXFP8
int fql_quant_mxfp8(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                    uint8_t* scales, void* stream) {
  return sc_quant(fql::SC_MXFP8, false, false, x, M, K, ldx, 0.0f, codes, scales, stream);
}
int fql_quant_mxfp8_f32(const float* w, int64_t N, int64_t K, int64_t ldw, uint8_t* codes,
                        uint8_t* scales, void* stream) {
  return sc_quant(fql::SC_MXFP8, true, false, w, N, K, ldw, 0.0f, codes, scales, stream);
}
int fql_packed_mxfp8_bytes(int64_t N, int64_t K, size_t* bytes) {
  return sc_packed_bytes(fql::SC_MXFP8, N, K, bytes);
}
int fql_pack_weight_mxfp8(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                          void* packed, size_t packed_bytes, void* stream) {
  return sc_pack(fql::SC_MXFP8, codes, scales, N, K, packed, packed_bytes, stream);
}
int fql_linear_mxfp8_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  return sc_workspace_bytes(fql::SC_MXFP8, M, N, K, bytes);
}
int fql_linear_mxfp8_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len) {
  return sc_describe(fql::SC_MXFP8, M, N, K, buf, buf_len);
}
int fql_linear_mxfp8(const void* x, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                     int64_t N, float alpha, const void* bias, void* y, int64_t ldy,
                     void* workspace, size_t workspace_bytes, void* stream) {
  return sc_linear(fql::SC_MXFP8, x, M, K, ldx, 1.0f, w_packed, N, alpha, bias, y, ldy, workspace,
                   workspace_bytes, stream);
}

// per-tensor FP8
int fql_quant_fp8(const void* x, int64_t M, int64_t K, int64_t ldx, float scale, uint8_t* codes,
                  void* stream) {
  return sc_quant(fql::SC_FP8, false, false, x, M, K, ldx, scale, codes, nullptr, stream);
}
int fql_quant_fp8_f32(const float* w, int64_t N, int64_t K, int64_t ldw, float scale,
                      uint8_t* codes, void* stream) {
  return sc_quant(fql::SC_FP8, true, false, w, N, K, ldw, scale, codes, nullptr, stream);
}
int fql_packed_fp8_bytes(int64_t N, int64_t K, size_t* bytes) {
  return sc_packed_bytes(fql::SC_FP8, N, K, bytes);
}
int fql_pack_weight_fp8(const uint8_t* codes, int64_t N, int64_t K, void* packed,
                        size_t packed_bytes, void* stream) {
  return sc_pack(fql::SC_FP8, codes, nullptr, N, K, packed, packed_bytes, stream);
}
int fql_linear_fp8_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  return sc_workspace_bytes(fql::SC_FP8, M, N, K, bytes);
}
int fql_linear_fp8_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len) {
  return sc_describe(fql::SC_FP8, M, N, K, buf, buf_len);
}
int fql_linear_fp8(const void* x, int64_t M, int64_t K, int64_t ldx, float input_scale,
                   const void* w_packed, int64_t N, float alpha, const void* bias, void* y,
                   int64_t ldy, void* workspace, size_t workspace_bytes, void* stream) {
  return sc_linear(fql::SC_FP8, x, M, K, ldx, input_scale, w_packed, N, alpha, bias, y, ldy,
                   workspace, workspace_bytes, stream);
}

int fql_linear_fp8_dev_alpha(const void* x, int64_t M, int64_t K, int64_t ldx, float input_scale,
                             const void* w_packed, int64_t N, const float* alpha_dev,
                             const void* bias, void* y, int64_t ldy, void* workspace,
                             size_t workspace_bytes, void* stream) {
  if (!alpha_dev || reinterpret_cast<uintptr_t>(alpha_dev) % 4 != 0)
    return fail(FQL_ERR_INVALID, "alpha_dev must be a 4-byte aligned device pointer");
  return sc_linear(fql::SC_FP8, x, M, K, ldx, input_scale, w_packed, N, 0.0f, bias, y, ldy,
                   workspace, workspace_bytes, stream, alpha_dev);
}

// block FP8
int fql_quant_fp8_block(const void* x, int64_t M, int64_t K, int64_t ldx, uint8_t* codes,
                        float* scales, void* stream) {
  return sc_quant(fql::SC_FP8_BLOCK, false, false, x, M, K, ldx, 0.0f, codes, scales, stream);
}
int fql_quant_fp8_block_weight_f32(const float* w, int64_t N, int64_t K, int64_t ldw,
                                   uint8_t* codes, float* scales, void* stream) {
  return sc_quant(fql::SC_FP8_BLOCK, true, true, w, N, K, ldw, 0.0f, codes, scales, stream);
}
int fql_packed_fp8_block_bytes(int64_t N, int64_t K, size_t* bytes) {
  return sc_packed_bytes(fql::SC_FP8_BLOCK, N, K, bytes);
}
int fql_pack_weight_fp8_block(const uint8_t* codes, const float* scales, int64_t N, int64_t K,
                              void* packed, size_t packed_bytes, void* stream) {
  return sc_pack(fql::SC_FP8_BLOCK, codes, scales, N, K, packed, packed_bytes, stream);
}
int fql_linear_fp8_block_workspace_bytes(int64_t M, int64_t N, int64_t K, size_t* bytes) {
  return sc_workspace_bytes(fql::SC_FP8_BLOCK, M, N, K, bytes);
}
int fql_linear_fp8_block_describe(int64_t M, int64_t N, int64_t K, char* buf, size_t buf_len) {
  return sc_describe(fql::SC_FP8_BLOCK, M, N, K, buf, buf_len);
}
int fql_linear_fp8_block(const void* x, int64_t M, int64_t K, int64_t ldx, const void* w_packed,
                         int64_t N, float alpha, const void* bias, void* y, int64_t ldy,
                         void* workspace, size_t workspace_bytes, void* stream) {
  return sc_linear(fql::SC_FP8_BLOCK, x, M, K, ldx, 1.0f, w_packed, N, alpha, bias, y, ldy,
                   workspace, workspace_bytes, stream);
}

}  // extern "C"
// ---- linear call without allocation: a static scratch buffer per device ------
//
// For callers that cannot allocate (code under HIP graph capture, tight
// serving loops): fql_linear_nvfp4_noalloc runs the same plan and kernels as
// fql_linear_nvfp4 with the workspace in a file-scope device array. In host
// code `scratch` names a host-side stand-in, never the device memory; its
// device address comes from hipGetSymbolAddress, once per device (each GPU
// holds its own copy), and only that address reaches kernels.

namespace {

constexpr size_t kNoAllocScratchBytes = FQL_NOALLOC_SCRATCH_BYTES;
static_assert(fql::kWorkspaceCounterBytes % 4 == 0, "counter words");

__device__ __align__(256) uint8_t scratch[kNoAllocScratchBytes];

__global__ void clear_words_kernel(uint32_t* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// The device address of this device's scratch, set up on the first call on
// the device: the address is looked up and the arrival counters at its start
// are cleared in stream order (every linear call leaves them zero again).
int scratch_for_current_device(hipStream_t st, uint8_t** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_status(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return fail(FQL_ERR_UNSUPPORTED, "device index %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return hip_status(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    const int words = (int)(fql::kWorkspaceCounterBytes / 4);
    clear_words_kernel<<<(words + 255) / 256, 256, 0, st>>>(static_cast<uint32_t*>(p), words);
    e = hipGetLastError();
    if (e != hipSuccess) return hip_status(e, "scratch clear launch");
    g_scratch_ptr[dev] = static_cast<uint8_t*>(p);
  }
  *out = g_scratch_ptr[dev];
  return FQL_OK;
}

}  // namespace

extern "C" {

int fql_linear_nvfp4_noalloc(const void* x, int64_t M, int64_t K, int64_t ldx,
                             float input_global_scale, int hadamard_block, const void* w_packed,
                             int64_t N, float alpha, const void* bias, void* y, int64_t ldy,
                             void* stream) {
  if (int r = check_linear_nvfp4(x, M, K, ldx, input_global_scale, hadamard_block, w_packed, N, y, ldy))
    return r;
  if (!std::isfinite(alpha)) return fail(FQL_ERR_INVALID, "alpha must be finite");
  const bool xal = aligned16(x, ldx, 2);
  const fql::GemmPlan plan = fql::cached_plan_gemm_nvfp4(M, N, K, xal, hadamard_block > 0);
  if ((size_t)plan.total_bytes > kNoAllocScratchBytes)
    return fail(FQL_ERR_WORKSPACE,
                "this call needs %lld bytes of scratch, more than the %zu bytes the "
                "allocation-free entry point holds per device; use fql_linear_nvfp4 with a workspace",
                (long long)plan.total_bytes, kNoAllocScratchBytes);
  hipStream_t st = static_cast<hipStream_t>(stream);
  uint8_t* ws = nullptr;
  if (int r = scratch_for_current_device(st, &ws)) return r;
  hipError_t e = fql::launch_linear_nvfp4(
      plan, static_cast<const uint16_t*>(x), M, K, ldx, input_global_scale, hadamard_block, xal,
      static_cast<const uint8_t*>(w_packed), N, alpha, static_cast<const uint16_t*>(bias),
      static_cast<uint16_t*>(y), ldy, ws, st);
  return hip_status(e, "linear launch");
}

}  // extern "C"
