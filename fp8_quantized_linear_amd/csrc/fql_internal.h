// Internal declarations shared by the library's translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

namespace fql {

// ---- packed NVFP4 weight layout -------------------------------------------
// N is padded to a multiple of 16 (one MFMA tile of output columns) and K to
// a multiple of 128 (four 32-deep MFMA steps, "a chunk"). The blob holds the
// code region followed by the scale region:
//   codes  [Np/16][KC][lane 64][16 bytes]        KC = Kp/128, lane = kq*16 + n
//          dword j of a lane = the eight codes of row n at k = 128c + 32j + 8kq + 0..7,
//          element i in nibble i (canonical nibble order).
//   scales [Np/16][KC4][slot 32][16 bytes]       KC4 = ceil(KC/4), slot = n*2 + h
//          byte 4q + j = scale of row n, block 8c + 2j + h, for chunk c = 4*group + q
//          (zero for chunks past KC).
// One 16-byte load per lane gives the B-operand codes of four MFMA steps of
// one chunk, and one 16-byte load per lane the scales of four chunks
// (lane = kq*16 + n reads slot n*2 + kq/2), so a wave issues a few large
// requests instead of many small ones.
struct PackedDims {
  int64_t Np, Kp;
  int64_t kc() const { return Kp / 128; }
  int64_t kc4() const { return (Kp / 128 + 3) / 4; }
  int64_t code_bytes() const { return Np * Kp / 2; }
  int64_t scale_bytes() const { return (Np / 16) * kc4() * 512; }
  int64_t total_bytes() const { return code_bytes() + scale_bytes(); }
};

inline int64_t round_up(int64_t v, int64_t m) { return (v + m - 1) / m * m; }
inline PackedDims packed_dims(int64_t N, int64_t K) { return PackedDims{round_up(N, 16), round_up(K, 128)}; }

// ---- launch-plan overrides -------------------------------------------------
// Benchmarking aid: a spec that replaces the plan heuristics (results change
// at most in the order of the float32 sum over K). Each starts as the
// environment variable FQL_PLAN, FQL_SC_PLAN or FQL_SC_GEMV, read once, and
// can be replaced at run time (fql_set_plan_override); every change bumps a
// generation number that invalidates the plan caches.
enum PlanOverrideKind { kOverrideNvfp4 = 0, kOverrideScGemm = 1, kOverrideScGemv = 2 };
std::string plan_override(int which);  // "" when unset
void set_plan_override(int which, const char* spec);
uint32_t plan_generation();

// ---- launchers (stream-ordered, return the launch status) -----------------
hipError_t launch_quant_nvfp4_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float g,
                                   int hb, bool aligned, uint8_t* codes, uint8_t* scales,
                                   hipStream_t st, const float* g_dev = nullptr);
hipError_t launch_quant_nvfp4_f32(const float* w, int64_t N, int64_t K, int64_t ldw, float g,
                                  int hb, bool aligned, uint8_t* codes, uint8_t* scales,
                                  hipStream_t st);
hipError_t launch_quant_nvfp4_xhat(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float g,
                                   int hb, bool aligned, int64_t Mp, int64_t Kp, _Float16* xhat,
                                   const float* g_dev, hipStream_t st);
// The same quantization written as a packed operand (the packed weight layout
// with Mp rows): codes [Mp/16][Kp/128][64][16 B], then scales; Mp % 16 == 0.
hipError_t launch_quant_nvfp4_apack(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float g,
                                    int hb, bool aligned, int64_t Mp, int64_t Kp, uint8_t* apack,
                                    const float* g_dev, hipStream_t st);
// max |v| into out (one float, or nslots partial maxima that launch_dynamic_scale folds)
hipError_t launch_amax_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int hb,
                            bool aligned, float* out, hipStream_t st, int nslots = 1);
hipError_t launch_amax_f32(const float* w, int64_t N, int64_t K, int64_t ldw, int hb, bool aligned,
                           float* out, hipStream_t st);

hipError_t launch_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                             uint8_t* packed, hipStream_t st);
hipError_t launch_unpack_nvfp4(const uint8_t* packed, int64_t N, int64_t K, uint8_t* codes,
                               uint8_t* scales, hipStream_t st);

// Launch plan of one linear call for (M, N, K).
//   kind 0: small M (M <= 16 and M*Kp*2 <= 64 KiB): one launch; each
//           workgroup quantizes the activation into LDS and computes one
//           16-column tile over the full K, its waves splitting K.
//   kind 1: quantizer kernel (x_hat in A-fragment order) + tiled GEMM.
//   kind 3: quantizer kernel + LDS-ring tiled GEMM on 32x32x16 MFMAs (direct
//           global->LDS loads; mt, nt count 32-row / 32-column tiles).
//   kind 4: quantizer kernel (packed activation) + per-wave-ring small-M GEMM.
// Workspace layout: [arrival counters | x_hat | split-K partial slabs]. The
// counters must be zero before the first call on a workspace; every call
// leaves them zero again.
struct GemmPlan {
  int kind;
  int mt;             // kind 1: 16-row M tiles per wave
  int nt;             // kind 1: 16-column N tiles per wave
  int wm;             // kind 1: wave rows (the 4 waves form a wm x 4/wm grid)
  int st;             // kinds 3, 4: LDS ring depth (chunks)
  int64_t Mp;         // M padded to a whole number of M tiles
  int64_t Np, Kp;     // packed weight dims
  int64_t groups;     // output tiles
  int64_t ngroups;    // column groups (kind 1)
  int splits;         // K splits of the split tiles (1 = epilogue directly in the GEMM)
  int kc_per_split;   // 128-deep K chunks per split
  int64_t dp_groups;  // kind 3: tiles computed whole, one workgroup each (the first
                      // dp_groups workgroups); the other groups - dp_groups tiles
                      // take `splits` consecutive workgroups each
  int kcmax;          // kind 0: weight register ring depth in chunks (4 or 8)
  int waves;          // kind 0: waves per workgroup (split of K inside the workgroup)
  int qpre;           // kind 0: activation blocks per thread loaded ahead of the weights
  int ntw;            // kind 0: 16-column tiles per workgroup
  int64_t lds_bytes;  // kind 0: dynamic LDS (compact activation copy / reduction)
  int cw;             // kind 3: column waves (4 or 8)
  int xg;             // kind 3, one K split: XCD-grouped tile order in bands of xg
                      // row groups (0: row-major order of the output tiles)
  int64_t counter_bytes, xhat_bytes, partial_bytes, total_bytes;
};
// `aligned`: x rows are 16-byte aligned (pointer and row stride); the
// fused small-M kernel needs it. Workspace sizes of both kinds are covered by
// the aligned=false plan, which never needs less. `rotated`: the call applies
// a block Hadamard transform to the activation (hadamard_block > 0); it only
// changes the column tiles per workgroup of the fused kernel, never the kind
// or the workspace.
GemmPlan plan_gemm_nvfp4(int64_t M, int64_t N, int64_t K, bool aligned, bool rotated);
// The same plan from a small per-thread cache (keyed by the shape, the
// alignment, the rotation and the override generation), so a hot call plans
// once per shape.
GemmPlan cached_plan_gemm_nvfp4(int64_t M, int64_t N, int64_t K, bool aligned, bool rotated);

// Whether gemm_tiled_kernel<mt, nt, wm> / gemm_lds32_kernel<mt, nt, st> is
// built into the library.
bool tiled_config_built(int mt, int nt, int wm);
bool lds32_config_built(int mt, int nt, int st, int cw);
bool gemv_ring_config_built(int w, int mt, int nt, int d);

// Kernel name and parameters of a plan (diagnostics).
std::string describe_plan(const GemmPlan& p);

// ---- general block-diagonal transform + dynamic global scale ---------------
// Device scalars of the dynamic-scale path (float words):
//   [0, kAmaxSlots)  partial maxima (uint bits), one per group of workgroups
//   kAmaxSlots       the tensor amax, then g_x, then alpha.
// The linear call keeps them in the last kWorkspaceScalarBytes of the
// workspace's kWorkspaceCounterBytes of split-K arrival counters.
constexpr int kAmaxSlots = 64;
constexpr int kDynScalarWords = kAmaxSlots + 3;
constexpr int64_t kWorkspaceCounterBytes = 64 * 1024;
constexpr int64_t kWorkspaceScalarBytes = 512;
constexpr int64_t kWorkspaceScalarOffset = kWorkspaceCounterBytes - kWorkspaceScalarBytes;

// One launch of the transform kernel. mode 0: canonical codes [M][K/2] and
// scales [M][K/16]; 1: x_hat (float16, GEMM A-fragment order, rows_out = Mp
// rows and Kp columns, zero padded); 2: max |v| into the kAmaxSlots partial
// maxima at amax (zeroed first); 3: float32 values v [M][ldv]; 4: the packed
// activation (the packed weight layout with rows_out = Mp rows, a multiple of
// 16, and Kp columns, zero padded) at xhat.
struct TransformArgs {
  int mode;
  const uint16_t* x;
  int64_t M, K, ldx;
  bool aligned;         // transform_aligned(x, ldx, b)
  const uint16_t* T;    // bf16 [b][b], 16-byte aligned
  int b;
  float g;
  const float* g_dev;   // non-null: g read from device memory
  uint8_t* codes;
  uint8_t* scales;
  _Float16* xhat;
  int64_t rows_out, Kp;
  float* v;
  int64_t ldv;
  uint32_t* amax;
};
bool transform_aligned(const void* x, int64_t ldx, int b);
hipError_t launch_transform_nvfp4(const TransformArgs& a, hipStream_t st);
// scal[kAmaxSlots] = max of the partial maxima, scal[kAmaxSlots + 1] =
// g = fl32(2688 / amax) (1 when amax = 0, at most 2^118), and, when
// with_alpha, scal[kAmaxSlots + 2] = alpha = fl32((1/g) * (1/g_w)).
hipError_t launch_dynamic_scale(float* scal, float g_w, bool with_alpha, hipStream_t st);
hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t st);

// Optional parts of a linear call: a general transform T (b = hb) in place
// of the Hadamard rotation (needs a plan with a quantizer pass: the
// aligned = false plan), and device-resident g / alpha (any plan).
struct LinearExtras {
  const uint16_t* T;
  bool t_aligned;
  const float* g_dev;
  const float* alpha_dev;
};

hipError_t launch_linear_nvfp4(const GemmPlan& p, const uint16_t* x, int64_t M, int64_t K,
                               int64_t ldx, float g, int hb, bool aligned, const uint8_t* packed,
                               int64_t N, float alpha, const uint16_t* bias, uint16_t* y,
                               int64_t ldy, uint8_t* workspace, hipStream_t st,
                               const LinearExtras* ex = nullptr);
// The two halves of launch_linear_nvfp4 for plans with a quantizer pass
// (has_quant_pass): the quantizer writes the activation operand into the
// workspace, the GEMM reads it. Both together equal one launch_linear_nvfp4.
bool has_quant_pass(const GemmPlan& p);
hipError_t launch_linear_quant(const GemmPlan& p, const uint16_t* x, int64_t M, int64_t K,
                               int64_t ldx, float g, int hb, bool aligned, uint8_t* workspace,
                               hipStream_t st, const LinearExtras* ex = nullptr);
hipError_t launch_linear_gemm(const GemmPlan& p, const uint8_t* packed, int64_t M, int64_t N,
                              float alpha, const uint16_t* bias, uint16_t* y, int64_t ldy,
                              uint8_t* workspace, hipStream_t st, const LinearExtras* ex = nullptr);

// ---- scaled-MFMA formats: MXFP4, MXFP8, per-tensor FP8, block FP8 ---------
// All four run on v_mfma_scale_f32_16x16x128_f8f6f4 (one instruction per
// 16x16 output tile and 128-deep "chunk" of K). Operand layout, shared by the
// quantized activation (workspace) and the packed weight; rows padded to 16,
// K to 128:
//   codes [rows_p/16][KC][H halves][lane 64][16 B]   H = 1 (FP4) or 2 (FP8)
//     FP4: lane l holds row l%16, k = 128c + 32(l/16) + i in nibble i.
//     FP8: half h of lane l holds row l%16, k = 128c + 64h + 16(l/16) + i in byte i.
//   MX scales (E8M0) [quads][KC][lane 64][4 B], quads = ceil(rows_p/64):
//     byte q of lane l = scale of row 64*quad + 16q + l%16, 32-block 4c + l/16
//     (the MFMA takes the scale of row r, block j from lane 16j + r).
//   block-FP8 activation row scales (float32) [quads][KC][row 64].
//   block-FP8 weight scales (float32) [N/128][KC], after the weight codes.
enum ScFmt { SC_MXFP4 = 0, SC_MXFP8 = 1, SC_FP8 = 2, SC_FP8_BLOCK = 3 };

struct ScDims {
  int64_t rows_p, Kp, KC, quads, code_bytes, scale_bytes;
  int64_t total_bytes() const { return code_bytes + scale_bytes; }
};
// Layout sizes of an operand of `rows` x K; `weight` selects the packed-weight
// scale region (block FP8: [N/128][KC] floats) over the activation one.
ScDims sc_dims(int fmt, int64_t rows, int64_t K, bool weight);

// Workspace: [64 KiB arrival counters | activation codes | activation scales | split-K slabs].
struct ScPlan {
  int fmt;
  int kind;                  // 0: LDS-ring GEMM, 1: register-streaming GEMV (small M)
  int wm, wn, mtw, ntw, st;  // GEMM: wave grid, 16x16 tiles per wave, LDS ring depth;
                             // GEMV: wn = waves splitting K, mtw = row tiles,
                             //       ntw = column tiles per workgroup, st = chunks in flight
  int64_t Mp, groups, ngroups;
  int splits, kc_per_split;  // K splits of the split tiles, chunks per split
  int64_t dp_groups;         // GEMM: tiles computed whole (the first dp_groups workgroups);
                             // the others take `splits` consecutive workgroups each
  int64_t counter_bytes, xcode_bytes, xscale_bytes, partial_bytes, total_bytes;
  int fq;           // GEMV: activation quantized inside the workgroups (one launch)
  int64_t dyn_lds;  // GEMV with fq: dynamic LDS bytes (the activation operand)
};
ScPlan plan_sc_gemm(int fmt, int64_t M, int64_t N, int64_t K);
ScPlan cached_plan_sc_gemm(int fmt, int64_t M, int64_t N, int64_t K);
std::string describe_sc_plan(const ScPlan& p);

// Canonical quantizers: codes [rows][K/2] (FP4) or [rows][K] (FP8);
// scales: MX [rows][K/32] bytes, block FP8 [rows][K/128] floats (activation)
// or [rows/128][K/128] floats (weight, f32 input only), per-tensor none
// (`inv_scale` = fl32(1/s) is applied instead).
hipError_t launch_sc_quant(int fmt, bool f32_input, bool weight_tiles, const void* x, int64_t rows,
                           int64_t K, int64_t ld, float inv_scale, uint8_t* codes, void* scales,
                           hipStream_t st);
// Canonical weight -> packed operand layout.
hipError_t launch_sc_pack(int fmt, const uint8_t* codes, const void* scales, int64_t N, int64_t K,
                          uint8_t* packed, hipStream_t st);
// Activation quantize (straight into the operand layout) + GEMM + epilogue.
// alpha_dev (nullable): the output scale read from device memory instead of alpha.
hipError_t launch_sc_linear(const ScPlan& p, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            bool aligned, float inv_scale, const uint8_t* packed, int64_t N,
                            float alpha, const float* alpha_dev, const uint16_t* bias, uint16_t* y,
                            int64_t ldy, uint8_t* workspace, hipStream_t st);
// Activation operand quantizer used by launch_sc_linear.
hipError_t launch_sc_quant_operand(int fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   bool aligned, float inv_scale, int64_t Mp, uint8_t* codes,
                                   void* scales, hipStream_t st);

}  // namespace fql
