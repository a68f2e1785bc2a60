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

// ---- launchers (stream-ordered, return the launch status) -----------------
hipError_t launch_quant_nvfp4_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float g,
                                   int hb, bool aligned, uint8_t* codes, uint8_t* scales,
                                   hipStream_t st);
hipError_t launch_quant_nvfp4_f32(const float* w, int64_t N, int64_t K, int64_t ldw, float g,
                                  int hb, bool aligned, uint8_t* codes, uint8_t* scales,
                                  hipStream_t st);
hipError_t launch_quant_nvfp4_xhat(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float g,
                                   int hb, bool aligned, int64_t Mp, int64_t Kp, _Float16* xhat,
                                   hipStream_t st);
hipError_t launch_amax_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int hb,
                            bool aligned, float* out, hipStream_t st);
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
//   kind 2: quantizer kernel + LDS-ring tiled GEMM (direct global->LDS loads).
//   kind 3: as kind 2 on 32x32x16 MFMAs (mt, nt count 32-row / 32-column tiles).
// Workspace layout: [arrival counters | x_hat | split-K partial slabs]. The
// counters must be zero before the first call on a workspace; every call
// leaves them zero again.
struct GemmPlan {
  int kind;
  int mt;             // kind 1: 16-row M tiles per wave
  int nt;             // kind 1: 16-column N tiles per wave
  int wm;             // kind 1: wave rows (the 4 waves form a wm x 4/wm grid)
  int st;             // kind 2: LDS ring depth (chunks)
  int64_t Mp;         // M padded to a whole number of M tiles
  int64_t Np, Kp;     // packed weight dims
  int64_t groups;     // output tiles (workgroups per split)
  int64_t ngroups;    // column groups (kind 1)
  int splits;         // K splits (1 = epilogue directly in the GEMM)
  int kc_per_split;   // 128-deep K chunks per split
  int kcmax;          // kind 0: weight register ring depth in chunks (4 or 8)
  int waves;          // kind 0: waves per workgroup (split of K inside the workgroup)
  int qpre;           // kind 0: activation blocks per thread loaded ahead of the weights
  int ntw;            // kind 0: 16-column tiles per workgroup
  int64_t lds_bytes;  // kind 0: dynamic LDS (compact activation copy / reduction)
  int64_t counter_bytes, xhat_bytes, partial_bytes, total_bytes;
};
// `aligned`: x rows are 16-byte aligned (pointer and row stride); the
// fused small-M kernel needs it. Workspace sizes of both kinds are covered by
// the aligned=false plan, which never needs less.
GemmPlan plan_gemm_nvfp4(int64_t M, int64_t N, int64_t K, bool aligned);

// Whether gemm_tiled_kernel<mt, nt, wm> / gemm_lds_kernel<mt, nt, st> is built
// into the library.
bool tiled_config_built(int mt, int nt, int wm);
bool lds_config_built(int mt, int nt, int st);
bool lds32_config_built(int mt, int nt, int st);

// Kernel name and parameters of a plan (diagnostics).
std::string describe_plan(const GemmPlan& p);

hipError_t launch_linear_nvfp4(const GemmPlan& p, const uint16_t* x, int64_t M, int64_t K,
                               int64_t ldx, float g, int hb, bool aligned, const uint8_t* packed,
                               int64_t N, float alpha, const uint16_t* bias, uint16_t* y,
                               int64_t ldy, uint8_t* workspace, hipStream_t st);

// ---- MXFP4 (E2M1 + E8M0 per 32) ------------------------------------------
// Operand layout (activation and packed weight): rows padded to 16, K to 128:
//   codes  [rows/16][KC][lane 64][16 B]   lane = kg*16 + r, 32 codes of
//          k = 128c + 32kg + 0..31 of row r
//   scales [rows/16][ceil(KC/4)][lane 64][4 B]  byte q = chunk 4*group + q
struct MxDims {
  int64_t rows_p, Kp, code_bytes, scale_bytes;
  int64_t total_bytes() const { return code_bytes + scale_bytes; }
};
MxDims mx_dims(int64_t rows, int64_t K);

// Workspace: [64 KiB arrival counters | x codes | x scales | split-K slabs].
struct MxPlan {
  int mt, nt, st;        // 16-row tiles per workgroup, 16-column tiles per wave, ring depth
  int splits_override;   // benchmarking override of the K split (0 = heuristic)
  int64_t Mp, groups, ngroups;
  int splits, kc_per_split;
  int64_t counter_bytes, xcode_bytes, xscale_bytes, partial_bytes, total_bytes;
};
MxPlan plan_gemm_mxfp4(int64_t M, int64_t N, int64_t K);
std::string describe_mx_plan(const MxPlan& p);

hipError_t launch_quant_mxfp4_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_quant_mxfp4_f32(const float* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* codes, uint8_t* scales, hipStream_t st);
hipError_t launch_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                             uint8_t* packed, hipStream_t st);
hipError_t launch_linear_mxfp4(const MxPlan& p, const uint16_t* x, int64_t M, int64_t K,
                               int64_t ldx, const uint8_t* packed, int64_t N, float alpha,
                               const uint16_t* bias, uint16_t* y, int64_t ldy, uint8_t* workspace,
                               hipStream_t st);

}  // namespace fql
