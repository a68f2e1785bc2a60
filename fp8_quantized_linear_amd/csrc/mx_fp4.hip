// MXFP4 sibling format for gfx950: quantizer, weight packer and linear layer.
//
// What is computed (B12X write-up, Implementation: MXFP4 is one of the five
// linear formats, with the activation quantized dynamically; formats per OCP
// Microscaling v1.0): E2M1 elements with one E8M0 (power-of-two) scale per 32
// consecutive elements along K and no global scale.
//   a = max |v| over the 32-block
//   E = floor(log2 a) - 2 clamped to [-127, 127] (a = 0 gives -127),
//       scale byte E + 127
//   q_i = E2M1_RNE_satfinite(fl32(v_i * 2^-E)), sign of v_i kept
//   y   = bf16(alpha * sum_k x_hat[m][k] w_hat[n][k] + bias[n])
//
// How (MI355X): this is the one format whose block scaling the CDNA4 matrix
// cores implement directly. v_mfma_scale_f32_16x16x128_f8f6f4 with FP4
// operands takes, per lane, 32 consecutive E2M1 codes of one row (A) or column
// (B) as 16 bytes and one E8M0 byte that scales exactly those 32 elements
// (checked against a float64 reference on random codes and scales: lane l
// holds row/column l%16 and k = 32*(l/16) + i in nibble i, low nibble first;
// the accumulator layout is that of the 16x16 MFMAs). So neither operand is
// dequantized: codes and scale bytes go from memory to the MFMA unchanged.
//
// Operand layout (activation and packed weight alike), rows padded to 16 and
// K to 128 ("a chunk"):
//   codes  [rows/16][KC][lane 64][16 B]   lane = kg*16 + r: row r of the tile,
//          the 32 codes of k = 128c + 32kg + 0..31 (canonical nibble order)
//   scales [rows/16][ceil(KC/4)][lane 64][4 B]   byte q = scale byte of the
//          lane's row and 32-block for chunk 4*group + q
#include <algorithm>
#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "fql_device.h"
#include "fql_gemm.h"
#include "fql_internal.h"

namespace fql {

typedef int int8v __attribute__((ext_vector_type(8)));

// E = floor(log2 a) - 2 clamped to [-127, 127] from the bits of a >= 0.
__device__ __forceinline__ int mx_shared_exponent(float a) {
  const uint32_t b = __float_as_uint(a);
  int fl;  // floor(log2 a)
  if (b == 0u) return -127;
  if (b < 0x00800000u) fl = (31 - __builtin_clz(b)) - 149;  // subnormal: a = b * 2^-149
  else fl = (int)(b >> 23) - 127;
  const int e = fl - 2;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

// Quantize one 32-block: codes as four words (element i in nibble i%8 of
// word i/8) and the scale byte.
__device__ __forceinline__ void mx_quant_block(const float v[32], uint32_t w[4], uint32_t& sbyte) {
#pragma clang fp contract(off)
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
  const int e = mx_shared_exponent(a);
  // 2^-e is a normal float32 for e in [-127, 125] (e cannot exceed 125)
  const float f = __uint_as_float((uint32_t)(127 - e) << 23);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    // the byte-select operand must be a literal
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[8 * j] * f, v[8 * j + 1] * f, 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * j + 2] * f, v[8 * j + 3] * f, 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * j + 4] * f, v[8 * j + 5] * f, 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * j + 6] * f, v[8 * j + 7] * f, 1.0f, 3);
    w[j] = r;
  }
  sbyte = (uint32_t)(e + 127);
}

template <typename TIn>
__device__ __forceinline__ void load32(const TIn* p, float v[32]);
template <>
__device__ __forceinline__ void load32<uint16_t>(const uint16_t* p, float v[32]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = bf16_bits_to_f32(p[i]);
}
template <>
__device__ __forceinline__ void load32<float>(const float* p, float v[32]) {
#pragma unroll
  for (int i = 0; i < 32; ++i) v[i] = p[i];
}

// Canonical output: codes [rows][K/2], scales [rows][K/32]. One thread per block.
template <typename TIn>
__global__ __launch_bounds__(256) void quant_mxfp4_canonical_kernel(const TIn* __restrict__ x,
                                                                   int64_t rows, int64_t K,
                                                                   int64_t ldx,
                                                                   uint8_t* __restrict__ codes,
                                                                   uint8_t* __restrict__ scales) {
  const int64_t nblk = K / 32;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= rows * nblk) return;
  const int64_t m = i / nblk, b = i - m * nblk;
  float v[32];
  load32<TIn>(x + m * ldx + b * 32, v);
  uint32_t w[4], s;
  mx_quant_block(v, w, s);
  uint32_t* dst = reinterpret_cast<uint32_t*>(codes + m * (K / 2) + b * 16);
#pragma unroll
  for (int j = 0; j < 4; ++j) dst[j] = w[j];
  scales[m * nblk + b] = (uint8_t)s;
}

// Activation straight into the operand layout (rows >= M and k >= K are
// written as zero codes with scale byte 0). One thread per (row, 32-block).
__global__ __launch_bounds__(256) void quant_mxfp4_operand_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, int64_t Mp, int64_t Kp,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
  const int64_t nblk = Kp / 32;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= Mp * nblk) return;
  const int64_t m = i / nblk, b = i - m * nblk;
  uint32_t w[4] = {0u, 0u, 0u, 0u}, s = 0u;
  if (m < M && b * 32 < K) {
    float v[32];
    load32<uint16_t>(x + m * ldx + b * 32, v);
    mx_quant_block(v, w, s);
  }
  const int64_t KC = Kp / 128, KC4 = (KC + 3) / 4;
  const int64_t c = b / 4, kg = b % 4, tile = m / 16;
  const int lane = (int)(kg * 16 + m % 16);
  *reinterpret_cast<uint4v*>(codes + ((tile * KC + c) * 64 + lane) * 16) = uint4v{w[0], w[1], w[2], w[3]};
  scales[((tile * KC4 + c / 4) * 64 + lane) * 4 + c % 4] = (uint8_t)s;
}

// Weight packer: canonical [N][K/2] codes + [N][K/32] scales -> operand layout.
// One thread per (tile, chunk, lane) code slot; the first chunk of each
// 4-chunk group also writes the lane's scale dword.
__global__ __launch_bounds__(256) void pack_mxfp4_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        int64_t N, int64_t K, int64_t Np,
                                                        int64_t Kp, uint8_t* __restrict__ packed) {
  const int64_t KC = Kp / 128, KC4 = (KC + 3) / 4;
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (t, c, lane)
  if (slot >= (Np / 16) * KC * 64) return;
  const int lane = (int)(slot & 63);
  const int64_t tc = slot >> 6, t = tc / KC, c = tc - t * KC;
  const int kg = lane >> 4;
  const int64_t n = t * 16 + (lane & 15);
  const int64_t k = c * 128 + 32 * kg;
  uint4v v = uint4v{0u, 0u, 0u, 0u};
  if (n < N && k < K) v = *reinterpret_cast<const uint4v*>(codes + n * (K / 2) + k / 2);
  *reinterpret_cast<uint4v*>(packed + slot * 16) = v;
  if (c % 4 == 0) {
    uint32_t sw = 0u;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int64_t b = (c + q) * 4 + kg;  // 32-block of chunk c+q
      if (n < N && c + q < KC && b * 32 < K) sw |= (uint32_t)scales[n * (K / 32) + b] << (8 * q);
    }
    uint32_t* sdst = reinterpret_cast<uint32_t*>(packed + Np * Kp / 2) + (t * KC4 + c / 4) * 64 + lane;
    *sdst = sw;
  }
}

// ---------------------------------------------------------------------------
// GEMM: LDS ring (direct global->LDS loads) feeding the scaled FP4 MFMA
// ---------------------------------------------------------------------------
//
// Workgroup: 4 waves; tile (MT*16) rows x (4*NT*16) columns; wave w owns
// columns [w*NT*16, (w+1)*NT*16). Per 128-deep chunk a stage holds the
// activation codes and scale dwords of the MT row tiles (shared by the
// waves; loaded by them in turn) and each wave's own weight codes and scale
// dwords. One MFMA per (row tile, column tile) covers the whole chunk.
template <int MT, int NT>
struct Mx4Stage {
  uint4v a[MT][64];
  uint32_t as[MT][64];
  uint4v bq[4 * NT][64];
  uint32_t bs[4 * NT][64];
};

template <int MT, int NT, int ST>
__global__ __launch_bounds__(256) void gemm_mx4_kernel(
    const uint8_t* __restrict__ xcodes, const uint8_t* __restrict__ xscales,
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales, int M, int N,
    int64_t Kp, int ntiles, int ngroups, int kc_per_split, int splits, float alpha,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t ldy,
    float4v* __restrict__ partial, uint32_t* __restrict__ counters) {
  static_assert(ST >= 2 && ST <= 4, "ring depth");
  constexpr int LA = (2 * MT + 3) / 4;  // shared activation loads per wave per chunk
  constexpr int L = LA + 2 * NT;         // LDS loads per wave per chunk
  static_assert(L * (ST - 2) <= 63, "vmcnt range");
  __shared__ Mx4Stage<MT, NT> stage[ST];
  __shared__ uint32_t s_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t KC = Kp / 128, KC4 = (KC + 3) / 4;
  const int split = blockIdx.x % splits;
  const int tilegrp = blockIdx.x / splits;
  const int ngroup = tilegrp % ngroups;
  const int mgroup = tilegrp / ngroups;
  const int64_t c_begin = (int64_t)split * kc_per_split;
  const int64_t c_end = c_begin + kc_per_split < KC ? c_begin + kc_per_split : KC;
  const int nch = (int)(c_end - c_begin);
  const int tile0 = (ngroup * 4 + wave) * NT;

  typedef Mx4Stage<MT, NT> Stage;
  const uint32_t q_voff = lane * 16, s_voff = lane * 4;
  // LDS byte addresses are formed as stage base + field offset + index * row
  // bytes (integer arithmetic on a constant base, so they stay scalar).
  auto issue = [&](Stage& sg, int64_t c) {
    c = c < c_end ? c : c_end - 1;  // clamped: a static number of loads per chunk
    const uint32_t base = lds_offset(&sg);
#pragma unroll
    for (int j = 0; j < LA; ++j) {
      // shared item e = wave + 4j: codes of row tile e, or scales of row tile e - MT
      // (waves past the last item repeat item 0: same data to the same place)
      int e = wave + 4 * j;
      e = e < 2 * MT ? e : 0;
      if (e < MT) {
        const int64_t t = (int64_t)mgroup * MT + e;
        lds_load16(xcodes + (t * KC + c) * 1024, q_voff, base + offsetof(Stage, a) + e * 1024);
      } else {
        const int64_t t = (int64_t)mgroup * MT + (e - MT);
        lds_load4(xscales + (t * KC4 + c / 4) * 256, s_voff, base + offsetof(Stage, as) + (e - MT) * 256);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int64_t t = tile0 + nt < ntiles ? tile0 + nt : 0;  // invalid tiles read tile 0, never stored
      const int slot = wave * NT + nt;
      lds_load16(wcodes + (t * KC + c) * 1024, q_voff, base + offsetof(Stage, bq) + slot * 1024);
      lds_load4(wscales + (t * KC4 + c / 4) * 256, s_voff, base + offsetof(Stage, bs) + slot * 256);
    }
  };

  float4v acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Mx4Stage<MT, NT>& sg, int64_t c) {
    const int sh = (int)(c & 3) * 8;  // the chunk's byte in the 4-chunk scale dwords
    int8v b[NT];
    int sb[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint4v q = sg.bq[wave * NT + nt][lane];
      b[nt] = int8v{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      sb[nt] = (int)((sg.bs[wave * NT + nt][lane] >> sh) & 0xFFu);
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4v q = sg.a[mt][lane];
      const int8v a = int8v{(int)q.x, (int)q.y, (int)q.z, (int)q.w, 0, 0, 0, 0};
      const int sa = (int)((sg.as[mt][lane] >> sh) & 0xFFu);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[nt], acc[mt][nt], 4, 4, 0,
                                                                       sa, 0, sb[nt]);
    }
  };

  // Ring: chunk i lives in stage i % ST. Before computing chunk i the wave
  // waits for its own loads of chunk i, passes the barrier (everyone's have
  // landed, and everyone has finished chunk i-1), and refills stage
  // (i-1) % ST with chunk i+ST-1.
#pragma unroll
  for (int p = 0; p < ST - 1; ++p) issue(stage[p], c_begin + p);
  for (int i0 = 0; i0 < nch; i0 += ST) {
#pragma unroll
    for (int j = 0; j < ST; ++j) {
      if (i0 + j < nch) {
        wait_vmcnt<L * (ST - 2)>();
        stage_barrier();
        issue(stage[(j + ST - 1) % ST], c_begin + i0 + j + ST - 1);
        compute(stage[j], c_begin + i0 + j);
      }
    }
  }
  wait_vmcnt<0>();  // no LDS load may still be in flight when the workgroup ends

  float4v* slab = partial + (int64_t)tilegrp * splits * (4 * MT * NT * 64);
  finish_tile<MT, NT, 1>(acc, M, N, mgroup * MT * 16, ngroup * 4 * NT * 16, split, splits, alpha,
                         bias, y, ldy, slab, counters + tilegrp, &s_flag);
}

// ---------------------------------------------------------------------------
// sizes, plan, launchers
// ---------------------------------------------------------------------------

MxDims mx_dims(int64_t rows, int64_t K) {
  MxDims d;
  d.rows_p = round_up(rows, 16);
  d.Kp = round_up(K, 128);
  d.code_bytes = d.rows_p * d.Kp / 2;
  d.scale_bytes = (d.rows_p / 16) * ((d.Kp / 128 + 3) / 4) * 256;
  return d;
}

#define FQL_MX4_CONFIGS(X) X(1, 4, 4) X(2, 4, 4) X(4, 4, 4) X(8, 4, 4) X(4, 2, 4) X(8, 2, 4)

static bool mx4_config_built(int mt, int nt, int st) {
#define FQL_X(A, B, C) if (mt == A && nt == B && st == C) return true;
  FQL_MX4_CONFIGS(FQL_X)
#undef FQL_X
  return false;
}

MxPlan plan_gemm_mxfp4(int64_t M, int64_t N, int64_t K) {
  MxPlan p{};
  const MxDims w = mx_dims(N, K);
  const int64_t KC = w.Kp / 128, ntiles = w.rows_p / 16;
  // Measured on the K=4096 shapes (N = 6144 .. 28672): one row tile with four
  // column tiles per wave for M <= 32; above that a 64 x 128 workgroup tile,
  // except for large M and N, where the 128 x 256 tile's reuse wins.
  if (M <= 32) { p.mt = 1; p.nt = 4; }
  else if (M >= 2048 && N >= 16384) { p.mt = 8; p.nt = 4; }
  else { p.mt = 4; p.nt = 2; }
  p.st = 4;
  if (const char* e = std::getenv("FQL_MX_PLAN")) {  // benchmarking aid: "mt,nt,st,splits"
    int a = 0, b = 0, c = 0, s = 0;
    if (std::sscanf(e, "%d,%d,%d,%d", &a, &b, &c, &s) >= 3 && mx4_config_built(a, b, c)) {
      p.mt = a; p.nt = b; p.st = c; p.splits_override = s;
    }
  }
  const MxDims x = mx_dims(round_up(M, 16 * p.mt), K);
  p.Mp = x.rows_p;
  p.ngroups = (ntiles + 4 * p.nt - 1) / (4 * p.nt);
  const int64_t groups = p.ngroups * (p.Mp / (16 * p.mt));
  // split K until about 160 workgroups are in flight (at most 4 ways)
  int64_t s = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(4, KC), (160 + groups / 2) / groups));
  if (p.splits_override > 0) s = std::min<int64_t>(p.splits_override, KC);
  p.kc_per_split = (int)((KC + s - 1) / s);
  p.splits = (int)((KC + p.kc_per_split - 1) / p.kc_per_split);
  p.groups = groups;
  p.xcode_bytes = round_up(x.code_bytes, 256);
  p.xscale_bytes = round_up(x.scale_bytes, 256);
  const int64_t slab = (int64_t)p.splits * 4 * p.mt * p.nt * 64 * 16;
  p.partial_bytes = p.splits > 1 ? round_up(groups * slab, 256) : 0;
  p.counter_bytes = 64 * 1024;
  p.total_bytes = p.counter_bytes + p.xcode_bytes + p.xscale_bytes + p.partial_bytes;
  return p;
}

std::string describe_mx_plan(const MxPlan& p) {
  char b[200];
  std::snprintf(b, sizeof(b), "quant_mxfp4_operand_kernel + gemm_mx4_kernel<MT=%d,NT=%d,ST=%d> grid=%lld splits=%d",
                p.mt, p.nt, p.st, (long long)(p.groups * p.splits), p.splits);
  return std::string(b);
}

hipError_t launch_quant_mxfp4_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t total = M * (K / 32);
  quant_mxfp4_canonical_kernel<uint16_t><<<(unsigned)((total + 255) / 256), 256, 0, st>>>(
      x, M, K, ldx, codes, scales);
  return hipGetLastError();
}

hipError_t launch_quant_mxfp4_f32(const float* w, int64_t N, int64_t K, int64_t ldw,
                                  uint8_t* codes, uint8_t* scales, hipStream_t st) {
  const int64_t total = N * (K / 32);
  quant_mxfp4_canonical_kernel<float><<<(unsigned)((total + 255) / 256), 256, 0, st>>>(
      w, N, K, ldw, codes, scales);
  return hipGetLastError();
}

hipError_t launch_pack_mxfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                             uint8_t* packed, hipStream_t st) {
  const MxDims d = mx_dims(N, K);
  const int64_t slots = (d.rows_p / 16) * (d.Kp / 128) * 64;
  pack_mxfp4_kernel<<<(unsigned)((slots + 255) / 256), 256, 0, st>>>(codes, scales, N, K, d.rows_p,
                                                                     d.Kp, packed);
  return hipGetLastError();
}

template <int MT, int NT, int ST>
static hipError_t launch_mx4_t(const MxPlan& p, const uint8_t* xc, const uint8_t* xs,
                               const uint8_t* packed, const MxDims& w, int64_t M, int64_t N,
                               float alpha, const uint16_t* bias, uint16_t* y, int64_t ldy,
                               float4v* partial, uint32_t* counters, hipStream_t st) {
  gemm_mx4_kernel<MT, NT, ST><<<(unsigned)(p.groups * p.splits), 256, 0, st>>>(
      xc, xs, packed, packed + w.code_bytes, (int)M, (int)N, w.Kp, (int)(w.rows_p / 16),
      (int)p.ngroups, p.kc_per_split, p.splits, alpha, bias, y, ldy, partial, counters);
  return hipGetLastError();
}

hipError_t launch_linear_mxfp4(const MxPlan& p, const uint16_t* x, int64_t M, int64_t K,
                               int64_t ldx, const uint8_t* packed, int64_t N, float alpha,
                               const uint16_t* bias, uint16_t* y, int64_t ldy, uint8_t* workspace,
                               hipStream_t st) {
  const MxDims w = mx_dims(N, K);
  uint32_t* counters = reinterpret_cast<uint32_t*>(workspace);
  uint8_t* xc = workspace + p.counter_bytes;
  uint8_t* xs = xc + p.xcode_bytes;
  float4v* partial = reinterpret_cast<float4v*>(xs + p.xscale_bytes);
  if (p.splits > 1 && p.groups > p.counter_bytes / 4) return hipErrorInvalidValue;
  const int64_t total = p.Mp * (w.Kp / 32);
  quant_mxfp4_operand_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(x, M, K, ldx, p.Mp,
                                                                              w.Kp, xc, xs);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
#define FQL_X(A, B, C) \
  if (p.mt == A && p.nt == B && p.st == C) \
    return launch_mx4_t<A, B, C>(p, xc, xs, packed, w, M, N, alpha, bias, y, ldy, partial, counters, st);
  FQL_MX4_CONFIGS(FQL_X)
#undef FQL_X
  return hipErrorInvalidValue;
}

}  // namespace fql
