// Quantizers and weight packers of the scaled-MFMA formats (gfx950): MXFP4,
// MXFP8, per-tensor FP8 and block FP8.
//
// What is computed (B12X write-up, Implementation: the five linear kernels;
// element and scale formats per OCP Microscaling v1.0):
//   MX formats, per 32-block along K: a = max|v|, E = floor(log2 a) - emax
//     (emax 2 for E2M1, 8 for E4M3) clamped to [-127, 127] (a = 0: -127),
//     scale byte E + 127, q = RNE_satfinite(fl32(v * 2^-E)).
//   Block FP8 (activation groups 1 x 128, weight tiles 128 x 128, float32
//     scales): s = fl32(a / 448), r = fl32(1 / s) (0 if s = 0, the largest
//     finite float32 if 1/s overflows), q = E4M3_RNE_satfinite(fl32(v * r)).
//   Per-tensor FP8: q = E4M3_RNE_satfinite(fl32(v * r)) with the caller's
//     r = fl32(1 / s).
// The float32 -> E4M3 conversion is v_cvt_scalef32_pk_fp8_f32 after a clamp
// to [-448, 448]: on that range the instruction rounds to nearest even with
// subnormals (checked against an integer reference for every float32 in
// [-448, 448]), so clamp + convert is RNE with saturation. E2M1 uses
// v_cvt_scalef32_pk_fp4_f32, which also saturates.
#include <algorithm>
#include <cstdio>

#include "fql_device.h"
#include "fql_internal.h"
#include "sc_quant.h"

namespace fql {

// ---------------------------------------------------------------------------
// canonical quantizers (one thread per 32-block of a row)
// ---------------------------------------------------------------------------

template <int F, typename TIn>
__global__ __launch_bounds__(256) void sc_quant_canonical_kernel(const TIn* __restrict__ x,
                                                                 int64_t rows, int64_t K, int64_t ld,
                                                                 bool aligned, float inv_scale,
                                                                 uint8_t* __restrict__ codes,
                                                                 void* __restrict__ scales) {
  const int64_t nblk = K / 32;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool valid = i < rows * nblk;
  const int64_t m = valid ? i / nblk : 0, b = valid ? i - m * nblk : 0;
  float v[32];
  if (valid) load32(x + m * ld + b * 32, aligned, v);
  else
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = 0.0f;
  uint32_t w[8], sb = 0;
  float gs = 0.0f;
  quant_block32<F>(v, valid, inv_scale, w, sb, gs);
  if (!valid) return;
  if (F == SC_MXFP4) {
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + m * (K / 2) + b * 16);
#pragma unroll
    for (int j = 0; j < 4; ++j) dst[j] = w[j];
  } else {
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + m * K + b * 32);
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = w[j];
  }
  if (F == SC_MXFP4 || F == SC_MXFP8) static_cast<uint8_t*>(scales)[m * nblk + b] = (uint8_t)sb;
  if (F == SC_FP8_BLOCK && (b & 3) == 0) static_cast<float*>(scales)[m * (K / 128) + b / 4] = gs;
}

// Block-FP8 weight: one workgroup per 128 x 128 tile, each thread 64
// consecutive elements of one row (row tid/2, half tid%2).
__global__ __launch_bounds__(256) void fp8_block_weight_kernel(const float* __restrict__ w,
                                                               int64_t N, int64_t K, int64_t ld,
                                                               bool aligned,
                                                               uint8_t* __restrict__ codes,
                                                               float* __restrict__ scales) {
  __shared__ float red[4];
  const int64_t KB = K / 128;
  const int64_t tn = blockIdx.x / KB, tk = blockIdx.x % KB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t n = tn * 128 + tid / 2;
  const int64_t k0 = tk * 128 + (tid & 1) * 64;
  float v[2][32];
  load32(w + n * ld + k0, aligned, v[0]);
  load32(w + n * ld + k0 + 32, aligned, v[1]);
  float a = __builtin_fmaxf(amax32(v[0]), amax32(v[1]));
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) a = __builtin_fmaxf(a, __shfl_xor(a, o));
  if (lane == 0) red[wave] = a;
  __syncthreads();
  a = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  const float s = a / 448.0f;
  const float r = safe_reciprocal(s);
  uint32_t q[8];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    encode_fp8x32(v[h], r, q);
    uint32_t* dst = reinterpret_cast<uint32_t*>(codes + n * K + k0 + 32 * h);
#pragma unroll
    for (int j = 0; j < 8; ++j) dst[j] = q[j];
  }
  if (tid == 0) scales[tn * KB + tk] = s;
}

hipError_t launch_sc_quant(int fmt, bool f32_input, bool weight_tiles, const void* x, int64_t rows,
                           int64_t K, int64_t ld, float inv_scale, uint8_t* codes, void* scales,
                           hipStream_t st) {
  const uintptr_t xa = reinterpret_cast<uintptr_t>(x);
  const bool aligned = xa % 16 == 0 && (ld * (f32_input ? 4 : 2)) % 16 == 0;
  if (fmt == SC_FP8_BLOCK && weight_tiles) {
    if (!f32_input) return hipErrorInvalidValue;
    const int64_t tiles = (rows / 128) * (K / 128);
    fp8_block_weight_kernel<<<(unsigned)tiles, 256, 0, st>>>(static_cast<const float*>(x), rows, K,
                                                            ld, aligned, codes,
                                                            static_cast<float*>(scales));
    return hipGetLastError();
  }
  const int64_t total = rows * (K / 32);
  const unsigned grid = (unsigned)((total + 255) / 256);
#define FQL_Q(F)                                                                                      \
  if (fmt == F) {                                                                                     \
    if (f32_input)                                                                                    \
      sc_quant_canonical_kernel<F, float><<<grid, 256, 0, st>>>(static_cast<const float*>(x), rows,   \
                                                                K, ld, aligned, inv_scale, codes,     \
                                                                scales);                              \
    else                                                                                              \
      sc_quant_canonical_kernel<F, uint16_t><<<grid, 256, 0, st>>>(                                   \
          static_cast<const uint16_t*>(x), rows, K, ld, aligned, inv_scale, codes, scales);           \
    return hipGetLastError();                                                                         \
  }
  FQL_Q(SC_MXFP4) FQL_Q(SC_MXFP8) FQL_Q(SC_FP8) FQL_Q(SC_FP8_BLOCK)
#undef FQL_Q
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// activation straight into the operand layout
// ---------------------------------------------------------------------------

// One thread per (row, 32-block) of the padded operand [Mp][Kp]; rows >= M
// and blocks past K are zero codes with scale 0.
template <int F>
__global__ __launch_bounds__(256) void sc_quant_operand_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t ldx, bool aligned,
    float inv_scale, int64_t Mp, int64_t Kp, uint8_t* __restrict__ codes, void* __restrict__ scales) {
  constexpr int H = F == SC_MXFP4 ? 1 : 2;
  const int64_t nblk = Kp / 32, KC = Kp / 128;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool inside = i < Mp * nblk;
  const int64_t m = inside ? i / nblk : 0, b = inside ? i - m * nblk : 0;
  const bool valid = inside && m < M && b * 32 < K;
  float v[32];
  if (valid) load32(x + m * ldx + b * 32, aligned, v);
  else
#pragma unroll
    for (int j = 0; j < 32; ++j) v[j] = 0.0f;
  uint32_t w[8], sb = 0;
  float gs = 0.0f;
  quant_block32<F>(v, valid, inv_scale, w, sb, gs);
  if (!inside) return;
  if (!valid) {
#pragma unroll
    for (int j = 0; j < 8; ++j) w[j] = 0u;
    sb = 0;
    gs = 0.0f;
  }
  const int64_t tile = m / 16, c = b / 4, quad = m / 64;
  const int r = (int)(m % 16), kg = (int)(b % 4);
  uint8_t* tbase = codes + (tile * KC + c) * (int64_t)(H * 1024);
  if (F == SC_MXFP4) {
    *reinterpret_cast<uint4v*>(tbase + (kg * 16 + r) * 16) = uint4v{w[0], w[1], w[2], w[3]};
  } else {
    // 16-element piece h16 = 2kg + j goes to half h16/4, lane (h16%4)*16 + r
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int h16 = 2 * kg + j;
      *reinterpret_cast<uint4v*>(tbase + (h16 / 4) * 1024 + ((h16 % 4) * 16 + r) * 16) =
          uint4v{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
    }
  }
  if (F == SC_MXFP4 || F == SC_MXFP8)
    static_cast<uint8_t*>(scales)[((quad * KC + c) * 64 + kg * 16 + r) * 4 + (m / 16) % 4] = (uint8_t)sb;
  if (F == SC_FP8_BLOCK && kg == 0) static_cast<float*>(scales)[(quad * KC + c) * 64 + m % 64] = gs;
}

hipError_t launch_sc_quant_operand(int fmt, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                                   bool aligned, float inv_scale, int64_t Mp, uint8_t* codes,
                                   void* scales, hipStream_t st) {
  const int64_t Kp = round_up(K, 128);
  const int64_t total = Mp * (Kp / 32);
  const unsigned grid = (unsigned)((total + 255) / 256);
#define FQL_Q(F)                                                                                    \
  if (fmt == F) {                                                                                   \
    sc_quant_operand_kernel<F><<<grid, 256, 0, st>>>(x, M, K, ldx, aligned, inv_scale, Mp, Kp,      \
                                                     codes, scales);                                \
    return hipGetLastError();                                                                       \
  }
  FQL_Q(SC_MXFP4) FQL_Q(SC_MXFP8) FQL_Q(SC_FP8) FQL_Q(SC_FP8_BLOCK)
#undef FQL_Q
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------------------
// weight packers: canonical -> operand layout
// ---------------------------------------------------------------------------

// One thread per 16-byte code slot (tile, chunk, half, lane).
template <int F>
__global__ __launch_bounds__(256) void sc_pack_codes_kernel(const uint8_t* __restrict__ codes,
                                                            int64_t N, int64_t K, int64_t Np,
                                                            int64_t KC, uint8_t* __restrict__ packed) {
  constexpr int H = F == SC_MXFP4 ? 1 : 2;
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (slot >= (Np / 16) * KC * H * 64) return;
  const int lane = (int)(slot & 63);
  const int64_t tch = slot >> 6;  // (tile, chunk, half)
  const int h = (int)(tch % H);
  const int64_t tc = tch / H, t = tc / KC, c = tc - t * KC;
  const int64_t n = t * 16 + (lane & 15);
  uint4v v = uint4v{0u, 0u, 0u, 0u};
  if (F == SC_MXFP4) {
    const int64_t k = c * 128 + 32 * (lane >> 4);
    if (n < N && k < K) v = *reinterpret_cast<const uint4v*>(codes + n * (K / 2) + k / 2);
  } else {
    const int64_t k = c * 128 + 64 * h + 16 * (lane >> 4);
    if (n < N && k < K) v = *reinterpret_cast<const uint4v*>(codes + n * K + k);
  }
  *reinterpret_cast<uint4v*>(packed + slot * 16) = v;
}

// MX scales: one thread per (quad, chunk, lane) dword.
__global__ __launch_bounds__(256) void sc_pack_mx_scales_kernel(const uint8_t* __restrict__ scales,
                                                                int64_t N, int64_t K, int64_t quads,
                                                                int64_t KC, uint32_t* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= quads * KC * 64) return;
  const int lane = (int)(i & 63);
  const int64_t qc = i >> 6, quad = qc / KC, c = qc - quad * KC;
  const int64_t j = 4 * c + (lane >> 4), nb = K / 32;
  uint32_t d = 0u;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t n = quad * 64 + 16 * q + (lane & 15);
    if (n < N && j < nb) d |= (uint32_t)scales[n * nb + j] << (8 * q);
  }
  out[i] = d;
}

__global__ __launch_bounds__(256) void copy_f32_kernel(const float* __restrict__ src, int64_t n,
                                                       float* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src[i];
}

hipError_t launch_sc_pack(int fmt, const uint8_t* codes, const void* scales, int64_t N, int64_t K,
                          uint8_t* packed, hipStream_t st) {
  const ScDims d = sc_dims(fmt, N, K, true);
  const int H = fmt == SC_MXFP4 ? 1 : 2;
  const int64_t slots = (d.rows_p / 16) * d.KC * H * 64;
  const unsigned g = (unsigned)((slots + 255) / 256);
  if (fmt == SC_MXFP4) sc_pack_codes_kernel<SC_MXFP4><<<g, 256, 0, st>>>(codes, N, K, d.rows_p, d.KC, packed);
  else if (fmt == SC_MXFP8) sc_pack_codes_kernel<SC_MXFP8><<<g, 256, 0, st>>>(codes, N, K, d.rows_p, d.KC, packed);
  else sc_pack_codes_kernel<SC_FP8><<<g, 256, 0, st>>>(codes, N, K, d.rows_p, d.KC, packed);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (fmt == SC_MXFP4 || fmt == SC_MXFP8) {
    const int64_t n = d.quads * d.KC * 64;
    sc_pack_mx_scales_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        static_cast<const uint8_t*>(scales), N, K, d.quads, d.KC,
        reinterpret_cast<uint32_t*>(packed + d.code_bytes));
    return hipGetLastError();
  }
  if (fmt == SC_FP8_BLOCK) {  // [N/128][K/128] floats, already the packed order (K % 128 == 0)
    const int64_t n = (N / 128) * d.KC;
    copy_f32_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(
        static_cast<const float*>(scales), n, reinterpret_cast<float*>(packed + d.code_bytes));
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace fql
