// Device-side quantization of one 32-element block for the scaled-MFMA
// formats (MXFP4, MXFP8, per-tensor FP8, block FP8), shared by the standalone
// quantizer kernels and the fused small-M linear kernel.
//
// What is computed (B12X write-up, Implementation: the five linear kernels;
// element and scale formats per OCP Microscaling v1.0):
//   MX formats, per 32-block along K: a = max|v|, E = floor(log2 a) - emax
//     (emax 2 for E2M1, 8 for E4M3) clamped to [-127, 127] (a = 0: -127),
//     scale byte E + 127, q = RNE_satfinite(fl32(v * 2^-E)).
//   Block FP8 (1 x 128 activation groups): s = fl32(a / 448), r = fl32(1 / s)
//     (0 if s = 0, the largest finite float32 if 1/s overflows),
//     q = E4M3_RNE_satfinite(fl32(v * r)).
//   Per-tensor FP8: q = E4M3_RNE_satfinite(fl32(v * r)) with the caller's
//     r = fl32(1 / s).
#pragma once

#include "fql_device.h"
#include "fql_internal.h"

namespace fql {

typedef short short2v __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------
// element encoders
// ---------------------------------------------------------------------------

// r = fl32(1 / s) for s > 0 (largest finite float32 when it overflows), 0 for s = 0.
__device__ __forceinline__ float safe_reciprocal(float s) {
  return s > 0.0f ? __builtin_fminf(1.0f / s, 3.4028234663852886e38f) : 0.0f;
}

__device__ __forceinline__ float e4m3_clamp(float v) {
  return __builtin_fminf(__builtin_fmaxf(v, -448.0f), 448.0f);
}

// Four float32 -> four E4M3 bytes (a in the lowest byte).
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  short2v o = {0, 0};
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, e4m3_clamp(a), e4m3_clamp(b), 1.0f, false);
  o = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(o, e4m3_clamp(c), e4m3_clamp(d), 1.0f, true);
  return __builtin_bit_cast(uint32_t, o);
}

// floor(log2 a) - emax clamped to [-127, 127]; a = 0 gives -127.
__device__ __forceinline__ int mx_exponent(float a, int emax) {
  const uint32_t b = __float_as_uint(a);
  if (b == 0u) return -127;
  const int fl = b < 0x00800000u ? (31 - __builtin_clz(b)) - 149 : (int)(b >> 23) - 127;
  const int e = fl - emax;
  return e < -127 ? -127 : (e > 127 ? 127 : e);
}

__device__ __forceinline__ float amax32(const float v[32]) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < 32; ++i) a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
  return a;
}

// 32 values -> FP4 codes (4 words, element i in nibble i%8 of word i/8), each
// value multiplied by f first.
__device__ __forceinline__ void encode_fp4x32(const float v[32], float f, uint32_t w[4]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    uint32_t r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[8 * j] * f, v[8 * j + 1] * f, 1.0f, 0);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * j + 2] * f, v[8 * j + 3] * f, 1.0f, 1);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * j + 4] * f, v[8 * j + 5] * f, 1.0f, 2);
    r = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(r, v[8 * j + 6] * f, v[8 * j + 7] * f, 1.0f, 3);
    w[j] = r;
  }
}

// 32 values -> E4M3 codes (8 words, element i in byte i%4 of word i/4), each
// value multiplied by f first.
__device__ __forceinline__ void encode_fp8x32(const float v[32], float f, uint32_t w[8]) {
#pragma clang fp contract(off)
#pragma unroll
  for (int j = 0; j < 8; ++j)
    w[j] = fp8x4(v[4 * j] * f, v[4 * j + 1] * f, v[4 * j + 2] * f, v[4 * j + 3] * f);
}

// 2^-e as a float32 for e in [-127, 126].
__device__ __forceinline__ float pow2_neg(int e) { return __uint_as_float((uint32_t)(127 - e) << 23); }

// ---------------------------------------------------------------------------
// input loads (32 consecutive elements)
// ---------------------------------------------------------------------------

__device__ __forceinline__ void load32(const uint16_t* p, bool aligned, float v[32]) {
  if (aligned) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const uint4v u = *reinterpret_cast<const uint4v*>(p + 8 * q);
      const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        v[8 * q + 2 * j] = __uint_as_float(w[j] << 16);
        v[8 * q + 2 * j + 1] = __uint_as_float(w[j] & 0xFFFF0000u);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = bf16_bits_to_f32(p[i]);
  }
}
__device__ __forceinline__ void load32(const float* p, bool aligned, float v[32]) {
  if (aligned) {
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      const float4v u = *reinterpret_cast<const float4v*>(p + 4 * q);
      v[4 * q] = u[0]; v[4 * q + 1] = u[1]; v[4 * q + 2] = u[2]; v[4 * q + 3] = u[3];
    }
  } else {
#pragma unroll
    for (int i = 0; i < 32; ++i) v[i] = p[i];
  }
}

// One 32-block of one row, every format: the codes as words (FP4: 4, FP8: 8)
// and the block's scale (MX: the E8M0 byte; block FP8: the group scale s,
// shared by the 4 lanes of a 128-group through shuffles). `valid` lanes only
// contribute; every lane of the wave must call it (shuffles).
template <int F>
__device__ __forceinline__ void quant_block32(const float v[32], bool valid, float inv_scale,
                                              uint32_t w[8], uint32_t& sbyte, float& gscale) {
  const float a = valid ? amax32(v) : 0.0f;
  if (F == SC_MXFP4) {
    const int e = mx_exponent(a, 2);
    encode_fp4x32(v, pow2_neg(e), w);
    sbyte = (uint32_t)(e + 127);
  } else if (F == SC_MXFP8) {
    const int e = mx_exponent(a, 8);
    encode_fp8x32(v, pow2_neg(e), w);
    sbyte = (uint32_t)(e + 127);
  } else if (F == SC_FP8) {
    encode_fp8x32(v, inv_scale, w);
  } else {
    float g = a;
    g = __builtin_fmaxf(g, __shfl_xor(g, 1));
    g = __builtin_fmaxf(g, __shfl_xor(g, 2));
    const float s = g / 448.0f;
    const float r = safe_reciprocal(s);
    encode_fp8x32(v, r, w);
    gscale = s;
  }
}

}  // namespace fql
