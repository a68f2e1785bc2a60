// Device-side NVFP4 block quantization shared by the quantizer kernels and the
// fused small-M linear kernel.
//
// One 16-element block (vLLM write-ups: activation NVFP4 quantize with the
// layer's input global scale, optionally after the block-diagonal Hadamard
// rotation normalised by 1/sqrt(n)):
//   a   = max |v|
//   s   = E4M3_RNE_satfinite(fl32(fl32(a / 6) * g))
//   r   = fl32(g / s), or 0 when s == 0
//   q_i = E2M1_RNE_satfinite(fl32(v_i * r)), sign of v_i kept
// Every float operation is a single IEEE float32 operation (contraction off),
// so codes and scales are bit-identical to any IEEE evaluation of the same
// sequence. The E2M1 encode uses gfx950's v_cvt_scalef32_pk_fp4_f32 with
// scale 1.0, which rounds to nearest even, saturates to +-6 and keeps the
// sign of zero; it was checked against the compare-based encoder
// (e2m1_encode) on every float32 bit pattern in [2^-100, 8] of both signs and
// on all denormals.
#pragma once

#include "fql_device.h"

namespace fql {

template <typename TIn>
struct Loader;

// bf16 rows: 16 elements = 32 bytes.
template <>
struct Loader<uint16_t> {
  static __device__ __forceinline__ void load16(const uint16_t* p, bool aligned16, float v[16]) {
    if (aligned16) {
      const uint4v* q = reinterpret_cast<const uint4v*>(p);
      uint4v a = q[0], b = q[1];
      uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = bf16_bits_to_f32(p[i]);
    }
  }
};

// float32 rows: 16 elements = 64 bytes.
template <>
struct Loader<float> {
  static __device__ __forceinline__ void load16(const float* p, bool aligned16, float v[16]) {
    if (aligned16) {
      const float4v* q = reinterpret_cast<const float4v*>(p);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float4v t = q[i];
        v[4 * i] = t.x;
        v[4 * i + 1] = t.y;
        v[4 * i + 2] = t.z;
        v[4 * i + 3] = t.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 16; ++i) v[i] = p[i];
    }
  }
};

// Rotate the thread's 16 values as part of its b-chunk (Sylvester H_b in
// natural order, scaled by fl32(1/sqrt(b))): in-thread butterfly strides 1,
// 2, 4, 8 (those below b), then cross-lane strides 16 .. b/2 with lane ^ LS,
// ^ 2LS, ^ 4LS, then one multiply. `blk` is the block index within the row;
// the b/16 blocks of a chunk must sit in lanes LS apart of one wave, in
// order. Every lane of those groups must execute this call.
template <int HB, int LS = 1>
__device__ __forceinline__ void fwht_block(float v[16], int64_t blk) {
#pragma clang fp contract(off)
#pragma unroll
  for (int h = 1; h < 16 && h < HB; h <<= 1) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      if ((e & h) == 0) {
        float a = v[e], b = v[e + h];
        v[e] = a + b;
        v[e + h] = a - b;
      }
    }
  }
#pragma unroll
  for (int hs = 1; hs < HB / 16; hs <<= 1) {
    const bool upper = (blk & hs) != 0;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      float other = __shfl_xor(v[e], hs * LS);
      // lower lane holds a, upper lane holds b: lower gets a + b, upper a - b
      v[e] = upper ? (other - v[e]) : (v[e] + other);
    }
  }
  // fl32(1/sqrt(b)): 0x3E800000, 0x3E3504F3, 0x3E000000, 0x3DB504F3
  const float cb = HB == 16 ? 0x1p-2f : HB == 32 ? 0x1.6a09e6p-3f : HB == 64 ? 0x1p-3f : 0x1.6a09e6p-4f;
#pragma unroll
  for (int e = 0; e < 16; ++e) v[e] = v[e] * cb;
}

// Quantize one 16-block: 16 codes as two words (element i in nibble i of
// lo, element 8+i in nibble i of hi) and the E4M3 scale byte.
__device__ __forceinline__ void quant_block(const float v[16], float g, uint32_t& lo, uint32_t& hi,
                                            uint32_t& sbyte) {
#pragma clang fp contract(off)
  float a = 0.0f;
#pragma unroll
  for (int e = 0; e < 16; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(v[e]));
  const float sf = (a / 6.0f) * g;
  const uint32_t s = e4m3_encode_nonneg(sf);
  const float sd = e4m3_decode_nonneg(s);
  const float r = sd == 0.0f ? 0.0f : g / sd;
  // the byte-select operand must be a literal
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0] * r, v[1] * r, 1.0f, 0);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[2] * r, v[3] * r, 1.0f, 1);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[4] * r, v[5] * r, 1.0f, 2);
  lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[6] * r, v[7] * r, 1.0f, 3);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[8] * r, v[9] * r, 1.0f, 0);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[10] * r, v[11] * r, 1.0f, 1);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[12] * r, v[13] * r, 1.0f, 2);
  hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[14] * r, v[15] * r, 1.0f, 3);
  sbyte = s;
}

// E4M3 byte -> float16 value (exact: E4M3 values are float16 values).
__device__ __forceinline__ _Float16 e4m3_to_f16(uint32_t c) { return (_Float16)e4m3_decode_nonneg(c); }

// Four E4M3 bytes -> four float16 values with two v_cvt_scalef32_pk_f16_fp8
// (scale 1.0; checked exact against the E4M3 definition for all 256 bytes):
// lo = (byte0, byte1), hi = (byte2, byte3).
__device__ __forceinline__ void e4m3x4_to_f16(uint32_t w, half2v& lo, half2v& hi) {
  lo = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, false);
  hi = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(w, 1.0f, true);
}

// Eight E2M1 codes (element i in nibble i) times a float16 scale -> eight
// float16 values in four words (element 2p in the low half of word p).
// Each product has at most 6 significant bits, so it is exact.
__device__ __forceinline__ void dequant8_f16(uint32_t codes, half2v s2, uint32_t out[4]) {
  // the byte-select operand must be a literal
  out[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 0) * s2);
  out[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 1) * s2);
  out[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 2) * s2);
  out[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(codes, 1.0f, 3) * s2);
}

}  // namespace fql
