// Device-side format helpers shared by the gfx950 kernels.
//
// Element formats (OCP Microscaling v1.0 and the NVFP4 convention):
//   E2M1: sign, 2-bit exponent, 1-bit mantissa; magnitudes {0,.5,1,1.5,2,3,4,6}.
//   E4M3 (fn): bias 7, largest finite 448, subnormals m * 2^-9.
// All encoders round to nearest, ties to even, and saturate at the largest
// finite value. Every float operation here is plain IEEE float32 (the build
// keeps denormals and correctly rounded division, and the quantizer file turns
// off FMA contraction), so results are bit-identical to any IEEE reference.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fql {

typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2v __attribute__((ext_vector_type(2)));
typedef float float2v __attribute__((ext_vector_type(2)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef uint32_t uint4v __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) { return __uint_as_float(h << 16); }

// float32 -> bfloat16 bits, round to nearest even (NaN stays NaN): gfx950's
// v_cvt_pk_bf16_f32, which was checked equal to the integer rounding
// (b + 0x7FFF + lsb) >> 16 on every non-NaN float32 bit pattern and to give a
// NaN for every NaN input.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

// E4M3 encode of a non-negative float32 (block scales are >= 0).
// Below 2^-6 the quantum is 2^-9 for subnormals and the smallest normal
// binade alike, so rounding there is rint(s * 2^9) (exact scaling); above,
// the float32 mantissa is rounded to 3 bits with ties to even and the
// exponent re-biased from 127 to 7. 448 and above (and +inf) saturate.
__device__ __forceinline__ uint32_t e4m3_encode_nonneg(float s) {
  if (!(s < 448.0f)) return 0x7Eu;
  if (s < 0.015625f) return (uint32_t)__builtin_rintf(s * 512.0f);
  uint32_t b = __float_as_uint(s);
  uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) >> 20;
  return r - (120u << 3);
}

// E4M3 byte (sign ignored) -> float32, exact.
__device__ __forceinline__ float e4m3_decode_nonneg(uint32_t c) {
  uint32_t e = (c >> 3) & 15u, m = c & 7u;
  return e == 0u ? (float)m * 0.001953125f : __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// E2M1 encode, RNE with saturation. The magnitude code counts how many
// decision points |u| has passed; a value exactly on a decision point goes
// to the even code (0.25, 1.25, 2.5, 5 round down; 0.75, 1.75, 3.5 up).
// The sign bit is taken from u, so -0 and small negatives give code 0x8.
__device__ __forceinline__ uint32_t e2m1_encode(float u) {
  float a = __builtin_fabsf(u);
  uint32_t q = (uint32_t)(a > 0.25f) + (uint32_t)(a >= 0.75f) + (uint32_t)(a > 1.25f) +
               (uint32_t)(a >= 1.75f) + (uint32_t)(a > 2.5f) + (uint32_t)(a >= 3.5f) +
               (uint32_t)(a > 5.0f);
  return q | ((__float_as_uint(u) >> 28) & 8u);
}

// E2M1 code -> float32 value, exact.
__device__ __forceinline__ float e2m1_decode(uint32_t c) {
  // magnitude m: 0 -> 0, 1 -> 0.5, 2..7 -> (1 + (m&1)/2) * 2^((m>>1)-1)
  uint32_t m = c & 7u;
  float v = m < 2u ? 0.5f * (float)m
                   : __uint_as_float(((126u + (m >> 1)) << 23) | ((m & 1u) << 22));
  return (c & 8u) ? -v : v;
}

// The float16 high bytes of the E2M1 magnitudes {0,.5,1,1.5,2,3,4,6}
// (their low bytes are zero), as two 4-byte lookup words for v_perm_b32.
constexpr uint32_t kE2M1F16HiLo = 0x3E3C3800u;  // magnitudes 0..3
constexpr uint32_t kE2M1F16HiHi = 0x46444240u;  // magnitudes 4..7

// Eight packed E2M1 codes (element i in bits 4i..4i+3) -> eight float16
// values, as four words (element 2p in the low half of word p).
// Byte lookups via v_perm_b32: magnitudes index the 8-byte table, the sign
// bits are merged in, and the bytes are spread into float16 high halves.
__device__ __forceinline__ void e2m1x8_to_f16(uint32_t w, uint32_t out[4]) {
  uint32_t sel_even = w & 0x07070707u;          // magnitudes of elements 0,2,4,6
  uint32_t sel_odd = (w >> 4) & 0x07070707u;    // magnitudes of elements 1,3,5,7
  uint32_t he = __builtin_amdgcn_perm(kE2M1F16HiHi, kE2M1F16HiLo, sel_even);
  uint32_t ho = __builtin_amdgcn_perm(kE2M1F16HiHi, kE2M1F16HiLo, sel_odd);
  he |= (w << 4) & 0x80808080u;                 // sign bits of even elements
  ho |= w & 0x80808080u;                        // sign bits of odd elements
  // word p = [0x00, he.byte p, 0x00, ho.byte p]; selector 0x0C yields 0x00
  out[0] = __builtin_amdgcn_perm(ho, he, 0x040C000Cu);
  out[1] = __builtin_amdgcn_perm(ho, he, 0x050C010Cu);
  out[2] = __builtin_amdgcn_perm(ho, he, 0x060C020Cu);
  out[3] = __builtin_amdgcn_perm(ho, he, 0x070C030Cu);
}

}  // namespace fql
