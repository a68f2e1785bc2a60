// NVFP4 quantizer kernels for gfx950: fused block-diagonal Hadamard (FWHT),
// per-16 amax, E4M3 block scale, E2M1 encode, nibble packing.
//
// What is computed (vLLM write-ups: "TorchNvFp4LinearKernel" quantizes the
// activation with the layer's input global scale into packed FP4 bytes plus
// block scales; "QUTLASS NVFP4 online transforms" fuses the block-diagonal
// Hadamard rotation, normalised by 1/sqrt(n) with n in {16,32,64,128}, into
// that quantizer):
//   v   = x (float32), rotated per b-chunk if b > 0
//   a   = max |v| over each 16-element block
//   s   = E4M3_RNE_satfinite(fl32(fl32(a / 6) * g))
//   r   = fl32(g / s), or 0 when s == 0
//   q_i = E2M1_RNE_satfinite(fl32(v_i * r)), sign of v_i kept
//
// Work mapping: one thread per 16-element block. Consecutive threads take
// consecutive blocks of a row, so a wave reads 64 * 32 contiguous bytes of
// bf16 (two 16-byte loads per lane) and writes 64 * 8 contiguous code bytes.
// The FWHT's first four butterfly strides (1, 2, 4, 8) stay inside a thread;
// strides 16, 32, 64 pair a lane with lane ^ 1, ^ 2, ^ 4 through cross-lane
// shuffles (a b-chunk is b/16 <= 8 adjacent lanes of one wave).
//
// The block arithmetic (fql_quant.h) runs with FMA contraction off: every
// float operation is the single IEEE operation the definition names.
#include <algorithm>

#include "fql_device.h"
#include "fql_internal.h"
#include "fql_quant.h"

namespace fql {

// Canonical output: codes [rows][K/2], scales [rows][K/16].
template <typename TIn, int HB>
__global__ __launch_bounds__(256) void quant_nvfp4_canonical_kernel(
    const TIn* __restrict__ x, int64_t rows, int64_t K, int64_t ldx, float g, int aligned16,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, const float* __restrict__ g_dev) {
  if (g_dev != nullptr) g = *g_dev;  // per-call global scale computed on the device
  const int64_t nblk = K / 16;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const bool active = i < rows * nblk;
  const int64_t m = active ? i / nblk : 0;
  const int64_t kb = active ? i - m * nblk : 0;
  float v[16];
  if (active) {
    Loader<TIn>::load16(x + m * ldx + kb * 16, aligned16 != 0, v);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = 0.0f;
  }
  if constexpr (HB > 0) fwht_block<HB>(v, kb);
  if (!active) return;
  uint32_t lo, hi, s;
  quant_block(v, g, lo, hi, s);
  *reinterpret_cast<uint2*>(codes + m * (K / 2) + kb * 8) = make_uint2(lo, hi);
  scales[m * nblk + kb] = (uint8_t)s;
}

// GEMM operand output: the exactly dequantized activation x_hat = e2m1(q)*s
// in float16, in the MFMA A-fragment order the GEMM reads (see gemm_nvfp4):
//   [Mp/16][Kp/32][lane 0..63][8 halves], lane = kq*16 + (m%16), k = 32*ks + 8*kq + i.
// Rows >= M and columns >= K are written as zeros.
// Work mapping: a wave takes R rows x J = 64/R consecutive 16-blocks, lane =
// r + R*j, so every 16-byte store of a block's halves lands next to the
// same block's stores for the wave's other rows: R * 16 contiguous bytes
// per store instruction group (a wave writes 2 * J runs of 16 * R bytes).
// R = 16 (J = 4) unless the rotation needs 8 blocks per chunk (b = 128: R = 8).
//
// PK = 1 writes the activation packed exactly like a weight (codes and scales
// in the packed weight layout, rows padded to Mp): 0.5625 bytes per element
// instead of x_hat's 2, and the small-M GEMV dequantizes its A fragments the
// way it dequantizes the weight's. The same block arithmetic gives the same
// codes and scales, so both forms hold the same operand values.
template <int HB, int PK>
__global__ __launch_bounds__(256) void quant_nvfp4_xhat_kernel(
    const uint16_t* __restrict__ x, int M, int K, int64_t ldx, float g, int aligned16, int Mp,
    int Kp, _Float16* __restrict__ xhat, const float* __restrict__ g_dev) {
  constexpr uint32_t R = HB == 128 ? 8u : 16u;
  constexpr uint32_t J = 64u / R;
  // 32-bit index arithmetic: the launcher checks Mp * Kp / 16 < 2^31
  const uint32_t ncg = (uint32_t)Kp / (16u * J);    // block groups per row
  const uint32_t w = blockIdx.x * 4u + (threadIdx.x >> 6);
  if (w >= ((uint32_t)Mp / R) * ncg) return;         // whole waves only
  if (g_dev != nullptr) g = *g_dev;                  // per-call global scale computed on the device
  const uint32_t lane = threadIdx.x & 63u;
  const uint32_t rg = w / ncg, cg = w - rg * ncg;
  const uint32_t m = rg * R + lane % R;
  const uint32_t kb = cg * J + lane / R;
  const bool real = (m < (uint32_t)M) && (kb * 16u < (uint32_t)K);
  float v[16];
  if (real) {
    Loader<uint16_t>::load16(x + (int64_t)m * ldx + kb * 16u, aligned16 != 0, v);
  } else {
#pragma unroll
    for (int e = 0; e < 16; ++e) v[e] = 0.0f;
  }
  if constexpr (HB > 0) fwht_block<HB, (int)R>(v, kb);
  uint32_t lo, hi, s;
  quant_block(v, g, lo, hi, s);
  if constexpr (PK) {
    // tile t = m/16, row n = m%16, chunk c = kb/8, step j = (kb%8)/2, half h = kb%2:
    // lo goes to lane (2h)*16 + n, hi to lane (2h+1)*16 + n, dword j of the chunk's
    // 16-byte lane slot; the scale to slot 2n + h, byte 4(c%4) + j of the 4-chunk group
    const uint32_t KC = (uint32_t)Kp / 128u, KC4 = (KC + 3u) / 4u;
    const uint32_t t = m >> 4, n = m & 15u, c = kb >> 3, j = (kb >> 1) & 3u, h = kb & 1u;
    uint8_t* out = reinterpret_cast<uint8_t*>(xhat);
    uint32_t* cw = reinterpret_cast<uint32_t*>(out + ((size_t)(t * KC + c) * 64u + 2u * h * 16u + n) * 16u) + j;
    cw[0] = lo;
    cw[64] = hi;  // next 16-lane group: 256 bytes on
    uint8_t* sc = out + (size_t)((uint32_t)Mp / 2u) * (uint32_t)Kp;
    sc[((size_t)(t * KC4 + (c >> 2)) * 32u + 2u * n + h) * 16u + 4u * (c & 3u) + j] = (uint8_t)s;
    return;
  }
  const _Float16 sh = e4m3_to_f16(s);
  const half2v s2 = {sh, sh};
  uint32_t hw[8];
  dequant8_f16(lo, s2, hw);
  dequant8_f16(hi, s2, hw + 4);
  const uint32_t ks = kb >> 1;           // 32-deep K step of the block
  const uint32_t kq0 = (kb & 1u) * 2u;   // first of its two 8-deep quarters
  const uint32_t ml = m & 15u;
  uint4v* base = reinterpret_cast<uint4v*>(xhat) + ((m >> 4) * ((uint32_t)Kp / 32u) + ks) * 64u;
  base[kq0 * 16u + ml] = uint4v{hw[0], hw[1], hw[2], hw[3]};
  base[(kq0 + 1u) * 16u + ml] = uint4v{hw[4], hw[5], hw[6], hw[7]};
}

// max |v| (after the optional rotation) into amax[0 .. nslots) (as ordered
// uint bits; non-negative floats compare like their bit patterns): workgroup w
// folds its maximum into slot w % nslots, so the atomics of many workgroups
// spread over several addresses. The slots must be 0 first.
// Grid-stride over 16-blocks (the stride is a multiple of 64, so the lanes of
// a Hadamard chunk stay adjacent in one wave); one atomic per workgroup.
template <typename TIn, int HB>
__global__ __launch_bounds__(256) void amax_kernel(const TIn* __restrict__ x, int64_t rows,
                                                   int64_t K, int64_t ldx, int aligned16,
                                                   uint32_t* __restrict__ amax, int nslots) {
  __shared__ float wmax[4];
  const int64_t nblk = K / 16;
  const int64_t total = rows * nblk;
  const int64_t stride = (int64_t)gridDim.x * 256;
  float a = 0.0f;
  for (int64_t base = (int64_t)blockIdx.x * 256; base < total; base += stride) {
    const int64_t i = base + threadIdx.x;
    const bool active = i < total;
    const int64_t m = active ? i / nblk : 0;
    const int64_t kb = active ? i - m * nblk : 0;
    float v[16];
    if (active) {
      Loader<TIn>::load16(x + m * ldx + kb * 16, aligned16 != 0, v);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = 0.0f;
    }
    if constexpr (HB > 0) fwht_block<HB>(v, kb);
#pragma unroll
    for (int e = 0; e < 16; ++e) a = __builtin_fmaxf(a, __builtin_fabsf(v[e]));
  }
  for (int off = 32; off > 0; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = a;
  __syncthreads();
  if (threadIdx.x == 0) {
    const float b = __builtin_fmaxf(__builtin_fmaxf(wmax[0], wmax[1]), __builtin_fmaxf(wmax[2], wmax[3]));
    atomicMax(amax + blockIdx.x % nslots, __float_as_uint(b));
  }
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------

template <typename TIn>
static hipError_t launch_canonical(const TIn* x, int64_t rows, int64_t K, int64_t ldx, float g,
                                   int hb, bool aligned, uint8_t* codes, uint8_t* scales,
                                   const float* g_dev, hipStream_t st) {
  const int64_t total = rows * (K / 16);
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  const int al = aligned ? 1 : 0;
  switch (hb) {
    case 0: quant_nvfp4_canonical_kernel<TIn, 0><<<grid, block, 0, st>>>(x, rows, K, ldx, g, al, codes, scales, g_dev); break;
    case 16: quant_nvfp4_canonical_kernel<TIn, 16><<<grid, block, 0, st>>>(x, rows, K, ldx, g, al, codes, scales, g_dev); break;
    case 32: quant_nvfp4_canonical_kernel<TIn, 32><<<grid, block, 0, st>>>(x, rows, K, ldx, g, al, codes, scales, g_dev); break;
    case 64: quant_nvfp4_canonical_kernel<TIn, 64><<<grid, block, 0, st>>>(x, rows, K, ldx, g, al, codes, scales, g_dev); break;
    case 128: quant_nvfp4_canonical_kernel<TIn, 128><<<grid, block, 0, st>>>(x, rows, K, ldx, g, al, codes, scales, g_dev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float g,
                                   int hb, bool aligned, uint8_t* codes, uint8_t* scales,
                                   hipStream_t st, const float* g_dev) {
  return launch_canonical<uint16_t>(x, M, K, ldx, g, hb, aligned, codes, scales, g_dev, st);
}

hipError_t launch_quant_nvfp4_f32(const float* w, int64_t N, int64_t K, int64_t ldw, float g,
                                  int hb, bool aligned, uint8_t* codes, uint8_t* scales,
                                  hipStream_t st) {
  return launch_canonical<float>(w, N, K, ldw, g, hb, aligned, codes, scales, nullptr, st);
}

template <int PK>
static hipError_t launch_xhat_t(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float g, int hb,
                                bool aligned, int64_t Mp, int64_t Kp, _Float16* xhat,
                                const float* g_dev, hipStream_t st) {
  const int64_t total = Mp * (Kp / 16);
  if (total >= ((int64_t)1 << 31) || Kp >= ((int64_t)1 << 31) || Mp % 16 != 0) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((total + 255) / 256)), block(256);
  const int al = aligned ? 1 : 0;
  const int m = (int)M, k = (int)K, mp = (int)Mp, kp = (int)Kp;
  switch (hb) {
    case 0: quant_nvfp4_xhat_kernel<0, PK><<<grid, block, 0, st>>>(x, m, k, ldx, g, al, mp, kp, xhat, g_dev); break;
    case 16: quant_nvfp4_xhat_kernel<16, PK><<<grid, block, 0, st>>>(x, m, k, ldx, g, al, mp, kp, xhat, g_dev); break;
    case 32: quant_nvfp4_xhat_kernel<32, PK><<<grid, block, 0, st>>>(x, m, k, ldx, g, al, mp, kp, xhat, g_dev); break;
    case 64: quant_nvfp4_xhat_kernel<64, PK><<<grid, block, 0, st>>>(x, m, k, ldx, g, al, mp, kp, xhat, g_dev); break;
    case 128: quant_nvfp4_xhat_kernel<128, PK><<<grid, block, 0, st>>>(x, m, k, ldx, g, al, mp, kp, xhat, g_dev); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_quant_nvfp4_xhat(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float g,
                                   int hb, bool aligned, int64_t Mp, int64_t Kp, _Float16* xhat,
                                   const float* g_dev, hipStream_t st) {
  return launch_xhat_t<0>(x, M, K, ldx, g, hb, aligned, Mp, Kp, xhat, g_dev, st);
}

hipError_t launch_quant_nvfp4_apack(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, float g,
                                    int hb, bool aligned, int64_t Mp, int64_t Kp, uint8_t* apack,
                                    const float* g_dev, hipStream_t st) {
  return launch_xhat_t<1>(x, M, K, ldx, g, hb, aligned, Mp, Kp, reinterpret_cast<_Float16*>(apack),
                          g_dev, st);
}

template <typename TIn>
static hipError_t launch_amax(const TIn* x, int64_t rows, int64_t K, int64_t ldx, int hb,
                              bool aligned, float* out, int nslots, hipStream_t st) {
  if (nslots < 1 || nslots > 64) return hipErrorInvalidValue;
  uint32_t* o = reinterpret_cast<uint32_t*>(out);
  zero_u32_kernel<<<1, 64, 0, st>>>(o, nslots);
  const int64_t total = rows * (K / 16);
  const dim3 grid((unsigned)std::min<int64_t>((total + 255) / 256, 2048)), block(256);
  const int al = aligned ? 1 : 0;
  switch (hb) {
    case 0: amax_kernel<TIn, 0><<<grid, block, 0, st>>>(x, rows, K, ldx, al, o, nslots); break;
    case 16: amax_kernel<TIn, 16><<<grid, block, 0, st>>>(x, rows, K, ldx, al, o, nslots); break;
    case 32: amax_kernel<TIn, 32><<<grid, block, 0, st>>>(x, rows, K, ldx, al, o, nslots); break;
    case 64: amax_kernel<TIn, 64><<<grid, block, 0, st>>>(x, rows, K, ldx, al, o, nslots); break;
    case 128: amax_kernel<TIn, 128><<<grid, block, 0, st>>>(x, rows, K, ldx, al, o, nslots); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_amax_bf16(const uint16_t* x, int64_t M, int64_t K, int64_t ldx, int hb,
                            bool aligned, float* out, hipStream_t st, int nslots) {
  return launch_amax<uint16_t>(x, M, K, ldx, hb, aligned, out, nslots, st);
}

hipError_t launch_amax_f32(const float* w, int64_t N, int64_t K, int64_t ldw, int hb, bool aligned,
                           float* out, hipStream_t st) {
  return launch_amax<float>(w, N, K, ldw, hb, aligned, out, 1, st);
}

}  // namespace fql
