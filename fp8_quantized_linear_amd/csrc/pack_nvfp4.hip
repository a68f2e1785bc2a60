// NVFP4 weight packer for gfx950: canonical codes [N][K/2] + scales [N][K/16]
// -> the GEMM operand order described in fql_internal.h (zero padded).
//
// The write-ups re-lay block scales into their GEMM's swizzled layout and pad
// the weight along K when the weight is loaded; here the re-layout targets
// the MFMA B-operand order instead, so that one 16-byte load per lane feeds
// four 16x16x32 MFMA steps and a wave reads 1 KB contiguous per step group.
#include "fql_device.h"
#include "fql_internal.h"

namespace fql {

// One thread per (tile, chunk, lane) 16-byte code slot; the first 16 threads
// of each slot group also move the scales of row n for that chunk.
__global__ __launch_bounds__(256) void pack_nvfp4_kernel(const uint8_t* __restrict__ codes,
                                                        const uint8_t* __restrict__ scales,
                                                        int64_t N, int64_t K, int64_t Np,
                                                        int64_t Kp, uint8_t* __restrict__ packed) {
  const int64_t KC = Kp / 128;
  const int64_t slot = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (t, c, lane)
  if (slot >= (Np / 16) * KC * 64) return;
  const int lane = (int)(slot & 63);
  const int64_t tc = slot >> 6;  // t * KC + c
  const int64_t t = tc / KC, c = tc - t * KC;
  const int n_in = lane & 15, kq = lane >> 4;
  const int64_t n = t * 16 + n_in;
  uint32_t w[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int64_t k = c * 128 + 32 * j + 8 * kq;  // 8 codes = 4 bytes
    uint32_t v = 0u;
    if (n < N && k < K) {
      const uint8_t* src = codes + n * (K / 2) + k / 2;
      // K % 16 == 0, so the 8 codes are all inside the row
      v = (uint32_t)src[0] | ((uint32_t)src[1] << 8) | ((uint32_t)src[2] << 16) |
          ((uint32_t)src[3] << 24);
    }
    w[j] = v;
  }
  *reinterpret_cast<uint4v*>(packed + slot * 16) = uint4v{w[0], w[1], w[2], w[3]};
  if (kq < 2) {
    // scale dword of (row n, chunk c, h = kq): byte j = block 8c + 2j + h
    const int h = kq;
    uint32_t sw = 0u;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t b = c * 8 + 2 * j + h;
      uint32_t v = 0u;
      if (n < N && b * 16 < K) v = scales[n * (K / 16) + b];
      sw |= v << (8 * j);
    }
    const int64_t KC4 = (KC + 3) / 4;
    uint8_t* sdst = packed + Np * Kp / 2 + ((t * KC4 + c / 4) * 32 + n_in * 2 + h) * 16 + (c % 4) * 4;
    *reinterpret_cast<uint32_t*>(sdst) = sw;
  }
}

// Inverse re-layout (packed -> canonical), one thread per canonical 16-block.
__global__ __launch_bounds__(256) void unpack_nvfp4_kernel(const uint8_t* __restrict__ packed,
                                                          int64_t N, int64_t K, int64_t Np,
                                                          int64_t Kp, uint8_t* __restrict__ codes,
                                                          uint8_t* __restrict__ scales) {
  const int64_t nblk = K / 16;
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N * nblk) return;
  const int64_t n = i / nblk, b = i - n * nblk;
  const int64_t KC = Kp / 128;
  const int64_t t = n / 16, c = b / 8;
  const int n_in = (int)(n % 16);
  const int64_t tc = t * KC + c;
  // the block's 16 codes are two 8-code groups: k = 16b and 16b + 8
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    const int64_t k = b * 16 + 8 * half;
    const int64_t kk = k - c * 128;
    const int j = (int)(kk / 32), kq = (int)((kk % 32) / 8);
    const int lane = kq * 16 + n_in;
    const uint8_t* src = packed + (tc * 64 + lane) * 16 + j * 4;
    uint8_t* dst = codes + n * (K / 2) + k / 2;
#pragma unroll
    for (int q = 0; q < 4; ++q) dst[q] = src[q];
  }
  const int jb = (int)((b % 8) / 2), h = (int)(b % 2);
  const int64_t KC4 = (KC + 3) / 4;
  scales[i] = packed[Np * Kp / 2 + ((t * KC4 + c / 4) * 32 + n_in * 2 + h) * 16 + (c % 4) * 4 + jb];
}

// Zero the scale dwords of chunks past KC in the last group of each tile
// (their codes are never read, but the group is loaded as a whole).
__global__ void pack_zero_tail_kernel(uint8_t* __restrict__ packed, int64_t Np, int64_t Kp) {
  const int64_t KC = Kp / 128, KC4 = (KC + 3) / 4;
  const int64_t tail = KC4 * 4 - KC;  // 0..3 chunks
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // (tile, slot, q)
  if (i >= (Np / 16) * 32 * tail) return;
  const int64_t t = i / (32 * tail), r = i - t * 32 * tail;
  const int64_t slot = r / tail, q = KC % 4 + r % tail;
  *reinterpret_cast<uint32_t*>(packed + Np * Kp / 2 + ((t * KC4 + KC4 - 1) * 32 + slot) * 16 + q * 4) = 0u;
}

hipError_t launch_pack_nvfp4(const uint8_t* codes, const uint8_t* scales, int64_t N, int64_t K,
                             uint8_t* packed, hipStream_t st) {
  const PackedDims d = packed_dims(N, K);
  const int64_t tail = d.kc4() * 4 - d.kc();
  if (tail > 0) {
    const int64_t n = (d.Np / 16) * 32 * tail;
    pack_zero_tail_kernel<<<(unsigned)((n + 255) / 256), 256, 0, st>>>(packed, d.Np, d.Kp);
  }
  const int64_t slots = (d.Np / 16) * (d.Kp / 128) * 64;
  pack_nvfp4_kernel<<<(unsigned)((slots + 255) / 256), 256, 0, st>>>(codes, scales, N, K, d.Np,
                                                                     d.Kp, packed);
  return hipGetLastError();
}

hipError_t launch_unpack_nvfp4(const uint8_t* packed, int64_t N, int64_t K, uint8_t* codes,
                               uint8_t* scales, hipStream_t st) {
  const PackedDims d = packed_dims(N, K);
  const int64_t total = N * (K / 16);
  unpack_nvfp4_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(packed, N, K, d.Np, d.Kp,
                                                                       codes, scales);
  return hipGetLastError();
}

}  // namespace fql
