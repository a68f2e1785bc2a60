// Measurement aids for bench.py, built as libfql_calib.so next to the layer's
// library and not part of the layer: a streaming read that gives the HBM
// bandwidth a kernel can reach for a given number of bytes, and loops of
// independent MFMAs that give the matrix-core rate a kernel can reach
// (float16 32x32x16, and the scaled 16x16x128 on FP8 and FP4 operands), to
// report next to the published peaks. Host-side functions only enqueue
// kernels on the caller's stream and return 0, or a negative value on a bad
// argument or launch error.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t uint4v __attribute__((ext_vector_type(4)));
typedef _Float16 half8 __attribute__((ext_vector_type(8)));
typedef float float4v __attribute__((ext_vector_type(4)));
typedef float float16v __attribute__((ext_vector_type(16)));
typedef int int8v __attribute__((ext_vector_type(8)));

// Each thread reads four 16-byte words per round (four loads in flight),
// grid-stride over n16 words; the XOR of everything read is folded into one
// word per workgroup so that no load can be dropped.
__global__ __launch_bounds__(256) void stream_read_kernel(const uint4v* __restrict__ p, int64_t n16,
                                                          uint32_t* __restrict__ sink) {
  uint32_t acc = 0;
  const int64_t stride = (int64_t)gridDim.x * 256;
  int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const uint4v a = __builtin_nontemporal_load(p + i);
    const uint4v b = __builtin_nontemporal_load(p + i + stride);
    const uint4v c = __builtin_nontemporal_load(p + i + 2 * stride);
    const uint4v d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const uint4v a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  for (int off = 32; off > 0; off >>= 1) acc ^= __shfl_xor(acc, off);
  __shared__ uint32_t w[4];
  if ((threadIdx.x & 63) == 0) w[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = w[0] ^ w[1] ^ w[2] ^ w[3];
}

// KIND 0: v_mfma_f32_32x32x16_f16 (32768 flops); 1: the scaled
// 16x16x128 MFMA on FP8 (E4M3) operands; 2: the same on FP4 (E2M1) operands
// (16x16x128: 65536 flops); 3 and 4: the scaled 32x32x64 MFMA on FP4 and on
// FP8 operands (131072 flops). Eight independent accumulators per wave, `iters`
// rounds; the operands depend on the lane so nothing folds away.
template <int KIND>
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  float acc_sum = 0.0f;
  if constexpr (KIND == 0) {
    half8 a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = (_Float16)(0.001f * (float)(lane + i));
      b[i] = (_Float16)(0.002f * (float)(lane - i));
    }
    // distinct starting values keep the chains from being merged
    float16v c[8];
    for (int j = 0; j < 8; ++j) {
      c[j] = float16v{};
      c[j][0] = (float)j;
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c[j], 0, 0, 0);
    for (int j = 0; j < 8; ++j) acc_sum += c[j][j];
  } else if constexpr (KIND >= 3) {
    constexpr int F = KIND == 4 ? 0 : 4;  // operand format: 0 = E4M3, 4 = E2M1
    int8v a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x01010101 * ((lane + i) & 7);
      b[i] = 0x02020202 * ((lane + 3 * i) & 3);
    }
    float16v c[8];
    for (int j = 0; j < 8; ++j) {
      c[j] = float16v{};
      c[j][0] = (float)j;
    }
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c[j], F, F, 0, 127, 0, 127);
    for (int j = 0; j < 8; ++j) acc_sum += c[j][j];
  } else {
    constexpr int F = KIND == 1 ? 0 : 4;  // operand format: 0 = E4M3, 4 = E2M1
    int8v a, b;
    for (int i = 0; i < 8; ++i) {
      a[i] = 0x01010101 * ((lane + i) & 7);
      b[i] = 0x02020202 * ((lane + 3 * i) & 3);
    }
    float4v c[8];
    for (int j = 0; j < 8; ++j) c[j] = float4v{(float)j, 0.f, 0.f, 0.f};
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        c[j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c[j], F, F, 0, 127, 0, 127);
    for (int j = 0; j < 8; ++j) acc_sum += c[j][j & 3];
  }
  if (acc_sum == 12345.678f) sink[blockIdx.x] = acc_sum;  // keeps the loop; never true in practice
}

}  // namespace

extern "C" {

// Streaming read of `bytes` (a positive multiple of 16, 16-byte aligned) at
// buf on `grid` workgroups of 256 threads; sink holds `grid` words.
int fql_calib_stream_read(const void* buf, int64_t bytes, int grid, uint32_t* sink, void* stream) {
  if (!buf || !sink || bytes <= 0 || bytes % 16 != 0 || grid < 1 ||
      reinterpret_cast<uintptr_t>(buf) % 16 != 0)
    return -1;
  stream_read_kernel<<<grid, 256, 0, static_cast<hipStream_t>(stream)>>>(
      static_cast<const uint4v*>(buf), bytes / 16, sink);
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

// `grid` workgroups of 4 waves, each wave `iters` rounds of 8 MFMAs of kind
// `kind` (0: float16 32x32x16, 1: scaled FP8 16x16x128, 2: scaled FP4
// 16x16x128, 3: scaled FP4 32x32x64, 4: scaled FP8 32x32x64). Flops =
// grid * 4 * iters * 8 * (32768 for kind 0, 65536 for 1 and 2, 131072 for 3 and 4).
int fql_calib_mfma_loop(int kind, int grid, int iters, float* sink, void* stream) {
  if (!sink || grid < 1 || iters < 1) return -1;
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (kind == 0) mfma_loop_kernel<0><<<grid, 256, 0, st>>>(iters, sink);
  else if (kind == 1) mfma_loop_kernel<1><<<grid, 256, 0, st>>>(iters, sink);
  else if (kind == 2) mfma_loop_kernel<2><<<grid, 256, 0, st>>>(iters, sink);
  else if (kind == 3) mfma_loop_kernel<3><<<grid, 256, 0, st>>>(iters, sink);
  else if (kind == 4) mfma_loop_kernel<4><<<grid, 256, 0, st>>>(iters, sink);
  else return -1;
  return hipGetLastError() == hipSuccess ? 0 : -3;
}

}  // extern "C"
