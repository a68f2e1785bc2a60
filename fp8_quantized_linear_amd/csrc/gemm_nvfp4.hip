// NVFP4 block-scaled GEMM + epilogue for gfx950.
//
// What is computed (vLLM write-ups "TorchNvFp4LinearKernel" and "B12X
// CuTe-DSL linear backends", NVFP4 apply path): the scaled matmul of the
// quantized activation with the packed NVFP4 weight, then multiplication by
// alpha (product of the two global dequant scales), then the bias, cast to
// the activation dtype (bf16), exactly N output columns:
//   y[m][n] = bf16( alpha * sum_k xh[m][k] * wh[n][k] + bias[n] )
// with xh = e2m1(q)*s and wh likewise (per-16 E4M3 scales, exact values).
//
// How (MI355X): a dequantized NVFP4 value e2m1 * e4m3 has at most 6
// significant bits and lies in [2^-10, 2688], so it is exact in float16; the
// products of two of them are exact in float32. The GEMM therefore runs on
// the dense f16 MFMA (v_mfma_f32_16x16x32_f16) with float32 accumulation,
// which keeps every product exact. The CDNA4 scaled FP4 MFMA only takes
// power-of-two (E8M0) scales per 32 elements, which cannot carry an E4M3
// per-16 scale exactly.
//
// Work split: a workgroup is 4 waves. It owns MT 16-row M tiles and
// 4 * NT 16-column N tiles (NT per wave) and one K range (split-K).
//  * A (activation): the quantizer already wrote x_hat as float16 in MFMA
//    A-fragment order [Mp/16][Kp/32][lane][8]; a K chunk (128) of the
//    workgroup's MT tiles is copied into LDS (double buffered) and every wave
//    reads its fragments with one conflict-free 16-byte LDS read per lane.
//  * B (weight): each wave streams its own N tiles straight from HBM into
//    registers: per 128-wide K chunk one 16-byte code load and one 4-byte
//    scale load per lane and tile, prefetched one chunk ahead, dequantized in
//    registers (byte-permute lookup + packed f16 multiply by the scale).
//  * Epilogue: with one split, alpha, bias and the bf16 cast are fused here;
//    with several splits each writes float32 partials and a reduce kernel
//    sums them in split order (deterministic) and applies the epilogue.
#include "fql_device.h"
#include "fql_internal.h"

namespace fql {

template <int MT, int NT>
__global__ __launch_bounds__(256) void gemm_nvfp4_kernel(
    const _Float16* __restrict__ xhat, const uint8_t* __restrict__ wcodes,
    const uint8_t* __restrict__ wscales, int M, int N, int64_t Kp, int ntiles_n,
    int kc_per_split, float alpha, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t ldy, float* __restrict__ partial, int64_t Np) {
  __shared__ __attribute__((aligned(16))) uint4v a_lds[2][MT * 4][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int64_t KC = Kp / 128;
  const int64_t KS = Kp / 32;
  const int mgroup = blockIdx.y;
  const int split = blockIdx.z;
  const int64_t c_begin = (int64_t)split * kc_per_split;
  int64_t c_end = c_begin + kc_per_split;
  if (c_end > KC) c_end = KC;
  const int tile0 = (blockIdx.x * 4 + wave) * NT;

  bool tvalid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) tvalid[nt] = (tile0 + nt) < ntiles_n;

  // A chunk copy: MT*4 KB per chunk, one 16-byte slot per thread per m tile.
  // Thread tid covers k step (tid >> 6) and fragment lane (tid & 63).
  const uint4v* xsrc = reinterpret_cast<const uint4v*>(xhat);
  auto a_src = [&](int mt, int64_t c) -> const uint4v* {
    return xsrc + ((((int64_t)mgroup * MT + mt) * KS + c * 4 + (tid >> 6)) * 64 + (tid & 63));
  };

  const uint4v* bq_base[NT];
  const uint32_t* bs_base[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t t = tvalid[nt] ? tile0 + nt : 0;
    bq_base[nt] = reinterpret_cast<const uint4v*>(wcodes) + (t * KC) * 64 + lane;
    bs_base[nt] = reinterpret_cast<const uint32_t*>(wscales) + (t * KC) * 32 + (lane & 15) * 2 +
                  ((lane >> 4) >> 1);
  }

  float4v acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};

  uint4v bq[NT], bq_next[NT];
  uint32_t bs[NT], bs_next[NT];
  uint4v areg[MT];

  if (c_begin < c_end) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a_lds[0][mt * 4 + (tid >> 6)][tid & 63] = *a_src(mt, c_begin);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bq[nt] = tvalid[nt] ? bq_base[nt][c_begin * 64] : uint4v{0u, 0u, 0u, 0u};
      bs[nt] = tvalid[nt] ? bs_base[nt][c_begin * 32] : 0u;
    }
  }
  __syncthreads();

  int buf = 0;
  for (int64_t c = c_begin; c < c_end; ++c) {
    const bool more = (c + 1) < c_end;
    if (more) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) areg[mt] = *a_src(mt, c + 1);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bq_next[nt] = tvalid[nt] ? bq_base[nt][(c + 1) * 64] : uint4v{0u, 0u, 0u, 0u};
        bs_next[nt] = tvalid[nt] ? bs_base[nt][(c + 1) * 32] : 0u;
      }
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      half8 bfrag[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const uint32_t w = ks == 0 ? bq[nt].x : ks == 1 ? bq[nt].y : ks == 2 ? bq[nt].z : bq[nt].w;
        const float sf = e4m3_decode_nonneg((bs[nt] >> (8 * ks)) & 0xFFu);
        const _Float16 sh = (_Float16)sf;  // exact: E4M3 values are float16 values
        const half2v s2 = {sh, sh};
        uint32_t hw[4];
        e2m1x8_to_f16(w, hw);
        half8 b;
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          half2v v = __builtin_bit_cast(half2v, hw[p]) * s2;  // exact product
          b[2 * p] = v[0];
          b[2 * p + 1] = v[1];
        }
        bfrag[nt] = b;
      }
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const half8 a = __builtin_bit_cast(half8, a_lds[buf][mt * 4 + ks][lane]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bfrag[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    }
    if (more) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) a_lds[buf ^ 1][mt * 4 + (tid >> 6)][tid & 63] = areg[mt];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        bq[nt] = bq_next[nt];
        bs[nt] = bs_next[nt];
      }
    }
    __syncthreads();
    buf ^= 1;
  }

  // Output: lane holds rows 4*(lane/16) + i, column lane % 16 of each tile.
  const int col = lane & 15;
  const int row0 = 4 * (lane >> 4);
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    if (!tvalid[nt]) continue;
    const int n = (tile0 + nt) * 16 + col;
    if (partial == nullptr) {
      if (n >= N) continue;
      const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = (mgroup * MT + mt) * 16 + row0 + i;
          if (m < M) y[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16_bits(alpha * acc[mt][nt][i] + bv);
        }
      }
    } else {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = (mgroup * MT + mt) * 16 + row0 + i;
          if (m < M) partial[((int64_t)split * M + m) * Np + n] = acc[mt][nt][i];
        }
      }
    }
  }
}

// Sum split-K partials in split order, then alpha, bias, bf16.
__global__ __launch_bounds__(256) void splitk_reduce_kernel(const float* __restrict__ partial,
                                                            int splits, int M, int N, int64_t Np,
                                                            float alpha,
                                                            const uint16_t* __restrict__ bias,
                                                            uint16_t* __restrict__ y, int64_t ldy) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (int64_t)M * N) return;
  const int64_t m = i / N, n = i - m * N;
  float s = 0.0f;
  for (int z = 0; z < splits; ++z) s += partial[((int64_t)z * M + m) * Np + n];
  const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
  y[m * ldy + n] = (uint16_t)f32_to_bf16_bits(alpha * s + bv);
}

GemmPlan plan_gemm_nvfp4(int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  const PackedDims d = packed_dims(N, K);
  p.Np = d.Np;
  p.Kp = d.Kp;
  p.mt = M <= 16 ? 1 : M <= 32 ? 2 : M <= 64 ? 4 : 8;
  p.nt = p.mt <= 2 ? 2 : 4;
  p.Mp = round_up(M, 16 * p.mt);
  const int64_t ntiles = p.Np / 16;
  const int64_t gx = (ntiles + 4 * p.nt - 1) / (4 * p.nt);
  const int64_t gy = p.Mp / (16 * p.mt);
  const int64_t KC = p.Kp / 128;
  int64_t splits = 1;
  const int64_t target = 1024;  // workgroups: 4 per CU on 256 CUs
  if (gx * gy < target) splits = (target + gx * gy - 1) / (gx * gy);
  if (splits > KC) splits = KC;
  if (splits < 1) splits = 1;
  p.kc_per_split = (int)((KC + splits - 1) / splits);
  p.splits = (int)((KC + p.kc_per_split - 1) / p.kc_per_split);
  p.xhat_bytes = round_up(p.Mp * p.Kp * 2, 256);
  p.partial_bytes = p.splits > 1 ? round_up((int64_t)p.splits * M * p.Np * 4, 256) : 0;
  p.total_bytes = p.xhat_bytes + p.partial_bytes;
  return p;
}

template <int MT, int NT>
static void launch_gemm_t(const GemmPlan& p, const _Float16* xhat, const uint8_t* packed, int64_t M,
                          int64_t N, float alpha, const uint16_t* bias, uint16_t* y, int64_t ldy,
                          float* partial, hipStream_t st) {
  const int64_t ntiles = p.Np / 16;
  const dim3 grid((unsigned)((ntiles + 4 * NT - 1) / (4 * NT)), (unsigned)(p.Mp / (16 * MT)),
                  (unsigned)p.splits);
  const uint8_t* wcodes = packed;
  const uint8_t* wscales = packed + p.Np * p.Kp / 2;
  gemm_nvfp4_kernel<MT, NT><<<grid, 256, 0, st>>>(
      xhat, wcodes, wscales, (int)M, (int)N, p.Kp, (int)ntiles, p.kc_per_split, alpha, bias, y, ldy,
      p.splits > 1 ? partial : nullptr, p.Np);
}

hipError_t launch_gemm_nvfp4(const GemmPlan& p, const _Float16* xhat, const uint8_t* packed,
                             int64_t M, int64_t N, float alpha, const uint16_t* bias, uint16_t* y,
                             int64_t ldy, float* partial, hipStream_t st) {
  if (p.mt == 1 && p.nt == 2) {
    launch_gemm_t<1, 2>(p, xhat, packed, M, N, alpha, bias, y, ldy, partial, st);
  } else if (p.mt == 2 && p.nt == 2) {
    launch_gemm_t<2, 2>(p, xhat, packed, M, N, alpha, bias, y, ldy, partial, st);
  } else if (p.mt == 4 && p.nt == 4) {
    launch_gemm_t<4, 4>(p, xhat, packed, M, N, alpha, bias, y, ldy, partial, st);
  } else if (p.mt == 8 && p.nt == 4) {
    launch_gemm_t<8, 4>(p, xhat, packed, M, N, alpha, bias, y, ldy, partial, st);
  } else {
    return hipErrorInvalidValue;
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || p.splits == 1) return e;
  const int64_t total = M * N;
  splitk_reduce_kernel<<<(unsigned)((total + 255) / 256), 256, 0, st>>>(
      partial, p.splits, (int)M, (int)N, p.Np, alpha, bias, y, ldy);
  return hipGetLastError();
}

}  // namespace fql
