// General block-diagonal transform fused into the NVFP4 activation quantizer
// (gfx950), and the device-side dynamic global scale.
//
// What is computed ("QUTLASS NVFP4 online transforms" write-up: the fused
// quantizer takes any block-diagonal transform of block size b in
// {16, 32, 64, 128}, with the normalisation folded into the stored matrix;
// its dense branch applies the matrix to the activation as a linear layer):
//   v[c*b + i] = sum_j T[i][j] * x[c*b + j]        per row, per b-chunk c
// then the NVFP4 block quantizer on v (16-element blocks, E4M3 scale from the
// block maximum and the global scale g, E2M1 codes), exactly as the plain
// quantizer does it.
//
// The transform is a small dense contraction, so it runs on MFMA: per
// 16-row tile of x and per chunk, D = T * X^T on v_mfma_f32_16x16x32_bf16
// (16x16x16 for b = 16), A = T (16 output rows i x 32 inputs j, held in
// registers for the wave's whole life), B = X^T (16 activation rows as
// columns). D's lane layout puts the 16 elements of one NVFP4 block (one
// 16-row tile of i) in the four lanes l, l^16, l^32, l^48 with the same
// activation row, four consecutive elements each, so the block maximum is
// two cross-lane steps and every lane encodes its own four codes.
//
// The products T[i][j] * x[j] are exact in float32; their sum is accumulated
// by the MFMA in float32 in the hardware's order, so v can differ from the
// exactly rounded sum in the last bits (codes and scales then differ only
// at near-ties). A zero sum is forced to +0 (v + 0.0f). The quantizer's own
// float steps are single IEEE float32 operations (contraction off).
//
// The input is HBM-bound (each x element is read once, x_hat written once);
// the MFMA work is 2*b flops per element, a few percent of the chip's bf16
// rate at the HBM-bound pace.
#include <algorithm>

#include "fql_device.h"
#include "fql_internal.h"

namespace fql {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t uint2v __attribute__((ext_vector_type(2)));

enum TrMode { TR_CANON = 0, TR_XHAT = 1, TR_AMAX = 2, TR_VALUES = 3, TR_PACKED = 4 };

template <int B>
struct TrShape {
  static constexpr int KD = B == 16 ? 16 : 32;  // MFMA depth
  static constexpr int JS = B / KD;             // depth steps per chunk
  static constexpr int IT = B / 16;             // 16-row output tiles per chunk (= NVFP4 blocks)
  static constexpr int XW = KD / 16 * 2;        // 32-bit words of x per lane per depth step (2 or 4)
};

// Operand fragment: 8 bf16 (depth 32) or 4 bf16 (depth 16) as 32-bit words.
template <int B>
struct Frag {
  uint32_t w[TrShape<B>::XW];
};

template <int B>
__device__ __forceinline__ float4v mfma_step(const Frag<B>& a, const Frag<B>& b, float4v c) {
  if constexpr (TrShape<B>::KD == 32) {
    const uint4v av = {a.w[0], a.w[1], a.w[2], a.w[3]};
    const uint4v bv = {b.w[0], b.w[1], b.w[2], b.w[3]};
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, av),
                                                   __builtin_bit_cast(bf16x8, bv), c, 0, 0, 0);
  } else {
    const uint2v av = {a.w[0], a.w[1]};
    const uint2v bv = {b.w[0], b.w[1]};
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, av),
                                                     __builtin_bit_cast(s16x4, bv), c, 0, 0, 0);
  }
}

// XW words (2*XW bf16) from p; AL: p is 16-byte (depth 32) or 8-byte aligned.
template <int B, int AL>
__device__ __forceinline__ void load_frag(const uint16_t* p, bool valid, Frag<B>& f) {
  constexpr int XW = TrShape<B>::XW;
  if (!valid) {
#pragma unroll
    for (int i = 0; i < XW; ++i) f.w[i] = 0u;
    return;
  }
  if constexpr (AL) {
    if constexpr (XW == 4) {
      const uint4v t = *reinterpret_cast<const uint4v*>(p);
      f.w[0] = t.x; f.w[1] = t.y; f.w[2] = t.z; f.w[3] = t.w;
    } else {
      const uint2v t = *reinterpret_cast<const uint2v*>(p);
      f.w[0] = t.x; f.w[1] = t.y;
    }
  } else {
#pragma unroll
    for (int i = 0; i < XW; ++i) f.w[i] = (uint32_t)p[2 * i] | ((uint32_t)p[2 * i + 1] << 16);
  }
}

// Chunks in flight per wave (register ring): DEPTH - 1 chunks are loading
// while one is computed. The T fragments take 128 VGPRs at b = 128, which
// leaves room for a 3-deep ring at two waves per SIMD.
template <int B>
constexpr int ring_depth() { return B == 128 ? 3 : 4; }

// One launch: waves = mtiles * cw_count; wave (mt, cw) takes chunks cw,
// cw + cw_count, ... of its 16-row tile. Rows >= M are loaded from row M - 1
// (in bounds) and masked at the output, so every load is unconditional and
// the loop is wave-uniform: the compiler then waits for exactly the ring
// slot a chunk needs.
template <int B, int MODE, int AL>
__global__ __launch_bounds__(256) void transform_quant_kernel(
    const uint16_t* __restrict__ x, int M, int K, int64_t ldx, const uint16_t* __restrict__ T,
    float g, const float* __restrict__ g_dev, int mtiles, int cw_count, uint8_t* __restrict__ codes,
    uint8_t* __restrict__ scales, _Float16* __restrict__ xhat, int Kp, float* __restrict__ vout,
    int64_t ldv, uint32_t* __restrict__ amax) {
#pragma clang fp contract(off)
  using S = TrShape<B>;
  constexpr int D = ring_depth<B>();
  const int lane = threadIdx.x & 63;
  const int wid = __builtin_amdgcn_readfirstlane(blockIdx.x * 4 + (threadIdx.x >> 6));
  // whole waves only; in the amax mode the surplus waves of the last workgroup
  // stay for its barrier (their maximum is not read)
  if (MODE != TR_AMAX && wid >= mtiles * cw_count) return;
  const bool wave_live = wid < mtiles * cw_count;
  const int mt = wid / cw_count;
  const int cw = wid - mt * cw_count;
  const int ml = lane & 15;   // activation row within the tile (D column)
  const int q = lane >> 4;    // lane group: D rows 4q..4q+3, operand depth 8q.. (4q.. at depth 16)
  const int m = mt * 16 + ml;
  const bool row_ok = m < M;
  if (MODE != TR_AMAX && g_dev != nullptr) g = *g_dev;

  // A fragments of T, kept for every chunk: row 16*it + ml, depth KD*js + q*(KD/4)
  Frag<B> ta[S::IT][S::JS];
#pragma unroll
  for (int it = 0; it < S::IT; ++it)
#pragma unroll
    for (int js = 0; js < S::JS; ++js)
      load_frag<B, 1>(T + (int64_t)(16 * it + ml) * B + S::KD * js + q * (S::KD / 4), true, ta[it][js]);

  const int nchunks = K / B;
  const uint16_t* xrow = x + (int64_t)(row_ok ? m : M - 1) * ldx + q * (S::KD / 4);
  // TR_PACKED: 16-block kb of row r into the packed weight layout with
  // mtiles * 16 rows (tile t = r/16, row n = r%16, chunk ch = kb/8, step
  // j = (kb%8)/2, half h = kb%2: lo to lane (2h)*16 + n and hi to lane
  // (2h+1)*16 + n, dword j of the chunk's 16-byte slot; the scale to slot
  // 2n + h, byte 4(ch%4) + j of the 4-chunk scale group)
  auto store_packed = [&](int r, int kb, uint32_t lo, uint32_t hi, uint32_t sb) {
    const uint32_t KC = (uint32_t)Kp / 128u, KC4 = (KC + 3u) / 4u;
    const uint32_t t = (uint32_t)r >> 4, n = (uint32_t)r & 15u, ch = (uint32_t)kb >> 3;
    const uint32_t j = ((uint32_t)kb >> 1) & 3u, h = (uint32_t)kb & 1u;
    uint8_t* out = reinterpret_cast<uint8_t*>(xhat);
    uint32_t* cw32 = reinterpret_cast<uint32_t*>(out + ((size_t)(t * KC + ch) * 64u + 2u * h * 16u + n) * 16u) + j;
    cw32[0] = lo;
    cw32[64] = hi;  // next 16-lane group: 256 bytes on
    out[(size_t)(mtiles * 8) * (uint32_t)Kp + ((size_t)(t * KC4 + (ch >> 2)) * 32u + 2u * n + h) * 16u +
        4u * (ch & 3u) + j] = (uint8_t)sb;
  };
  float wave_max = 0.0f;

  // ring slot n % D holds the chunk cw + n * cw_count (loads past the last
  // chunk re-read the last one; they are never used)
  Frag<B> xr[D][S::JS];
  auto load_chunk = [&](int c, Frag<B>* dst) {
    const int cc = c < nchunks ? c : nchunks - 1;
#pragma unroll
    for (int js = 0; js < S::JS; ++js) load_frag<B, AL>(xrow + (int64_t)cc * B + S::KD * js, true, dst[js]);
  };
  if (wave_live) {
#pragma unroll
    for (int d = 0; d < D - 1; ++d) load_chunk(cw + d * cw_count, xr[d]);
  }

  for (int c = wave_live ? cw : nchunks; c < nchunks;) {
#pragma unroll
    for (int u = 0; u < D; ++u) {
      if (c >= nchunks) break;
      load_chunk(c + (D - 1) * cw_count, xr[(u + D - 1) % D]);
#pragma unroll
      for (int it = 0; it < S::IT; ++it) {
        float4v acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int js = 0; js < S::JS; ++js) acc = mfma_step<B>(ta[it][js], xr[u][js], acc);
        float v[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = row_ok ? acc[r] + 0.0f : 0.0f;  // an exactly zero sum is +0
        const int k0 = c * B + 16 * it + 4 * q;  // first of this lane's four elements
        float a = __builtin_fmaxf(__builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1])),
                                  __builtin_fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3])));
        if constexpr (MODE == TR_VALUES) {
          if (row_ok) *reinterpret_cast<float4v*>(vout + (int64_t)m * ldv + k0) = float4v{v[0], v[1], v[2], v[3]};
          continue;
        }
        if constexpr (MODE == TR_AMAX) {
          wave_max = __builtin_fmaxf(wave_max, a);
          continue;
        }
        // block maximum over the four lanes holding this row's 16 elements
        a = __builtin_fmaxf(a, __shfl_xor(a, 16));
        a = __builtin_fmaxf(a, __shfl_xor(a, 32));
        const float sf = (a / 6.0f) * g;
        const uint32_t s = e4m3_encode_nonneg(sf);
        const float sd = e4m3_decode_nonneg(s);
        const float rcp = sd == 0.0f ? 0.0f : g / sd;
        uint32_t c16 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(0u, v[0] * rcp, v[1] * rcp, 1.0f, 0);
        c16 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(c16, v[2] * rcp, v[3] * rcp, 1.0f, 1);
        if constexpr (MODE == TR_CANON || MODE == TR_PACKED) {
          // gather the block's 8 code bytes into lane q == 0: words (q0 | q1 << 16), (q2 | q3 << 16)
          const uint32_t mine = c16 & 0xFFFFu;
          const uint32_t nb = __shfl_xor(mine, 16);
          const uint32_t lo = (q & 1) == 0 ? (mine | (nb << 16)) : 0u;
          const uint32_t hi = __shfl_xor(lo, 32);
          if constexpr (MODE == TR_CANON) {
            if (q == 0 && row_ok) {
              *reinterpret_cast<uint2v*>(codes + (int64_t)m * (K / 2) + (c * B + 16 * it) / 2) = uint2v{lo, hi};
              scales[(int64_t)m * (K / 16) + c * (B / 16) + it] = (uint8_t)s;
            }
          } else if (q == 0) {  // every row of the tile (rows >= M are zero)
            store_packed(m, c * (B / 16) + it, lo, hi, s);
          }
        } else {  // TR_XHAT: e2m1(q) * s_d in float16 (exact), GEMM A-fragment order
          const _Float16 sh = (_Float16)sd;
          const half2v s2 = {sh, sh};
          const uint32_t h0 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c16, 1.0f, 0) * s2);
          const uint32_t h1 = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(c16, 1.0f, 1) * s2);
          const int ks = k0 >> 5, kq = (k0 >> 3) & 3, e0 = k0 & 7;
          const int64_t idx = (((int64_t)mt * (Kp / 32) + ks) * 64 + kq * 16 + ml) * 8 + e0;
          *reinterpret_cast<uint2v*>(xhat + idx) = uint2v{h0, h1};
        }
      }
      c += cw_count;
    }
  }

  if constexpr (MODE == TR_AMAX) {
    for (int off = 32; off > 0; off >>= 1) wave_max = __builtin_fmaxf(wave_max, __shfl_xor(wave_max, off));
    // one atomic per workgroup, spread over kAmaxSlots addresses (non-negative
    // floats order like their bits)
    __shared__ float wg_max[4];
    if (lane == 0) wg_max[threadIdx.x >> 6] = wave_max;
    __syncthreads();
    if (threadIdx.x == 0) {
      float b = wg_max[0];
      const int nw = min(4, mtiles * cw_count - (int)blockIdx.x * 4);  // waves of this workgroup
      for (int w = 1; w < nw; ++w) b = __builtin_fmaxf(b, wg_max[w]);
      atomicMax(amax + blockIdx.x % kAmaxSlots, __float_as_uint(b));
    }
  }
  if constexpr (MODE == TR_PACKED) {
    // blocks K/16 .. Kp/16 of the tile are zero (codes and scales)
    if (wave_live && cw == 0) {
      for (int kb = K / 16 + q; kb < Kp / 16; kb += 4) store_packed(m, kb, 0u, 0u, 0u);
    }
  }
  if constexpr (MODE == TR_XHAT) {
    // columns K .. Kp of the tile are zero (8 halves per lane per step)
    if (wave_live && cw == 0) {
      for (int k8 = K / 8 + q; k8 < Kp / 8; k8 += 4) {
        const int64_t idx = ((int64_t)mt * (Kp / 32) + (k8 >> 2)) * 64 + (k8 & 3) * 16 + ml;
        reinterpret_cast<uint4v*>(xhat)[idx] = uint4v{0u, 0u, 0u, 0u};
      }
    }
  }
}

__global__ void zero_words_kernel(uint32_t* p, int n) {
  if ((int)threadIdx.x < n) p[threadIdx.x] = 0u;
}

// D1-D3 on the device (one wave): amax = max of the kAmaxSlots partial
// maxima, g = fl32(2688 / amax) (1 when amax = 0, at most 2^118),
// alpha = fl32((1 / g) * (1 / g_w)) in float64.
__global__ void dynamic_scale_kernel(float* __restrict__ scal, float g_w, int with_alpha) {
#pragma clang fp contract(off)
  const int lane = threadIdx.x;
  float a = __uint_as_float(reinterpret_cast<const uint32_t*>(scal)[lane]);
  for (int off = 32; off > 0; off >>= 1) a = __builtin_fmaxf(a, __shfl_xor(a, off));
  if (lane != 0) return;
  float g = 1.0f;
  if (a > 0.0f) g = __builtin_fminf(2688.0f / a, 0x1p118f);
  scal[kAmaxSlots] = a;
  scal[kAmaxSlots + 1] = g;
  if (with_alpha) scal[kAmaxSlots + 2] = (float)((1.0 / (double)g) * (1.0 / (double)g_w));
}

template <int MODE, int AL>
hipError_t launch_tr_mode(int b, dim3 grid, hipStream_t st, const uint16_t* x, int M, int K,
                          int64_t ldx, const uint16_t* T, float g, const float* g_dev, int mtiles,
                          int cwc, uint8_t* codes, uint8_t* scales, _Float16* xhat, int Kp,
                          float* v, int64_t ldv, uint32_t* amax) {
#define FQL_TR(BB)                                                                               \
  transform_quant_kernel<BB, MODE, AL><<<grid, 256, 0, st>>>(x, M, K, ldx, T, g, g_dev, mtiles, cwc, \
                                                             codes, scales, xhat, Kp, v, ldv, amax)
  switch (b) {
    case 16: FQL_TR(16); break;
    case 32: FQL_TR(32); break;
    case 64: FQL_TR(64); break;
    case 128: FQL_TR(128); break;
    default: return hipErrorInvalidValue;
  }
#undef FQL_TR
  return hipGetLastError();
}

}  // namespace

bool transform_aligned(const void* x, int64_t ldx, int b) {
  // operand loads are 16 bytes (8 bf16) for b >= 32 and 8 bytes for b = 16
  const int64_t elems = b == 16 ? 4 : 8;
  return reinterpret_cast<uintptr_t>(x) % (2 * elems) == 0 && ldx % elems == 0;
}

hipError_t launch_transform_nvfp4(const TransformArgs& a, hipStream_t st) {
  if (a.M < 1 || a.K < a.b || a.K % a.b != 0 || a.K >= (1 << 30) || a.rows_out < a.M)
    return hipErrorInvalidValue;
  const int mtiles = (int)((a.rows_out + 15) / 16);
  const int nchunks = (int)(a.K / a.b);
  // as many waves as the chip keeps resident (8 per SIMD, 2 at b = 128 where T
  // takes 128 registers); with few row tiles every wave takes a single chunk
  // (the T fragments come from L2, so reloading them per wave is cheap)
  const int64_t target = a.b == 128 ? 2048 : 8192;
  const int cwc = (int)std::min<int64_t>(nchunks, std::max<int64_t>(1, (target + mtiles - 1) / mtiles));
  const int64_t waves = (int64_t)mtiles * cwc;
  if (waves >= ((int64_t)1 << 31) - 4) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((waves + 3) / 4));
  const int M = (int)a.M, K = (int)a.K, Kp = (int)a.Kp;
  if (a.mode == TR_AMAX) {
    zero_words_kernel<<<1, 64, 0, st>>>(a.amax, kAmaxSlots);
  }
#define FQL_TRM(MODE)                                                                              \
  return a.aligned ? launch_tr_mode<MODE, 1>(a.b, grid, st, a.x, M, K, a.ldx, a.T, a.g, a.g_dev,  \
                                             mtiles, cwc, a.codes, a.scales, a.xhat, Kp, a.v,       \
                                             a.ldv, a.amax)                                         \
                   : launch_tr_mode<MODE, 0>(a.b, grid, st, a.x, M, K, a.ldx, a.T, a.g, a.g_dev,  \
                                             mtiles, cwc, a.codes, a.scales, a.xhat, Kp, a.v,       \
                                             a.ldv, a.amax)
  switch (a.mode) {
    case TR_CANON: FQL_TRM(TR_CANON);
    case TR_XHAT: FQL_TRM(TR_XHAT);
    case TR_AMAX: FQL_TRM(TR_AMAX);
    case TR_VALUES: FQL_TRM(TR_VALUES);
    case TR_PACKED: FQL_TRM(TR_PACKED);
    default: return hipErrorInvalidValue;
  }
#undef FQL_TRM
}

hipError_t launch_dynamic_scale(float* scal, float g_w, bool with_alpha, hipStream_t st) {
  static_assert(kAmaxSlots == 64, "one wave folds the partial maxima");
  dynamic_scale_kernel<<<1, 64, 0, st>>>(scal, g_w, with_alpha ? 1 : 0);
  return hipGetLastError();
}

hipError_t launch_zero_words(uint32_t* p, int n, hipStream_t st) {
  if (n < 0 || n > 64) return hipErrorInvalidValue;
  zero_words_kernel<<<1, 64, 0, st>>>(p, n);
  return hipGetLastError();
}

}  // namespace fql
