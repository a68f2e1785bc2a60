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
// significant bits and lies in [2^-10, 2688], so it is exact in float16, and
// the product of two is exact in float32. The GEMM therefore runs on the
// dense f16 MFMA (v_mfma_f32_16x16x32_f16) with float32 accumulation, which
// keeps every product exact. (The CDNA4 scaled FP4 MFMA takes power-of-two
// E8M0 scales per 32 elements, which cannot carry an E4M3 per-16 scale.)
//
// Operand flow. B (weight) streams from HBM straight into registers: per
// 128-deep K chunk and 16-column tile one 16-byte code load and one 4-byte
// scale load per lane (packed layout in fql_internal.h), dequantized with
// v_cvt_scalef32_pk_f16_fp4 and one packed f16 multiply per two elements.
// A (activation) lives in LDS in MFMA A-fragment order (one conflict-free
// 16-byte read per lane per fragment) and is shared by the 4 waves of a
// workgroup, which own different 16-column tiles.
//
// Two kernels:
//  * linear_gemv_kernel (small M, x rows 16-byte aligned): ONE launch per
//    layer call. Each workgroup quantizes the activation rows straight into
//    LDS (the quantizer's arithmetic, fql_quant.h) and computes its 16-column
//    tiles over the full K, its waves splitting K and adding their partial
//    tiles through LDS in wave order.
//  * gemm_tiled_kernel (larger M): x_hat comes pre-quantized from the
//    quantizer kernel; A chunks are double-buffered through LDS and B is
//    prefetched one chunk ahead. When there are too few output tiles to
//    occupy the GPU, K is split across workgroups: the last workgroup of a
//    tile to arrive sums the float32 partials in split order
//    (deterministic) and applies the epilogue.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "fql_device.h"
#include "fql_gemm.h"
#include "fql_internal.h"
#include "fql_quant.h"

namespace fql {

// ---------------------------------------------------------------------------
// small-M kernel with per-wave LDS rings (kind 4)
// ---------------------------------------------------------------------------
//
// A linear call with M <= 32 is a stream over the weight. W waves of a
// workgroup share NT 16-column tiles and split the K chunks, interleaved (wave
// w takes chunks w, w + W, ..., so a workgroup's waves read neighbouring
// chunks at any time); each wave streams its own chunks (activation, weight
// codes, scale dwords) into a private D-stage LDS ring with direct
// global->LDS loads and waits only for its own loads (explicit vmcnt, no
// workgroup barrier in the loop), so D chunks per wave stay in flight. The
// activation arrives packed like a weight (the quantizer pass writes the MT
// row tiles' codes, then their scales) and each A fragment is dequantized
// exactly like a B fragment: 1.25 KiB per row tile and chunk through the
// ring, the same fp16 operand values as x_hat. Lanes of rows >= M skip their
// loads (an output row depends only on its own A row and rows >= M are never
// stored); a row tile with no row below M loads whole, so every load
// instruction issues and the vmcnt counts hold. The W partial sums are added
// in wave order through LDS at the end (deterministic, no atomics).
template <int MT, int NT>
struct GemvStage {
  uint4v ac[MT][64];   // activation codes of the chunk, per row tile
  uint32_t as[MT][64];  // the lane's activation scale dword, per row tile
  uint4v b[NT][64];     // weight codes (one 16-byte slot per lane and tile)
  uint32_t s[NT][64];   // the lane's weight scale dword of this chunk, per tile
};

template <int L, int K>
struct GemvWait {
  static __device__ __forceinline__ void run(int k) {
    if (k >= K) wait_vmcnt<L * K>();
    else GemvWait<L, K - 1>::run(k);
  }
};
template <int L>
struct GemvWait<L, 0> {
  static __device__ __forceinline__ void run(int) { wait_vmcnt<0>(); }
};

// xa: the packed activation (codes of the 16·MT rows, then their scales).
template <int W, int MT, int NT, int D>
__global__ __launch_bounds__(64 * W) void gemv_ring_kernel(
    const uint8_t* __restrict__ xa, const uint8_t* __restrict__ wcodes,
    const uint8_t* __restrict__ wscales, int M, int N, int64_t Kp, int ntiles, float alpha,
    const float* __restrict__ alpha_dev, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int64_t ldy) {
  if (alpha_dev != nullptr) alpha = *alpha_dev;  // per-call scale computed on the device
  typedef GemvStage<MT, NT> Stage;
  constexpr int L = MT * 2 + NT * 2;  // loads per chunk
  static_assert(L * (D - 1) <= 63, "vmcnt range");
  __shared__ Stage ring[W][D];
  static_assert(sizeof(ring) >= sizeof(float4v) * W * MT * NT * 64, "reduction buffer aliases the ring");
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t KC = Kp / 128, KC4 = (KC + 3) / 4;
  const int64_t tile0 = (int64_t)blockIdx.x * NT;
  // chunk idx of this wave is wave + idx * W
  const int64_t c0 = wave, cs = W;
  const int n = wave < KC ? (int)((KC - wave + W - 1) / W) : 0;
  int64_t bt[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bt[nt] = tile0 + nt < ntiles ? tile0 + nt : ntiles - 1;  // never stored
  // this lane's scale dword within a tile's 512-byte group of four chunks
  const uint32_t s_voff_lane = (uint32_t)(((lane & 15) * 2 + (lane >> 5)) * 16);

  auto issue = [&](Stage& sg, int64_t c) {
    const uint32_t base = lds_offset(&sg);
    // rows >= M are never stored: skip their bytes (the instructions still issue)
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint8_t* ac = uniform_ptr(xa + (mt * KC + c) * 1024);
      const uint8_t* as = uniform_ptr(xa + 8 * MT * Kp + (mt * KC4 + c / 4) * 512);
      if (16 * mt + (lane & 15) < M || 16 * mt >= M) {
        lds_load16(ac, lane * 16, base + (uint32_t)offsetof(Stage, ac) + mt * 1024);
        lds_load4(as, s_voff_lane + (uint32_t)(c & 3) * 4, base + (uint32_t)offsetof(Stage, as) + mt * 256);
      }
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      lds_load16(wcodes + (bt[nt] * KC + c) * 1024, lane * 16,
                 base + (uint32_t)offsetof(Stage, b) + nt * 1024);
      lds_load4(wscales + (bt[nt] * KC4 + c / 4) * 512, s_voff_lane + (uint32_t)(c & 3) * 4,
                base + (uint32_t)offsetof(Stage, s) + nt * 256);
    }
  };

  float4v acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const Stage& sg) {
    uint4v codes[NT];
    uint32_t sw[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      codes[nt] = sg.b[nt][lane];
      sw[nt] = sg.s[nt][lane];
    }
    uint4v acodes[MT];
    uint32_t asw[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      acodes[mt] = sg.ac[mt][lane];
      asw[mt] = sg.as[mt][lane];
    }
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      half8 bf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bf[nt] = b_fragment(dword_of(codes[nt], ks), ChunkScales(sw[nt])[ks]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const half8 a = b_fragment(dword_of(acodes[mt], ks), ChunkScales(asw[mt])[ks]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[nt], acc[mt][nt], 0, 0, 0);
      }
    }
  };

  // chunk idx of this wave lives in stage idx % D; before computing it the
  // wave waits until at most min(D-1, n-1-idx) later chunks are in flight
  Stage* mine = ring[wave];
  const int pre = n < D ? n : D;
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < pre) issue(mine[j], c0 + j * cs);
  for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int idx = i0 + j;
      if (idx < n) {
        const int later = n - 1 - idx;
        GemvWait<L, D - 1>::run(later < D - 1 ? later : D - 1);
        compute(mine[j]);
        if (idx + D < n) {
          __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage reads done before the refill
          issue(mine[j], c0 + (idx + D) * cs);
        }
      }
    }
  }
  wait_vmcnt<0>();
  __syncthreads();  // every wave is done with the ring, which now holds the partial sums

  float4v(*red)[MT * NT][64] = reinterpret_cast<float4v(*)[MT * NT][64]>(&ring[0][0]);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) red[wave][mt * NT + nt][lane] = acc[mt][nt];
  __syncthreads();
#pragma unroll
  for (int f = 0; f < MT * NT; ++f) {
    if (f % W != wave) continue;
    float4v sum = red[0][f][lane];
#pragma unroll
    for (int w = 1; w < W; ++w) sum += red[w][f][lane];
    const int n_col = (int)((tile0 + f % NT) * 16) + (lane & 15);
    if (n_col >= N) continue;
    const float bv = bias ? bf16_bits_to_f32(bias[n_col]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = (f / NT) * 16 + 4 * (lane >> 4) + i;
      if (m < M) y[(int64_t)m * ldy + n_col] = (uint16_t)f32_to_bf16_bits(alpha * sum[i] + bv);
    }
  }
}

// ---------------------------------------------------------------------------
// full-K matrix-vector kernel (small M): no cross-workgroup reduction
// ---------------------------------------------------------------------------
//
// One workgroup owns NTW 16-column tiles and the whole K range; its W waves
// split K into W contiguous parts and their partial sums are added in wave
// order through LDS at the end (deterministic, no global atomics: a
// device-scope arrival counter costs about a microsecond per round trip and
// serialises under contention, which is the whole budget of a decode call).
// The activation's M rows are quantized once per workgroup straight into a
// compact LDS copy x_hat[M][Kp] (float16, 16-byte groups XOR-swizzled by
// row so the 16 fragment rows of a read hit distinct banks); fragment lanes
// for rows >= M read nothing and supply zeros. Weight loads are issued in
// rounds of RC chunks per tile before the round's MFMAs.
// (x is deliberately not __restrict__: the compiler barriers below must pin
//  its loads ahead of the weight loads, which they cannot do for memory the
//  compiler knows no asm statement can touch.)
template <int W, int NTW, int HB, int RC, int QPRE>
__global__ __launch_bounds__(64 * W) void linear_gemv_kernel(
    const uint16_t* x, int M, int K, int64_t ldx, float g, const float* __restrict__ g_dev,
    int aligned16, const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales, int N,
    int64_t Kp, int ntiles, float alpha, const float* __restrict__ alpha_dev,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t ldy) {
  if (g_dev != nullptr) g = *g_dev;  // scales kept in device memory
  if (alpha_dev != nullptr) alpha = *alpha_dev;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  uint4v* xs = reinterpret_cast<uint4v*>(smem);  // [M][Kp/8] 16-byte groups, swizzled
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t KC = Kp / 128;
  const int64_t G8 = Kp / 8;  // 16-byte groups per row
  const int tile0 = blockIdx.x * NTW;
  const int64_t KC4 = (KC + 3) / 4;
  // per-wave K part in whole 4-chunk scale groups
  const int64_t cpw = ((KC + W - 1) / W + 3) / 4 * 4;
  const int64_t cw0 = wave * cpw < KC ? wave * cpw : KC;
  const int64_t cw1 = cw0 + cpw < KC ? cw0 + cpw : KC;

  // weight pointers of this workgroup's tiles (invalid tiles read tile 0)
  const uint4v* qp[NTW];
  const uint4v* sp[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) {
    const int64_t t = (tile0 + j) < ntiles ? tile0 + j : 0;
    qp[j] = reinterpret_cast<const uint4v*>(wcodes) + (t * KC) * 64 + lane;
    sp[j] = reinterpret_cast<const uint4v*>(wscales) + (t * KC4) * 32 + (lane & 15) * 2 + (lane >> 5);
  }
  // register ring of RC chunks per tile (RC a multiple of 4): slot i holds
  // chunk cr + i of the current round; sg holds the matching scale groups
  uint4v bq[NTW][RC];
  uint4v sg[NTW][RC / 4];
  const int64_t c_last = cw1 > cw0 ? cw1 - 1 : 0;  // clamp target: a valid chunk of this tile
  // codes of chunk c into slot i; the scale group of slots 4q..4q+3 is
  // (re)loaded with the first slot of the group at start-up and after the
  // group's last slot has been consumed in the loop
  auto load_codes = [&](int i, int64_t c) {
    c = c < c_last ? c : c_last;  // unconditional, clamped: static outstanding-load count
#pragma unroll
    for (int j = 0; j < NTW; ++j) bq[j][i] = __builtin_nontemporal_load(&qp[j][c * 64]);
  };
  auto load_group = [&](int q, int64_t c_first) {
    const int64_t c = c_first < c_last ? c_first : c_last;
#pragma unroll
    for (int j = 0; j < NTW; ++j) sg[j][q] = __builtin_nontemporal_load(&sp[j][(c / 4) * 32]);
  };
  auto load_slot = [&](int i, int64_t c) {
    load_codes(i, c);
    if ((i & 3) == 0) load_group(i / 4, c);
  };
  // Activation loads go out first: the load counter retires in order, so
  // waiting for x must not have to wait for the (slower) weight stream too.
  // QPRE blocks per thread are prefetched (the plan sizes it to cover all
  // rows when it can); the weight ring follows.
  const int64_t nblk = Kp / 16;
  const int64_t qtotal = (int64_t)M * nblk;
  uint4v xq[QPRE][2];
  bool xact[QPRE];
  int64_t xm[QPRE], xkb[QPRE];
#pragma unroll
  for (int q = 0; q < QPRE; ++q) {
    // branch-free: inactive lanes read block 0 of row 0 (in bounds) and zero it
    const int64_t b = (int64_t)q * 64 * W + tid;
    xact[q] = b < qtotal;
    xm[q] = xact[q] ? b / nblk : 0;
    xkb[q] = xact[q] ? b - xm[q] * nblk : 0;
    const bool real = xact[q] && xkb[q] * 16 < K;
    const uint4v* px = reinterpret_cast<const uint4v*>(x + (real ? xm[q] * ldx + xkb[q] * 16 : 0));
    const uint4v z = uint4v{0u, 0u, 0u, 0u};
    const uint4v l0 = px[0], l1 = px[1];
    xq[q][0] = real ? l0 : z;
    xq[q][1] = real ? l1 : z;
  }
  __asm__ volatile("" ::: "memory");  // keep every x load ahead of the weight loads
#pragma unroll
  for (int i = 0; i < RC; ++i) load_slot(i, cw0 + i);
  __asm__ volatile("" ::: "memory");

  // quantize x rows [0, M) over the full K into the compact LDS copy
  auto quant_store = [&](const float (&v)[16], int64_t m, int64_t kb) {
    uint32_t lo, hi, sc;
    quant_block(v, g, lo, hi, sc);
    const _Float16 sh = e4m3_to_f16(sc);
    const half2v s2 = {sh, sh};
    uint32_t hw[8];
    dequant8_f16(lo, s2, hw);
    dequant8_f16(hi, s2, hw + 4);
    const int64_t gi = kb * 2;  // first 16-byte group of the block
    const int sw = (int)(m & 15);
    xs[m * G8 + ((gi & ~15) | ((gi & 15) ^ sw))] = uint4v{hw[0], hw[1], hw[2], hw[3]};
    xs[m * G8 + (((gi + 1) & ~15) | (((gi + 1) & 15) ^ sw))] = uint4v{hw[4], hw[5], hw[6], hw[7]};
  };
#pragma unroll
  for (int q = 0; q < QPRE; ++q) {  // static trip count: the loads cannot be sunk
    float v[16];
    const uint32_t w[8] = {xq[q][0].x, xq[q][0].y, xq[q][0].z, xq[q][0].w,
                           xq[q][1].x, xq[q][1].y, xq[q][1].z, xq[q][1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      v[2 * i] = __uint_as_float(w[i] << 16);
      v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
    if constexpr (HB > 0) fwht_block<HB>(v, xkb[q]);
    if (xact[q]) quant_store(v, xm[q], xkb[q]);
  }
  for (int64_t b0 = (int64_t)QPRE * 64 * W; b0 < qtotal; b0 += 64 * W) {  // rows beyond the prefetch
    const int64_t b = b0 + tid;
    const bool act = b < qtotal;
    const int64_t m = act ? b / nblk : 0;
    const int64_t kb = act ? b - m * nblk : 0;
    float v[16];
    if (act && kb * 16 < K) {
      Loader<uint16_t>::load16(x + m * ldx + kb * 16, aligned16 != 0, v);
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] = 0.0f;
    }
    if constexpr (HB > 0) fwht_block<HB>(v, kb);
    if (act) quant_store(v, m, kb);
  }
  __syncthreads();

  // MFMA over this wave's K part
  const int r = lane & 15, kq = lane >> 4;
  const bool row_real = r < M;
  float4v acc[NTW];
#pragma unroll
  for (int j = 0; j < NTW; ++j) acc[j] = float4v{0.f, 0.f, 0.f, 0.f};
  for (int64_t cr = cw0; cr < cw1; cr += RC) {
#pragma unroll
    for (int i = 0; i < RC; ++i) {
      const int64_t c = cr + i;
      if (c < cw1) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int64_t gi = c * 16 + ks * 4 + kq;  // 16-byte group of this lane's 8 k values
          uint4v av = uint4v{0u, 0u, 0u, 0u};
          if (row_real) av = xs[r * G8 + ((gi & ~15) | ((gi & 15) ^ r))];
          const half8 a = __builtin_bit_cast(half8, av);
#pragma unroll
          for (int j = 0; j < NTW; ++j) {
            const ChunkScales cs(dword_of(sg[j][i / 4], i & 3));
            const half8 bf = b_fragment(dword_of(bq[j][i], ks), cs[ks]);
            acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf, acc[j], 0, 0, 0);
          }
        }
      }
      load_codes(i, c + RC);  // refill this slot with the chunk RC ahead
      if ((i & 3) == 3) load_group(i / 4, c - 3 + RC);  // group fully consumed
    }
  }

  // reduce the W partial tiles in wave order through LDS (reusing x_hat space)
  __syncthreads();
  float4v* red = reinterpret_cast<float4v*>(smem);  // [W][NTW][64]
#pragma unroll
  for (int j = 0; j < NTW; ++j) red[(wave * NTW + j) * 64 + lane] = acc[j];
  __syncthreads();
  if (wave == 0) {
    const int col = lane & 15, row0 = 4 * (lane >> 4);
#pragma unroll
    for (int j = 0; j < NTW; ++j) {
      float4v s4 = red[j * 64 + lane];
      for (int w = 1; w < W; ++w) {
        const float4v t = red[(w * NTW + j) * 64 + lane];
        s4 = s4 + t;
      }
      const int n = (tile0 + j) * 16 + col;
      if (n < N) {
        const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = row0 + i;
          if (m < M) y[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16_bits(alpha * s4[i] + bv);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// tiled kernel (x_hat from the quantizer kernel)
// ---------------------------------------------------------------------------

// The 4 waves form a WM x (4/WM) grid over the workgroup tile: wave (wm, wn)
// owns MT 16-row tiles and NT 16-column tiles. A (x_hat) chunks for all WM*MT
// row tiles are staged through LDS and read by the 4/WM waves of a row; each
// wave dequantizes only its own NT weight tiles (WM > 1 dequantizes a tile in
// WM waves, trading VALU work for fewer LDS reads: a wave reads MT A fragments
// per NT*MT MFMAs).
template <int MT, int NT, int WM>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(
    const _Float16* __restrict__ xhat, const uint8_t* __restrict__ wcodes,
    const uint8_t* __restrict__ wscales, int M, int N, int64_t Kp, int ntiles, int ngroups,
    int kc_per_split, int splits, float alpha,
    const float* __restrict__ alpha_dev, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int64_t ldy, float4v* __restrict__ partial,
    uint32_t* __restrict__ counters) {
  if (alpha_dev != nullptr) alpha = *alpha_dev;  // per-call scale computed on the device
  constexpr int WN = 4 / WM;
  constexpr int AM = WM * MT;  // 16-row A tiles per workgroup
  __shared__ uint4v a_lds[2][AM * 4][64];
  __shared__ uint32_t s_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int64_t KC = Kp / 128;
  const int64_t KS = Kp / 32;
  // blockIdx.x = (mgroup * ngroups + ngroup) * splits + split
  const int split = blockIdx.x % splits;
  const int tilegrp = blockIdx.x / splits;
  const int ngroup = tilegrp % ngroups;
  const int mgroup = tilegrp / ngroups;
  const int64_t c_begin = (int64_t)split * kc_per_split;
  const int64_t c_end = c_begin + kc_per_split < KC ? c_begin + kc_per_split : KC;
  const int tile0 = (ngroup * WN + wn) * NT;

  bool tvalid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) tvalid[nt] = (tile0 + nt) < ntiles;

  // thread tid stages fragment (f, ks = tid / 64) of every A row tile f
  const uint4v* xsrc = reinterpret_cast<const uint4v*>(xhat);
  auto a_src = [&](int f, int64_t c) -> const uint4v* {
    return xsrc + ((((int64_t)mgroup * AM + f) * KS + c * 4 + wave) * 64 + lane);
  };

  const int64_t KC4 = (KC + 3) / 4;
  const uint4v* bq_base[NT];
  const uint32_t* bs_base[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int64_t t = tvalid[nt] ? tile0 + nt : 0;
    bq_base[nt] = reinterpret_cast<const uint4v*>(wcodes) + (t * KC) * 64 + lane;
    bs_base[nt] = reinterpret_cast<const uint32_t*>(wscales) +
                  ((t * KC4) * 32 + (lane & 15) * 2 + (lane >> 5)) * 4;
  }
  // scale dword of chunk c in the 4-chunk group layout
  auto bs_at = [&](int nt, int64_t c) -> uint32_t {
    return __builtin_nontemporal_load(&bs_base[nt][(c >> 2) * 128 + (c & 3)]);
  };

  float4v acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};

  // Software pipeline over 128-deep chunks, unrolled by two with ping-pong
  // register sets R0/R1 (no register copies, which would force waits):
  //   chunk c (parity p): LDS[p] holds A(c), R[p].b holds B(c), R[1-p].a A(c+1).
  //   compute c; store R[1-p].a to LDS[1-p]; load A(c+2), B(c+2) into R[p].
  // Every global load has one whole iteration to arrive before its use.
  // Indices past the range are clamped (re-reads, cache hits) so the number
  // of outstanding loads is static.
  auto clampc = [&](int64_t c) -> int64_t { return c < c_end ? c : c_end - 1; };
  uint4v bq0[NT], bq1[NT];
  uint32_t bs0[NT], bs1[NT];
  uint4v ar0[AM], ar1[AM];
#pragma unroll
  for (int f = 0; f < AM; ++f) a_lds[0][f * 4 + wave][lane] = *a_src(f, c_begin);
#pragma unroll
  for (int f = 0; f < AM; ++f) ar1[f] = *a_src(f, clampc(c_begin + 1));
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {  // invalid tiles read tile 0 (in bounds, never stored)
    bq0[nt] = __builtin_nontemporal_load(&bq_base[nt][c_begin * 64]);
    bs0[nt] = bs_at(nt, c_begin);
    bq1[nt] = __builtin_nontemporal_load(&bq_base[nt][clampc(c_begin + 1) * 64]);
    bs1[nt] = bs_at(nt, clampc(c_begin + 1));
  }
  __syncthreads();

  auto compute = [&](int buf, const uint4v (&bq)[NT], const uint32_t (&bs)[NT]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      half8 bf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bf[nt] = b_fragment(dword_of(bq[nt], ks), ChunkScales(bs[nt])[ks]);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const half8 a = __builtin_bit_cast(half8, a_lds[buf][(wm * MT + mt) * 4 + ks][lane]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[nt], acc[mt][nt], 0, 0, 0);
      }
    }
  };
  auto advance = [&](int buf, int64_t c, uint4v (&ar_store)[AM], uint4v (&ar_load)[AM],
                     uint4v (&bq)[NT], uint32_t (&bs)[NT]) {
#pragma unroll
    for (int f = 0; f < AM; ++f) a_lds[buf ^ 1][f * 4 + wave][lane] = ar_store[f];
    const int64_t c2 = clampc(c + 2);
#pragma unroll
    for (int f = 0; f < AM; ++f) ar_load[f] = *a_src(f, c2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bq[nt] = __builtin_nontemporal_load(&bq_base[nt][c2 * 64]);
      bs[nt] = bs_at(nt, c2);
    }
    __syncthreads();
  };

  int64_t c = c_begin;
  // (scheduling barriers keep each half's work from being hoisted into the
  //  other half, where it would wait on the youngest loads)
  for (; c + 1 < c_end; c += 2) {
    compute(0, bq0, bs0);
    __builtin_amdgcn_sched_barrier(0);
    advance(0, c, ar1, ar0, bq0, bs0);
    __builtin_amdgcn_sched_barrier(0);
    compute(1, bq1, bs1);
    __builtin_amdgcn_sched_barrier(0);
    advance(1, c + 1, ar0, ar1, bq1, bs1);
    __builtin_amdgcn_sched_barrier(0);
  }
  if (c < c_end) compute(0, bq0, bs0);  // odd chunk count: last chunk

  float4v* slab = partial + (int64_t)tilegrp * splits * (4 * MT * NT * 64);
  finish_tile<MT, NT, WM>(acc, M, N, mgroup * AM * 16, ngroup * WN * NT * 16, split, splits,
                          alpha, bias, y, ldy, slab, counters + tilegrp, &s_flag);
}

// ---------------------------------------------------------------------------
// LDS-ring tiled kernel on 32x32x16 MFMAs
// ---------------------------------------------------------------------------
//
// Workgroup: 4 waves; wave w owns a column slice of the tile and all of its
// rows, so every weight tile is dequantized by exactly one wave and the
// activation fragments (read by all four waves) come from LDS. Every global
// -> LDS transfer is a direct LDS load (global_load_lds_*), so the data in
// flight holds no registers and an ST-deep ring of per-chunk stages runs
// ST-1 chunks (128-deep K slices) ahead of the MFMAs. The loads are issued
// with inline assembly and waited for with explicit s_waitcnt vmcnt(n): the
// compiler does not track LDS-DMA completion per stage and would otherwise
// wait for the whole ring before every LDS read.
// The MFMA is v_mfma_f32_32x32x16_f16: twice the work of a 16x16x32 one for
// the same operand bytes, so a wave spends half as many issue slots on MFMAs
// and the dequantization, LDS reads and loads fit between them (one wave per
// SIMD: VALU work only overlaps the matrix pipe when it is issued between the
// MFMAs, in program order). One 16-deep K step is exactly one NVFP4 block, so
// a weight fragment carries a single scale per lane.
//   Workgroup tile (MT*32) rows x (4*NT*32) columns; wave w owns columns
//   [w*NT*32, (w+1)*NT*32) and all rows.
//   A fragment (32 rows x 16 k) of step s: lane l takes row l%32 and
//   k = 16s + 8*(l/32) + 0..7, i.e. 16-row tile 2a + (l%32)/16, 32-deep step
//   s/2, quarter kq = 2*(s%2) + l/32 of the x_hat fragment layout.
//   B fragment (16 k x 32 columns) of step s: lane l takes column l%32 of
//   the 32-column tile (16-column packed tile 2b + (l%32)/16) and the same k;
//   its codes are dword s/2 of the packed slot kq*16 + l%16, its scale byte
//   s/2 of the slot's scale dword (l%16)*2 + s%2 for the chunk.
// Per chunk and 32-column tile a lane therefore loads two code slots (even
// and odd steps) and two scale dwords.
template <int MT, int NT, int WN>
struct LdsStage32 {
  uint4v a[MT * 2 * 4][64];       // [16-row tile][32-deep step][lane] x_hat fragments
  uint4v bq[WN * NT * 2][64];     // [column wave][32-col tile][even/odd steps][lane] codes
  uint32_t bs[WN * NT * 2][64];   // [column wave][32-col tile][even/odd steps][lane] scales
};

// WN = 8 doubles the column waves: two per SIMD, so a stalled wave (a
// barrier, a wait) leaves the matrix pipe to the other wave of its SIMD; each
// owns all MT row tiles and its own NT column tiles, so every weight fragment
// is dequantized once and feeds MT MFMAs, and loads half as many activation
// pieces per chunk (every other 16-row tile).
template <int MT, int NT, int ST, int OCC, int WN = 4>
__global__ __launch_bounds__(64 * WN, OCC) void gemm_lds32_kernel(
    const _Float16* __restrict__ xhat, const uint8_t* __restrict__ wcodes,
    const uint8_t* __restrict__ wscales, int M, int N, int64_t Kp, int ntiles, int ngroups,
    int kc_per_split, int dp, int splits, int xg, float alpha,
    const float* __restrict__ alpha_dev, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int64_t ldy, float4v* __restrict__ partial,
    uint32_t* __restrict__ counters) {
  if (alpha_dev != nullptr) alpha = *alpha_dev;  // per-call scale computed on the device
  static_assert(ST >= 3 && ST <= 4, "ring depth (chunk i+1 must be issued a whole chunk ahead)");
  static_assert(WN == 4 || WN == 8, "4 or 8 column waves");
  constexpr int TS = WN / 4;             // 16-row tile stride of a wave's activation pieces
  constexpr int NA = 2 * MT / TS;        // activation piece loads per chunk per wave
  static_assert(NA >= 1, "every wave loads activation pieces");
  constexpr int NLB = 2 * NT;            // code (and scale) slot loads per chunk per wave
  constexpr int L = NA + 2 * NLB;        // LDS loads per chunk per wave
  static_assert(L * (ST - 2) <= 63, "vmcnt range");
  typedef LdsStage32<MT, NT, WN> Stage;
  __shared__ Stage stage[ST];
  __shared__ uint32_t s_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wn = wave;  // column slice
  const int64_t KC = Kp / 128;
  const int64_t KC4 = (KC + 3) / 4;
  // Workgroups [0, dp) compute whole tiles; after them each remaining tile
  // takes `splits` consecutive workgroups, one K range each. Tile slot v
  // (v < dp: workgroup v itself) maps to a tile in the XCD-grouped order when
  // xg > 0 (a bijection over all slots, and for v < dp the order of the
  // hardware's XCD assignment), else row-major: mgroup * ngroups + ngroup.
  const int b = blockIdx.x;
  const bool whole = b < dp;
  const int vslot = whole ? b : dp + (b - dp) / splits;
  const int split = whole ? 0 : (b - dp) % splits;
  const int nsplit = whole ? 1 : splits;
  const int ntile = dp + ((int)gridDim.x - dp) / splits;
  const int tilegrp = xg > 0 ? xcd_grouped_tile(vslot, ntile, ngroups, xg) : vslot;
  const int sslot = whole ? 0 : vslot - dp;  // partial slab and counter of a split tile
  const int ngroup = tilegrp % ngroups;
  const int mgroup = tilegrp / ngroups;
  const int64_t c_begin = whole ? 0 : (int64_t)split * kc_per_split;
  const int64_t c_last = whole ? KC : c_begin + kc_per_split;
  const int64_t c_end = c_last < KC ? c_last : KC;
  const int nch = (int)(c_end - c_begin);
  const int tile16_0 = (ngroup * WN + wn) * NT * 2;  // first packed 16-column tile of the wave

  // wave-uniform global bases; per-lane byte offsets. A wave loads the
  // 32-deep step wn % 4 of every TS-th 16-row tile, from tile wn / 4 on.
  const int64_t a_tile_stride = (Kp / 32) * 1024;  // bytes between 16-row x_hat tiles
  const uint8_t* a_base = reinterpret_cast<const uint8_t*>(xhat) +
                          ((int64_t)mgroup * MT * 2 * (Kp / 32) + wn % 4) * 1024 +
                          (wn / 4) * a_tile_stride;
  const uint32_t a_voff = lane * 16;
  const int jc = lane & 31, hh = lane >> 5;  // column in the 32-column tile, k half
  // Per-lane offsets of the code and scale slots this wave loads: slot (b, e)
  // of 32-column tile b holds the even (e = 0) or odd (e = 1) steps. A
  // 16-column tile past the end is clamped to the last one (read, never
  // stored); the host keeps the packed blob below 4 GiB so that these 32-bit
  // offsets cannot wrap.
  uint32_t q_voff[NLB], s_voff[NLB];
#pragma unroll
  for (int i = 0; i < NLB; ++i) {
    const int b = i / 2;
    const int e = i % 2;
    int64_t tl = tile16_0 + 2 * b + (jc >> 4);
    tl = tl < ntiles ? tl : ntiles - 1;
    q_voff[i] = (uint32_t)(tl * KC * 1024 + ((2 * e + hh) * 16 + (jc & 15)) * 16);
    s_voff[i] = (uint32_t)(tl * KC4 * 512 + ((jc & 15) * 2 + e) * 16);
  }

  // The scalar bases of chunk c's loads into stage sg, computed once per chunk
  // (chunks past the range are clamped: a static number of loads per chunk).
  struct Refill {
    const uint8_t* a;  // activation row tile 0 of the chunk
    const uint8_t* q;  // weight codes of the chunk
    const uint8_t* s;  // the chunk's scale dword column
    uint32_t la, lq, ls;  // this wave's LDS destinations in the stage
  };
  // the wave's slot i sits at slot index (wn*NT + b)*2 + e = wn*NT*2 + i of the stage
  auto refill_of = [&](Stage& sg, int64_t c) -> Refill {
    c = c < c_end ? c : c_end - 1;
    Refill r;
    r.a = uniform_ptr(a_base + c * 4096);
    r.q = uniform_ptr(wcodes + c * 1024);
    r.s = uniform_ptr(wscales + (c >> 2) * 512 + (c & 3) * 4);
    r.la = __builtin_amdgcn_readfirstlane(lds_offset(&sg.a[(wn / 4) * 4 + wn % 4][0]));
    r.lq = __builtin_amdgcn_readfirstlane(lds_offset(&sg.bq[wn * NT * 2][0]));
    r.ls = __builtin_amdgcn_readfirstlane(lds_offset(&sg.bs[wn * NT * 2][0]));
    return r;
  };
  // LDS load number e (0 <= e < L) of a chunk
  auto issue_one = [&](const Refill& r, int e) {
    if (e < NA) {
      lds_load16(r.a + e * TS * a_tile_stride, a_voff, r.la + e * TS * 4 * 1024);
    } else if (e < NA + NLB) {
      const int i = e - NA;
      lds_load16(r.q, q_voff[i], r.lq + i * 1024);
    } else {
      const int i = e - NA - NLB;
      lds_load4(r.s, s_voff[i], r.ls + i * 256);
    }
  };
  auto issue = [&](Stage& sg, int64_t c) {
    const Refill r = refill_of(sg, c);
#pragma unroll
    for (int e = 0; e < L; ++e) issue_one(r, e);
  };

  float16v acc[MT][NT];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b) acc[a][b] = float16v{};

  // Software pipeline over the eight 16-deep steps of a chunk: step s issues
  // the LDS reads of step s+1's activation fragments, then its MFMAs
  // interleaved with step s+1's dequantization; between steps 6 and 7 the
  // wave waits for the next chunk's stage, passes the workgroup barrier and
  // reads the next chunk's weight codes and first activation fragments.
  constexpr int MFMAS = MT * NT;                              // per step
  constexpr int VPM = (8 * NT + MFMAS - 1) / MFMAS;           // dequantization VALU per MFMA
  const int a_lane = ((lane & 31) >> 4) * 4 * 64 + hh * 16 + (lane & 15);  // within a[][] of stage
  uint4v bq[NT][2];
  uint32_t bsw[NT][2];
  half8 bf[2][NT];
  uint4v af[2][MT];
  auto a_frag = [&](const Stage& sg, int a, int s) -> uint4v {
    return (&sg.a[0][0])[a_lane + ((2 * a) * 4 + (s >> 1)) * 64 + 2 * (s & 1) * 16];
  };
  // the column slice's codes and scales (the wave's own loads)
  auto read_head_b = [&](const Stage& sg) {
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        bq[b][e] = sg.bq[(wn * NT + b) * 2 + e][lane];
        bsw[b][e] = sg.bs[(wn * NT + b) * 2 + e][lane];
      }
  };
  // the first step's activation fragments (loaded by all waves)
  auto read_head_a = [&](const Stage& sg) {
#pragma unroll
    for (int a = 0; a < MT; ++a) af[0][a] = a_frag(sg, a, 0);
  };
  auto read_head = [&](const Stage& sg) {
    read_head_b(sg);
    read_head_a(sg);
  };
  auto dequant = [&](int buf, int s) {
#pragma unroll
    for (int b = 0; b < NT; ++b)
      bf[buf][b] = b_fragment(dword_of(bq[b][s & 1], s >> 1), ChunkScales(bsw[b][s & 1])[s >> 1]);
  };
  auto mfmas = [&](int buf) {
#pragma unroll
    for (int a = 0; a < MT; ++a) {
      const half8 av = __builtin_bit_cast(half8, af[buf][a]);
#pragma unroll
      for (int b = 0; b < NT; ++b)
        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bf[buf][b], acc[a][b], 0, 0, 0);
    }
  };
  // refill (when given) receives chunk rc's loads, spread over the seven steps
  // so that the address unit works while the MFMAs run
  auto steps0to6 = [&](const Stage& sg, Stage& refill, int64_t rc) {
    const Refill rf = refill_of(refill, rc);
#pragma unroll
    for (int s = 0; s < 7; ++s) {
      const int cur = s & 1, nxt = cur ^ 1;
#pragma unroll
      for (int a = 0; a < MT; ++a) af[nxt][a] = a_frag(sg, a, s + 1);
#pragma unroll
      for (int e = s * L / 7; e < (s + 1) * L / 7; ++e) issue_one(rf, e);
      __builtin_amdgcn_sched_barrier(0);
      dequant(nxt, s + 1);
      mfmas(cur);
#pragma unroll
      for (int i = 0; i < MFMAS; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x002, VPM, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // prologue: chunks 0 .. ST-2 in flight, chunk 0's head in registers
#pragma unroll
  for (int p = 0; p < ST - 1; ++p) issue(stage[p], c_begin + p);
  wait_vmcnt<L * (ST - 2)>();
  stage_barrier();
  read_head(stage[0]);
  dequant(0, 0);
  __builtin_amdgcn_sched_barrier(0);

  // Ring protocol: chunk i lives in stage i % ST. While chunk i is computed,
  // stage (i-1) % ST (chunk i-1's, freed by the previous mid-chunk barrier;
  // for i = 0 the one stage the prologue left empty) receives chunk i+ST-1.
  // At the mid-chunk barrier of chunk i, chunk i+1 has landed and everyone
  // has finished reading chunk i's activation fragments.
  for (int i0 = 0; i0 < nch; i0 += ST) {
#pragma unroll
    for (int j = 0; j < ST; ++j) {
      if (i0 + j < nch) {
        steps0to6(stage[j], stage[(j + ST - 1) % ST], c_begin + i0 + j + ST - 1);
        const bool more = i0 + j + 1 < nch;
        wait_vmcnt<L * (ST - 2)>();  // this wave's loads of chunk i+1 have landed
        if (more) read_head_b(stage[(j + 1) % ST]);  // its own loads
        stage_barrier();             // everyone's have, and stage j has been read by all
        if (more) read_head_a(stage[(j + 1) % ST]);
        __builtin_amdgcn_sched_barrier(0);
        if (more) dequant(0, 0);
        mfmas(1);
#pragma unroll
        for (int i = 0; i < MFMAS; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i >= MFMAS / 4) __builtin_amdgcn_sched_group_barrier(0x002, VPM + 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    }
  }
  wait_vmcnt<0>();  // no LDS load may still be in flight when the workgroup ends

  const int m0 = mgroup * MT * 32, n0 = ngroup * WN * NT * 32;
  if (nsplit == 1) {
    // a whole tile: through the ring's LDS, once every wave's loads have landed
    static_assert(sizeof(stage) >= (size_t)MT * 32 * StagedPitch<WN * NT * 32>::P * 2, "staged tile fits the ring");
    __syncthreads();
    write_tile32_staged<MT, NT, WN>(acc, M, N, m0, n0, wn, alpha, bias, y, ldy,
                                    reinterpret_cast<uint16_t*>(&stage[0]));
  } else {
    float4v* slab = partial + (int64_t)sslot * splits * (WN * MT * NT * 4 * 64);
    finish_tile32<MT, NT, WN>(acc, M, N, m0, n0, wn, split, nsplit, alpha, bias, y, ldy, slab,
                              counters + sslot, &s_flag);
  }
}

// ---------------------------------------------------------------------------
// planning and launch
// ---------------------------------------------------------------------------

static constexpr int kCUs = 256;

// Benchmarking aid: the override spec "kind=0,waves=8,ntw=2,rc=4" or
// "kind=1,mt=4,nt=1,splits=2" (FQL_PLAN, or fql_set_plan_override) replaces
// the launch-plan heuristics (results change at most in the order of the
// float32 sum over K).
struct GemmOverride {
  int kind = -1, waves = 0, ntw = 0, rc = 0, mt = 0, nt = 0, wm = 0, st = 0, splits = 0, xg = -1, cw = 0;
  int tail = 0;  // kind 3: 1 = never split the last round's tiles, 2..4 = split them that many ways
};
static GemmOverride gemm_override() {
  GemmOverride o;
  const std::string s = plan_override(kOverrideNvfp4);
  if (s.empty()) return o;
  size_t pos = 0;
  while (pos < s.size()) {
    size_t end = s.find(',', pos);
    if (end == std::string::npos) end = s.size();
    const std::string kv = s.substr(pos, end - pos);
    const size_t eq = kv.find('=');
    if (eq != std::string::npos) {
      const std::string k = kv.substr(0, eq);
      const int v = std::atoi(kv.c_str() + eq + 1);
      if (k == "kind") o.kind = v;
      else if (k == "waves" && (v == 4 || v == 8 || v == 16)) o.waves = v;
      else if (k == "ntw" && (v == 1 || v == 2 || v == 4)) o.ntw = v;
      else if (k == "rc" && (v == 4 || v == 8)) o.rc = v;
      else if (k == "mt" && (v == 1 || v == 2 || v == 4 || v == 8)) o.mt = v;
      else if (k == "nt" && (v == 1 || v == 2 || v == 4)) o.nt = v;
      else if (k == "wm" && (v == 1 || v == 2 || v == 4)) o.wm = v;
      else if (k == "st" && v >= 2 && v <= 8) o.st = v;
      else if (k == "splits" && v >= 1 && v <= 64) o.splits = v;
      else if (k == "xg" && v >= 0 && v <= 64) o.xg = v;
      else if (k == "cw" && (v == 4 || v == 8)) o.cw = v;
      else if (k == "tail" && v >= 1 && v <= 4) o.tail = v;
    }
    pos = end + 1;
  }
  return o;
}
static constexpr int64_t kCounterBytes = kWorkspaceCounterBytes;
static constexpr int64_t kGemvMaxLds = 64 * 1024;    // compact activation copy in LDS
static constexpr int64_t kGemvMaxRedundantBlocks = 1 << 20;  // workgroups x 16-blocks quantized

GemmPlan plan_gemm_nvfp4(int64_t M, int64_t N, int64_t K, bool aligned, bool rotated) {
  GemmPlan p{};
  const PackedDims d = packed_dims(N, K);
  p.Np = d.Np;
  p.Kp = d.Kp;
  const int64_t KC = p.Kp / 128;
  const int64_t ntiles = p.Np / 16;
  const GemmOverride ov = gemm_override();
  // The fused kernel re-quantizes the activation in every workgroup; keep it
  // while that redundant work stays small (measured: gate_up at M = 8 is
  // faster through the quantizer kernel + tiled GEMM).
  const int64_t quant_blocks = (int64_t)M * (p.Kp / 16);
  bool gemv_ok = aligned && M <= 16 && M * p.Kp * 2 <= kGemvMaxLds &&
                 (ov.kind == 0 || ntiles * quant_blocks <= kGemvMaxRedundantBlocks);
  // Measured on the decode shapes: the fused kernel wins at M = 1 and, for
  // narrow layers with K = 4096 (N < 16384), up to M = 16; long K (K = 14336)
  // and wide layers stream better through kinds 4 and 1 once M > 1.
  if (ov.kind < 0 && gemv_ok && M > 1 && (p.Kp >= 8192 || N >= 16384)) gemv_ok = false;
  // With a rotation, every workgroup of the fused kernel also rotates the
  // whole activation; on the wide layers (>= 1024 column tiles, one per
  // workgroup) quantizing and rotating once, then the per-wave-ring GEMV, is
  // faster (Qwen3-32B gate_up at M = 1: 37-40 against 42-50 us for b = 32..128,
  // a tie at b = 16).
  if (ov.kind < 0 && gemv_ok && rotated && ntiles >= 1024) gemv_ok = false;
  if (gemv_ok && ov.kind <= 0) {
    // one workgroup per NTW 16-column tiles over the full K (no cross-workgroup reduction)
    p.kind = 0;
    p.mt = 1;
    p.nt = 1;
    p.wm = 1;
    p.Mp = M;
    p.waves = ntiles < 1024 ? 8 : 4;
    // Two column tiles per workgroup halve the workgroups that each quantize
    // (and, with a rotation, transform) the whole activation. Measured: a win
    // from M = 2 on, and at M = 1 with a rotation on the narrow layers
    // (Qwen3-32B down, 320 tiles: ~10%); at M = 1 without one they lose
    // (Llama-3.1-8B down 11.0 -> 14.7 us), and the wide layers (>= 1024
    // tiles, without a rotation: with one they leave the fused kernel) keep one.
    p.ntw = (M > 1 || rotated) && ntiles < 1024 ? 2 : 1;
    if (ov.waves == 4 || ov.waves == 8) p.waves = ov.waves;  // the built kind-0 widths
    if (ov.ntw == 1 || ov.ntw == 2) p.ntw = ov.ntw;
    const int64_t cpw = (KC + p.waves - 1) / p.waves;
    p.kcmax = cpw <= 8 ? 4 : 8;  // register ring depth (chunks)
    if (ov.rc) p.kcmax = ov.rc;
    const int64_t qblk = (M * p.Kp / 16 + 64 * p.waves - 1) / (64 * p.waves);  // blocks per thread
    p.qpre = qblk <= 1 ? 1 : qblk <= 2 ? 2 : 4;
    p.groups = (ntiles + p.ntw - 1) / p.ntw;
    p.splits = 1;
    p.kc_per_split = (int)KC;
    p.xhat_bytes = 0;
    p.lds_bytes = std::max<int64_t>(M * p.Kp * 2, (int64_t)p.waves * p.ntw * 1024);
  } else {
    // Workgroup tile (WM*MT*16) x ((4/WM)*NT*16) (kind 1) or (MT*32) x (4*NT*32) (kind 3).
    // Defaults (measured on the decode and prefill layer shapes): up to 32
    // rows the per-wave-ring kernel, except wide layers with short K (gate_up)
    // above 16 rows, which stream better through the register-staged tiled
    // kernel; from 33 rows on the LDS-ring kernel on 32x32 MFMAs.
    const bool wide_short = N >= 16384 && p.Kp < 8192;
    p.kind = M <= 32 ? (wide_short && M > 16 ? 1 : 4) : 3;
    if (ov.kind == 1 || ov.kind == 3 || ov.kind == 4) p.kind = ov.kind;
    if (p.kind == 4) {
      // per-wave rings: W waves split K, NT tiles per workgroup, D chunks in flight
      p.mt = (int)((M + 15) / 16);
      p.waves = p.Kp >= 8192 ? 8 : 4;
      p.nt = p.Kp >= 8192 ? 1 : 2;
      p.st = 3;
      if (M <= 16 && wide_short) p.nt = 4;
      if (ov.waves) p.waves = ov.waves;
      if (ov.nt) p.nt = ov.nt;
      if (ov.st) p.st = ov.st;
      // the quantizer pass (or the transform's) writes the activation packed like a weight
      if (p.mt <= 2 && gemv_ring_config_built(p.waves, p.mt, p.nt, p.st)) {
        p.wm = 1;
        p.Mp = 16 * p.mt;
        p.groups = (ntiles + p.nt - 1) / p.nt;
        p.ngroups = p.groups;
        p.splits = 1;
        p.kc_per_split = (int)KC;
        p.xhat_bytes = round_up(p.Mp * p.Kp * 2, 256);
        p.partial_bytes = 0;
        p.counter_bytes = kCounterBytes;
        p.total_bytes = p.counter_bytes + p.xhat_bytes;
        return p;
      }
      p.kind = 1;
    }
    // kind 3 addresses the packed blob with 32-bit per-lane offsets; the
    // tiled kernel's 64-bit addresses take weights of 4 GiB and more
    if (p.kind == 3 && d.total_bytes() >= ((int64_t)1 << 32)) p.kind = 1;
    const bool lds_ring = p.kind == 3;
    p.wm = 1;  // kind 1's wave grid; kind 3 has one row of 4 or 8 column waves
    p.cw = 4;
    p.st = 3;
    if (!lds_ring) {
      if (M <= 16) { p.mt = 1; p.nt = 1; }
      else if (M <= 32) { p.mt = 2; p.nt = 1; }
      else if (M <= 64) { p.mt = 2; p.nt = 2; p.wm = 2; }
      else if (M <= 128) { p.mt = 4; p.nt = 2; p.wm = 2; }
      else { p.mt = 8; p.nt = 4; }
    } else {  // kind 3, 32x32 tiles: MT x 32 rows, 4 x NT x 32 columns
      if (M <= 128) {
        // 64 x 256 tiles on 8 column waves (two per SIMD) when they alone
        // fill the GPU (gate_up at M = 128: 41.7 against 44.3 us for 128 x 128
        // tiles on 4 waves); else 128 x 128 tiles when those fill it, else
        // 64 x 128 tiles with a deeper ring and split K
        p.mt = 4; p.nt = 1; p.st = 3;
        if ((M + 63) / 64 * ((ntiles + 15) / 16) >= 192) {
          p.mt = 2; p.st = 4; p.cw = 8;
        } else if ((M + 127) / 128 * ((ntiles + 7) / 8) < 192) {
          p.mt = 2; p.st = 4;
        }
      } else {
        // 128 x 256 tiles on 8 waves, two per SIMD (measured 3-8% faster than
        // one wave per SIMD with 128-row waves on the prefill shapes), each
        // wave 128 x 32 so that a weight fragment feeds 4 MFMAs (about 1%
        // faster again than 64 x 64 waves)
        p.mt = 4; p.nt = 1; p.st = 3; p.cw = 8;
      }
    }
    if (ov.mt || ov.nt || ov.wm || ov.st || ov.cw) {
      if (ov.mt) p.mt = ov.mt;
      if (ov.nt) p.nt = ov.nt;
      if (ov.wm && !lds_ring) p.wm = ov.wm;
      if (ov.st) p.st = ov.st;
      if (lds_ring && ov.cw) p.cw = ov.cw;
    }
    const bool built = p.kind == 3 ? lds32_config_built(p.mt, p.nt, p.st, p.cw)
                                   : tiled_config_built(p.mt, p.nt, p.wm);
    if (!built) { p.kind = 1; p.mt = 1; p.nt = 1; p.wm = 1; p.cw = 4; }
    // rows and 16-column tiles per workgroup
    const int tile_rows = p.kind == 3 ? 32 * p.mt : 16 * p.mt * p.wm;
    const int tile_cols16 = p.kind == 3 ? 2 * p.cw * p.nt : (4 / p.wm) * p.nt;
    p.Mp = round_up(M, tile_rows);
    const int64_t ngroups = (ntiles + tile_cols16 - 1) / tile_cols16;
    const int64_t mgroups = p.Mp / tile_rows;
    const int64_t groups = ngroups * mgroups;
    // Split K across workgroups only when there are too few output tiles to
    // occupy the GPU: the arrival counter of the split-K reduction costs
    // about a microsecond plus ~0.35 us per split contending on it. Up to 4
    // splits, or 6 for long K (at least 144 chunks: Qwen3-32B down at M = 256,
    // 40 tiles, took 91 us with 6 splits against 101 us with 4).
    int64_t s = 1;
    const int64_t max_splits = KC >= 144 ? 6 : 4;
    if (groups < 192) s = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(max_splits, KC), 256 / groups));
    if (ov.splits) s = std::min<int64_t>(ov.splits, KC);
    p.kc_per_split = (int)((KC + s - 1) / s);
    p.splits = (int)((KC + p.kc_per_split - 1) / p.kc_per_split);
    p.groups = groups;
    p.ngroups = ngroups;
    // kind 3 without a K split: tiles in bands of 4 row groups per XCD
    // (measured 1-2% faster on the prefill and Qwen3-32B M = 4096 shapes
    // than the row-major order; bands of 1, 2 and 8 were in between)
    p.xg = 0;
    if (p.kind == 3 && p.splits == 1 && groups < ((int64_t)1 << 31)) {
      p.xg = ov.xg >= 0 ? ov.xg : 4;
      if (p.xg > mgroups) p.xg = (int)mgroups;
    }
    // Whole tiles use one workgroup each. When the tiles leave the last round
    // of the GPU's 256 workgroup slots (one per CU) at most half full and K
    // is long, the tiles of that round are split along K instead (up to 4
    // ways, through the split-K partial sums), so that round takes a fraction
    // of a tile's time. Measured: Qwen3-32B down at M = 4096 (640 tiles, 2.5
    // rounds, 200 chunks of K) 940 -> 875 us; with 32 chunks the saving is
    // gone (prefill qkv at M = 2048: 111 us either way), as the half-empty
    // round already runs at a higher clock and the partial sums cost a few
    // microseconds per tile.
    p.dp_groups = p.splits > 1 ? 0 : groups;
    if (p.kind == 3 && p.splits == 1 && ov.tail != 1 && groups >= kCUs) {
      const int64_t r = groups % kCUs;
      int64_t ts = r > 0 && r <= kCUs / 2 && KC >= 64 ? std::min<int64_t>(4, kCUs / r) : 1;
      if (ov.tail >= 2 && r > 0) ts = ov.tail;
      if (ts > 1 && KC >= 4 * ts && r <= (kCounterBytes - kWorkspaceScalarBytes) / 4) {
        p.dp_groups = groups - r;
        p.splits = (int)ts;
        p.kc_per_split = (int)((KC + ts - 1) / ts);
        p.splits = (int)((KC + p.kc_per_split - 1) / p.kc_per_split);
      }
    }
    p.xhat_bytes = round_up(p.Mp * p.Kp * 2, 256);
  }
  // [splits][waves][fragments][64 lanes] float4 per output tile
  const int64_t frags = (int64_t)p.mt * p.nt * (p.kind == 3 ? 4 : 1);
  const int64_t slab = (int64_t)p.splits * (p.kind == 3 ? p.cw : 4) * frags * 64 * 16;
  p.partial_bytes = p.splits > 1 ? round_up((p.groups - p.dp_groups) * slab, 256) : 0;
  p.counter_bytes = kCounterBytes;
  p.total_bytes = p.counter_bytes + p.xhat_bytes + p.partial_bytes;
  return p;
}

std::string describe_plan(const GemmPlan& p) {
  char b[256];
  if (p.kind == 4) {
    std::snprintf(b, sizeof(b), "quant_nvfp4_apack_kernel + gemv_ring_kernel<W=%d,MT=%d,NT=%d,D=%d> grid=%lld splits=1",
                  p.waves, p.mt, p.nt, p.st, (long long)p.groups);
  } else if (p.kind == 3) {
    // whole tiles first; a split tail reads "tail=<tiles>x<splits>"
    const bool tail = p.dp_groups > 0 && p.splits > 1;
    std::string extra = p.xg > 0 ? " xcd_bands=" + std::to_string(p.xg) : "";
    if (tail) extra += " tail=" + std::to_string(p.groups - p.dp_groups) + "x" + std::to_string(p.splits);
    const std::string wn = p.cw != 4 ? ",WN=" + std::to_string(p.cw) : "";
    std::snprintf(b, sizeof(b),
                  "quant_nvfp4_xhat_kernel + gemm_lds32_kernel<MT=%d,NT=%d,ST=%d%s> grid=%lld splits=%d%s",
                  p.mt, p.nt, p.st, wn.c_str(), (long long)(p.dp_groups + (p.groups - p.dp_groups) * p.splits),
                  tail ? 1 : p.splits, extra.c_str());
  } else if (p.kind == 0) {
    std::snprintf(b, sizeof(b), "linear_gemv_kernel<W=%d,NTW=%d,RC=%d,QPRE=%d> grid=%lld lds=%lld",
                  p.waves, p.ntw, p.kcmax, p.qpre, (long long)p.groups, (long long)p.lds_bytes);
  } else {
    std::snprintf(b, sizeof(b),
                  "quant_nvfp4_xhat_kernel + gemm_tiled_kernel<MT=%d,NT=%d,WM=%d> grid=%lld splits=%d",
                  p.mt, p.nt, p.wm, (long long)(p.groups * p.splits), p.splits);
  }
  return std::string(b);
}

// Arguments of one fused small-M launch (kind 0).
struct GemvLaunch {
  const GemmPlan* p;
  const uint16_t* x;
  int64_t M, K, ldx;
  float g;
  bool aligned;
  const uint8_t* packed;
  int64_t N;
  float alpha;
  const float* g_dev;
  const float* alpha_dev;
  const uint16_t* bias;
  uint16_t* y;
  int64_t ldy;
  hipStream_t st;
};

template <int W, int NTW, int HB, int RC, int QPRE>
static void launch_gemv_t(const GemvLaunch& a) {
  const GemmPlan& p = *a.p;
  const uint8_t* wcodes = a.packed;
  const uint8_t* wscales = a.packed + p.Np * p.Kp / 2;
  linear_gemv_kernel<W, NTW, HB, RC, QPRE><<<(unsigned)p.groups, 64 * W, (size_t)p.lds_bytes, a.st>>>(
      a.x, (int)a.M, (int)a.K, a.ldx, a.g, a.g_dev, a.aligned ? 1 : 0, wcodes, wscales, (int)a.N,
      p.Kp, (int)(p.Np / 16), a.alpha, a.alpha_dev, a.bias, a.y, a.ldy);
}

template <int W, int NTW, int HB>
static void launch_gemv_q(const GemvLaunch& a) {
  const GemmPlan& p = *a.p;
  if (p.kcmax == 4) {
    if (p.qpre == 1) launch_gemv_t<W, NTW, HB, 4, 1>(a);
    else if (p.qpre == 2) launch_gemv_t<W, NTW, HB, 4, 2>(a);
    else launch_gemv_t<W, NTW, HB, 4, 4>(a);
  } else {
    if (p.qpre == 1) launch_gemv_t<W, NTW, HB, 8, 1>(a);
    else if (p.qpre == 2) launch_gemv_t<W, NTW, HB, 8, 2>(a);
    else launch_gemv_t<W, NTW, HB, 8, 4>(a);
  }
}

// The built kind-0 shapes: 4 or 8 waves, one or two 16-column tiles per workgroup.
static bool gemv_shape_built(int waves, int ntw) {
  return (waves == 4 || waves == 8) && (ntw == 1 || ntw == 2);
}

template <int HB>
static void launch_gemv_hb(const GemvLaunch& a) {
  const GemmPlan& p = *a.p;
  if (p.waves == 8) {
    if (p.ntw == 1) launch_gemv_q<8, 1, HB>(a);
    else launch_gemv_q<8, 2, HB>(a);
  } else {
    if (p.ntw == 1) launch_gemv_q<4, 1, HB>(a);
    else launch_gemv_q<4, 2, HB>(a);
  }
}

template <int MT, int NT, int WM>
static hipError_t launch_tiled_t(const GemmPlan& p, const _Float16* xhat, const uint8_t* packed,
                                 int64_t M, int64_t N, float alpha, const float* alpha_dev,
                                 const uint16_t* bias,
                                 uint16_t* y, int64_t ldy, float4v* partial, uint32_t* counters,
                                 hipStream_t st) {
  const uint8_t* wcodes = packed;
  const uint8_t* wscales = packed + p.Np * p.Kp / 2;
  gemm_tiled_kernel<MT, NT, WM><<<(unsigned)(p.groups * p.splits), 256, 0, st>>>(
      xhat, wcodes, wscales, (int)M, (int)N, p.Kp, (int)(p.Np / 16), (int)p.ngroups,
      p.kc_per_split, p.splits, alpha, alpha_dev, bias, y, ldy, partial, counters);
  return hipGetLastError();
}

// The (MT, NT, WM) tiled configurations built into the library.
// (the planner's choices: M <= 16, <= 32, <= 64, <= 128 and larger, the last
// for weights of 4 GiB or more, whose offsets exceed the 32-bit ring kernel's)
#define FQL_TILED_CONFIGS(X) X(1, 1, 1) X(2, 1, 1) X(2, 2, 2) X(4, 2, 2) X(8, 4, 1)

template <int MT, int NT, int ST, int OCC, int WN>
static hipError_t launch_lds32_t(const GemmPlan& p, const _Float16* xhat, const uint8_t* packed,
                                 int64_t M, int64_t N, float alpha, const float* alpha_dev,
                                 const uint16_t* bias,
                                 uint16_t* y, int64_t ldy, float4v* partial, uint32_t* counters,
                                 hipStream_t st) {
  const uint8_t* wcodes = packed;
  const uint8_t* wscales = packed + p.Np * p.Kp / 2;
  const int64_t grid = p.dp_groups + (p.groups - p.dp_groups) * p.splits;
  gemm_lds32_kernel<MT, NT, ST, OCC, WN><<<(unsigned)grid, 64 * WN, 0, st>>>(
      xhat, wcodes, wscales, (int)M, (int)N, p.Kp, (int)(p.Np / 16), (int)p.ngroups,
      p.kc_per_split, (int)p.dp_groups, p.splits, p.xg, alpha, alpha_dev, bias, y, ldy, partial,
      counters);
  return hipGetLastError();
}

// The (MT, NT, ST, OCC, WN) 32x32 LDS-ring configurations built into the
// library, the planner's choices: 128 x 128 tiles (4 waves), 64 x 128 tiles
// with a 4-deep ring (split K at M <= 128), 128 x 256 and 64 x 256 tiles on 8
// column waves.
#define FQL_LDS32_CONFIGS(X) X(4, 1, 3, 1, 4) X(2, 1, 4, 2, 4) X(4, 1, 3, 1, 8) X(2, 1, 4, 1, 8)

bool lds32_config_built(int mt, int nt, int st, int cw) {
#define FQL_X(A, B, C, D, F) if (mt == A && nt == B && st == C && cw == F) return true;
  FQL_LDS32_CONFIGS(FQL_X)
#undef FQL_X
  return false;
}

// The (W, MT, NT, D) per-wave-ring configurations built into the library
// (the planner's choices: 4 waves with 2 tiles, wide short-K layers 4 tiles,
// long K 8 waves with one tile, each for one or two row tiles).
#define FQL_GEMV_RING_CONFIGS(X) X(4, 1, 2, 3) X(4, 1, 4, 3) X(8, 1, 1, 3) X(4, 2, 2, 3) X(8, 2, 1, 3)

bool gemv_ring_config_built(int w, int mt, int nt, int d) {
#define FQL_X(A, B, C, E) if (w == A && mt == B && nt == C && d == E) return true;
  FQL_GEMV_RING_CONFIGS(FQL_X)
#undef FQL_X
  return false;
}

bool tiled_config_built(int mt, int nt, int wm) {
#define FQL_X(A, B, C) if (mt == A && nt == B && wm == C) return true;
  FQL_TILED_CONFIGS(FQL_X)
#undef FQL_X
  return false;
}

// Workspace regions of a plan: [arrival counters | activation operand | split-K slabs].
static uint32_t* ws_counters(uint8_t* ws) { return reinterpret_cast<uint32_t*>(ws); }
static uint8_t* ws_operand(const GemmPlan& p, uint8_t* ws) { return ws + p.counter_bytes; }
static float4v* ws_partial(const GemmPlan& p, uint8_t* ws) {
  return reinterpret_cast<float4v*>(ws + p.counter_bytes + p.xhat_bytes);
}

bool has_quant_pass(const GemmPlan& p) { return p.kind != 0; }

hipError_t launch_linear_quant(const GemmPlan& p, const uint16_t* x, int64_t M, int64_t K,
                               int64_t ldx, float g, int hb, bool aligned, uint8_t* workspace,
                               hipStream_t st, const LinearExtras* ex) {
  if (!has_quant_pass(p)) return hipErrorInvalidValue;
  const bool transform = ex != nullptr && ex->T != nullptr;
  const float* g_dev = ex != nullptr ? ex->g_dev : nullptr;
  uint8_t* operand = ws_operand(p, workspace);
  // the packed activation (kind 4) or x_hat, from the plain quantizer or the transform's
  const bool packed_a = p.kind == 4;
  if (packed_a && p.Mp != 16 * p.mt) return hipErrorInvalidValue;
  if (transform) {
    TransformArgs ta{};
    ta.mode = packed_a ? 4 : 1;
    ta.x = x; ta.M = M; ta.K = K; ta.ldx = ldx; ta.aligned = ex->t_aligned;
    ta.T = ex->T; ta.b = hb; ta.g = g; ta.g_dev = g_dev;
    ta.xhat = reinterpret_cast<_Float16*>(operand); ta.rows_out = p.Mp; ta.Kp = p.Kp;
    return launch_transform_nvfp4(ta, st);
  }
  if (packed_a)
    return launch_quant_nvfp4_apack(x, M, K, ldx, g, hb, aligned, p.Mp, p.Kp, operand, g_dev, st);
  return launch_quant_nvfp4_xhat(x, M, K, ldx, g, hb, aligned, p.Mp, p.Kp,
                                 reinterpret_cast<_Float16*>(operand), g_dev, st);
}

// The GEMM of kinds 1, 3 and 4 on the operand in the workspace.
static hipError_t launch_gemm_part(const GemmPlan& p, const uint8_t* packed, int64_t M, int64_t N,
                                   float alpha, const uint16_t* bias, uint16_t* y, int64_t ldy,
                                   uint8_t* workspace, hipStream_t st, const LinearExtras* ex) {
  const float* alpha_dev = ex != nullptr ? ex->alpha_dev : nullptr;
  uint32_t* counters = ws_counters(workspace);
  _Float16* xhat = reinterpret_cast<_Float16*>(ws_operand(p, workspace));
  float4v* partial4 = ws_partial(p, workspace);
  // one arrival counter per split tile
  if (p.splits > 1 && p.groups - (p.kind == 3 ? p.dp_groups : 0) > (p.counter_bytes - kWorkspaceScalarBytes) / 4)
    return hipErrorInvalidValue;
  if (p.kind == 4) {
#define FQL_X(A, B, C, E)                                                                             \
  if (p.waves == A && p.mt == B && p.nt == C && p.st == E) {                                          \
    gemv_ring_kernel<A, B, C, E><<<(unsigned)p.groups, 64 * A, 0, st>>>(                              \
        ws_operand(p, workspace), packed, packed + p.Np * p.Kp / 2, (int)M, (int)N, p.Kp,              \
        (int)(p.Np / 16), alpha, alpha_dev, bias, y, ldy);                                             \
    return hipGetLastError();                                                                          \
  }
    FQL_GEMV_RING_CONFIGS(FQL_X)
#undef FQL_X
    return hipErrorInvalidValue;
  }
  if (p.kind == 3) {
#define FQL_X(A, B, C, D, F)                                                                     \
  if (p.mt == A && p.nt == B && p.st == C && p.cw == F)                                          \
    return launch_lds32_t<A, B, C, D, F>(p, xhat, packed, M, N, alpha, alpha_dev, bias, y, ldy, partial4, counters, st);
    FQL_LDS32_CONFIGS(FQL_X)
#undef FQL_X
    return hipErrorInvalidValue;
  }
  if (p.kind != 1) return hipErrorInvalidValue;
#define FQL_X(A, B, C)                                                                           \
  if (p.mt == A && p.nt == B && p.wm == C)                                                       \
    return launch_tiled_t<A, B, C>(p, xhat, packed, M, N, alpha, alpha_dev, bias, y, ldy, partial4, counters, st);
  FQL_TILED_CONFIGS(FQL_X)
#undef FQL_X
  return hipErrorInvalidValue;
}

hipError_t launch_linear_gemm(const GemmPlan& p, const uint8_t* packed, int64_t M, int64_t N,
                              float alpha, const uint16_t* bias, uint16_t* y, int64_t ldy,
                              uint8_t* workspace, hipStream_t st, const LinearExtras* ex) {
  if (p.kind == 0) return hipErrorInvalidValue;  // no separate operand
  return launch_gemm_part(p, packed, M, N, alpha, bias, y, ldy, workspace, st, ex);
}

hipError_t launch_linear_nvfp4(const GemmPlan& p, const uint16_t* x, int64_t M, int64_t K,
                               int64_t ldx, float g, int hb, bool aligned, const uint8_t* packed,
                               int64_t N, float alpha, const uint16_t* bias, uint16_t* y,
                               int64_t ldy, uint8_t* workspace, hipStream_t st,
                               const LinearExtras* ex) {
  if (p.kind == 0) {
    // the fused path reads x rows with 16-byte loads and cannot apply a general transform
    if (!aligned || (ex != nullptr && ex->T != nullptr)) return hipErrorInvalidValue;
    if (!gemv_shape_built(p.waves, p.ntw)) return hipErrorInvalidValue;
    const GemvLaunch a{&p, x, M, K, ldx, g, aligned, packed, N, alpha,
                       ex != nullptr ? ex->g_dev : nullptr, ex != nullptr ? ex->alpha_dev : nullptr,
                       bias, y, ldy, st};
    switch (hb) {
      case 0: launch_gemv_hb<0>(a); break;
      case 16: launch_gemv_hb<16>(a); break;
      case 32: launch_gemv_hb<32>(a); break;
      case 64: launch_gemv_hb<64>(a); break;
      case 128: launch_gemv_hb<128>(a); break;
      default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
  }
  const hipError_t e = launch_linear_quant(p, x, M, K, ldx, g, hb, aligned, workspace, st, ex);
  if (e != hipSuccess) return e;
  return launch_gemm_part(p, packed, M, N, alpha, bias, y, ldy, workspace, st, ex);
}

}  // namespace fql
