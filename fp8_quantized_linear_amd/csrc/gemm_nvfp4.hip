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
//  * linear_small_kernel (M <= 32): ONE launch per layer call. Each
//    workgroup quantizes the activation rows for its K range straight into
//    LDS (the quantizer's arithmetic, fql_quant.h), issues all of its weight
//    loads up front (one HBM round trip), and reduces split-K partials
//    itself: the last workgroup of a column group to arrive sums the float32
//    partials in split order (deterministic) and applies the epilogue.
//  * gemm_tiled_kernel (M > 32): x_hat comes pre-quantized from the
//    quantizer kernel; A chunks are double-buffered through LDS and B is
//    prefetched one chunk ahead; split-K (if any) uses the same last-arriver
//    reduction.
#include <algorithm>
#include <cmath>

#include "fql_device.h"
#include "fql_internal.h"
#include "fql_quant.h"

namespace fql {

// ---------------------------------------------------------------------------
// shared pieces
// ---------------------------------------------------------------------------

// B fragments for one 32-deep K step of one 16-column tile.
__device__ __forceinline__ half8 b_fragment(uint32_t codes, uint32_t scale_byte) {
  const _Float16 sh = e4m3_to_f16(scale_byte);
  const half2v s2 = {sh, sh};
  uint32_t hw[4];
  dequant8_f16(codes, s2, hw);
  return __builtin_bit_cast(half8, uint4v{hw[0], hw[1], hw[2], hw[3]});
}

__device__ __forceinline__ uint32_t dword_of(const uint4v& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Write the workgroup's output tile: directly (one split) or through the
// split-K slab and the last-arriver reduction.
//   rows: MT*16 rows starting at m0; cols: 64*NT columns starting at n0.
//   slab: [splits][MT*16][64*NT] float32 for this workgroup's tile.
template <int MT, int NT>
__device__ __forceinline__ void finish_tile(float4v (&acc)[MT][NT], int M, int N, int m0, int n0,
                                            int split, int splits, float alpha,
                                            const uint16_t* __restrict__ bias,
                                            uint16_t* __restrict__ y, int64_t ldy,
                                            float* __restrict__ slab, uint32_t* counter,
                                            uint32_t* s_flag) {
  constexpr int WGC = 64 * NT;
  constexpr int ROWS = MT * 16;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, row0 = 4 * (lane >> 4);
  if (splits == 1) {
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const int n = n0 + (wave * NT + nt) * 16 + col;
      if (n >= N) continue;
      const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int m = m0 + mt * 16 + row0 + i;
          if (m < M) y[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16_bits(alpha * acc[mt][nt][i] + bv);
        }
      }
    }
    return;
  }
  // Split-K: publish this split's float32 partial tile, count arrivals, and
  // let the last workgroup to arrive sum the splits in order. The partials
  // are written and read with agent-scope relaxed atomics, which on gfx950
  // write through / read past the per-XCD L2s to the device coherence point;
  // waiting for the stores to complete before the arrival increment orders
  // them without any whole-cache write-back or invalidate.
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = (wave * NT + nt) * 16 + col;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = mt * 16 + row0 + i;
        if (m0 + r < M)
          __hip_atomic_store(slab + ((int64_t)split * ROWS + r) * WGC + c, acc[mt][nt][i],
                             __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const uint32_t arrived =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = arrived == (uint32_t)(splits - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (*s_flag == 0u) return;
  // Sum in split order. Loads are issued in unconditional batches of 8 (a
  // clamped split index) so they overlap instead of costing one memory
  // round trip each.
  const int rows = min(ROWS, M - m0);
  for (int e = tid; e < rows * WGC; e += 256) {
    const int r = e / WGC, c = e - r * WGC;
    const int n = n0 + c;
    const float* base = slab + (int64_t)r * WGC + c;
    float s = 0.0f;
    for (int z0 = 0; z0 < splits; z0 += 8) {
      float v[8];
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int z = z0 + j < splits ? z0 + j : splits - 1;
        v[j] = __hip_atomic_load(base + (int64_t)z * ROWS * WGC, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int j = 0; j < 8; ++j)
        if (z0 + j < splits) s += v[j];
    }
    if (n < N) {
      const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
      y[(int64_t)(m0 + r) * ldy + n] = (uint16_t)f32_to_bf16_bits(alpha * s + bv);
    }
  }
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// small-M fused kernel
// ---------------------------------------------------------------------------

template <int MT, int NT, int HB, int KCMAX>
__global__ __launch_bounds__(256) void linear_small_kernel(
    const uint16_t* __restrict__ x, int M, int K, int64_t ldx, float g, int aligned16,
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales, int N, int64_t Kp,
    int ntiles, int kc_per_split, int splits, float alpha, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int64_t ldy, float* __restrict__ partial,
    uint32_t* __restrict__ counters) {
  // KCMAX: chunks per split this instantiation holds (A in LDS = MT*KCMAX*4 KB,
  // weight registers = 5*KCMAX per tile); the plan picks the smallest that fits
  constexpr int WGC = 64 * NT;
  __shared__ uint4v a_lds[MT][KCMAX * 4][64];
  __shared__ uint32_t s_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t KC = Kp / 128;
  const int group = blockIdx.x / splits;
  const int split = blockIdx.x - group * splits;
  const int64_t c0 = (int64_t)split * kc_per_split;
  const int nck = (int)(KC - c0 < kc_per_split ? KC - c0 : kc_per_split);
  const int tile0 = (group * 4 + wave) * NT;

  // 1. all weight loads of this workgroup's K range, issued first
  uint4v bq[NT][KCMAX];
  uint32_t bs[NT][KCMAX];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const bool tv = (tile0 + nt) < ntiles;
    const int64_t t = tv ? tile0 + nt : 0;
    const uint4v* qp = reinterpret_cast<const uint4v*>(wcodes) + (t * KC + c0) * 64 + lane;
    const uint32_t* sp = reinterpret_cast<const uint32_t*>(wscales) + (t * KC + c0) * 32 +
                         (lane & 15) * 2 + (lane >> 5);
    // unconditional loads (chunks past the range re-read the last one, a cache
    // hit) keep the outstanding-load count static, so each chunk's compute
    // waits only for its own data
#pragma unroll
    for (int c = 0; c < KCMAX; ++c) {
      const int cc = c < nck ? c : nck - 1;
      bq[nt][c] = qp[cc * 64];
      bs[nt][c] = sp[cc * 32];
    }
  }

  // 2. quantize x[0:M, c0*128 : (c0+nck)*128] into LDS A fragments
  //    slot (mt, ks, lane') holds x_hat[mt*16 + lane'%16][k = 32 ks + 8 (lane'/16) + 0..7]
  {
    // zero the fragment rows >= M
    const int nslots = MT * nck * 4 * 64;
    for (int s = tid; s < nslots; s += 256) {
      const int l2 = s & 63, ks = (s >> 6) % (nck * 4), mt = (s >> 6) / (nck * 4);
      if (mt * 16 + (l2 & 15) >= M) a_lds[mt][ks][l2] = uint4v{0u, 0u, 0u, 0u};
    }
    const int nblk = nck * 8;  // 16-blocks per row in range
    const int total = M * nblk;
    const uint16_t* xk = x + c0 * 128;
    for (int b0 = 0; b0 < total; b0 += 256) {
      const int b = b0 + tid;
      const bool act = b < total;
      const int m = act ? b / nblk : 0;
      const int kb = act ? b - m * nblk : 0;
      float v[16];
      if (act && (c0 * 128 + kb * 16) < K) {
        Loader<uint16_t>::load16(xk + (int64_t)m * ldx + kb * 16, aligned16 != 0, v);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = 0.0f;
      }
      if constexpr (HB > 0) fwht_block<HB>(v, kb);
      if (act) {
        uint32_t lo, hi, s;
        quant_block(v, g, lo, hi, s);
        const _Float16 sh = e4m3_to_f16(s);
        const half2v s2 = {sh, sh};
        uint32_t hw[8];
        dequant8_f16(lo, s2, hw);
        dequant8_f16(hi, s2, hw + 4);
        const int ks = kb >> 1, kq0 = (kb & 1) * 2, ml = m & 15, mt = m >> 4;
        a_lds[mt][ks][kq0 * 16 + ml] = uint4v{hw[0], hw[1], hw[2], hw[3]};
        a_lds[mt][ks][(kq0 + 1) * 16 + ml] = uint4v{hw[4], hw[5], hw[6], hw[7]};
      }
    }
  }
  __syncthreads();

  // 3. MFMA over the K range
  float4v acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < KCMAX; ++c) {
    if (c < nck) {
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        half8 bf[NT];
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          bf[nt] = b_fragment(dword_of(bq[nt][c], ks), (bs[nt][c] >> (8 * ks)) & 0xFFu);
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
          const half8 a = __builtin_bit_cast(half8, a_lds[mt][c * 4 + ks][lane]);
#pragma unroll
          for (int nt = 0; nt < NT; ++nt)
            acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[nt], acc[mt][nt], 0, 0, 0);
        }
      }
    }
  }

  // 4. output (direct, or split-K partials + last-arriver reduction)
  float* slab = partial + (int64_t)group * splits * (MT * 16) * WGC;
  finish_tile<MT, NT>(acc, M, N, 0, group * WGC, split, splits, alpha, bias, y, ldy, slab,
                      counters + group, &s_flag);
}

// ---------------------------------------------------------------------------
// tiled kernel (x_hat from the quantizer kernel)
// ---------------------------------------------------------------------------

template <int MT, int NT>
__global__ __launch_bounds__(256) void gemm_tiled_kernel(
    const _Float16* __restrict__ xhat, const uint8_t* __restrict__ wcodes,
    const uint8_t* __restrict__ wscales, int M, int N, int64_t Kp, int ntiles, int ngroups,
    int kc_per_split, int splits, float alpha, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int64_t ldy, float* __restrict__ partial,
    uint32_t* __restrict__ counters) {
  constexpr int WGC = 64 * NT;
  __shared__ uint4v a_lds[2][MT * 4][64];
  __shared__ uint32_t s_flag;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t KC = Kp / 128;
  const int64_t KS = Kp / 32;
  // blockIdx.x = (mgroup * ngroups + ngroup) * splits + split
  const int split = blockIdx.x % splits;
  const int tilegrp = blockIdx.x / splits;
  const int ngroup = tilegrp % ngroups;
  const int mgroup = tilegrp / ngroups;
  const int64_t c_begin = (int64_t)split * kc_per_split;
  const int64_t c_end = c_begin + kc_per_split < KC ? c_begin + kc_per_split : KC;
  const int tile0 = (ngroup * 4 + wave) * NT;

  bool tvalid[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) tvalid[nt] = (tile0 + nt) < ntiles;

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
                  (lane >> 5);
  }

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
  uint4v ar0[MT], ar1[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) a_lds[0][mt * 4 + (tid >> 6)][tid & 63] = *a_src(mt, c_begin);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) ar1[mt] = *a_src(mt, clampc(c_begin + 1));
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {  // invalid tiles read tile 0 (in bounds, never stored)
    bq0[nt] = bq_base[nt][c_begin * 64];
    bs0[nt] = bs_base[nt][c_begin * 32];
    bq1[nt] = bq_base[nt][clampc(c_begin + 1) * 64];
    bs1[nt] = bs_base[nt][clampc(c_begin + 1) * 32];
  }
  __syncthreads();

  auto compute = [&](int buf, const uint4v (&bq)[NT], const uint32_t (&bs)[NT]) {
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      half8 bf[NT];
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) bf[nt] = b_fragment(dword_of(bq[nt], ks), (bs[nt] >> (8 * ks)) & 0xFFu);
#pragma unroll
      for (int mt = 0; mt < MT; ++mt) {
        const half8 a = __builtin_bit_cast(half8, a_lds[buf][mt * 4 + ks][lane]);
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
          acc[mt][nt] = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, bf[nt], acc[mt][nt], 0, 0, 0);
      }
    }
  };
  auto advance = [&](int buf, int64_t c, uint4v (&ar_store)[MT], uint4v (&ar_load)[MT],
                     uint4v (&bq)[NT], uint32_t (&bs)[NT]) {
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) a_lds[buf ^ 1][mt * 4 + (tid >> 6)][tid & 63] = ar_store[mt];
    const int64_t c2 = clampc(c + 2);
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) ar_load[mt] = *a_src(mt, c2);
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      bq[nt] = bq_base[nt][c2 * 64];
      bs[nt] = bs_base[nt][c2 * 32];
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

  float* slab = partial + (int64_t)tilegrp * splits * (MT * 16) * WGC;
  finish_tile<MT, NT>(acc, M, N, mgroup * MT * 16, ngroup * WGC, split, splits, alpha, bias, y,
                      ldy, slab, counters + tilegrp, &s_flag);
}

// ---------------------------------------------------------------------------
// planning and launch
// ---------------------------------------------------------------------------

static constexpr int kCUs = 256;
static constexpr int64_t kCounterBytes = 64 * 1024;  // arrival counters at the workspace start

// Pick a split count in [s_lo, s_hi]: the estimated cost is the bytes moved
// (weight, plus split-K partials written and read back, which mostly stay in
// the last-level cache and are weighted by one half) divided by how evenly
// and how fully the workgroups occupy the CUs.
static int pick_splits(int64_t groups, int64_t s_lo, int64_t s_hi, int64_t min_wgs,
                       double w_bytes, double partial_bytes_per_split) {
  if (s_lo < 1) s_lo = 1;
  if (s_hi < s_lo) s_hi = s_lo;
  int best = (int)s_lo;
  double best_cost = 1e300;
  for (int64_t s = s_lo; s <= s_hi; ++s) {
    const int64_t wgs = groups * s;
    const double waves = (double)wgs / kCUs;
    const double balance = waves / std::ceil(waves);
    const double fill = wgs >= min_wgs ? 1.0 : (double)wgs / (double)min_wgs;
    const double traffic = w_bytes + (s > 1 ? (double)s * partial_bytes_per_split : 0.0);
    const double cost = traffic / (balance * fill);
    if (cost < best_cost * (1.0 - 1e-6)) {
      best_cost = cost;
      best = (int)s;
    }
  }
  return best;
}

GemmPlan plan_gemm_nvfp4(int64_t M, int64_t N, int64_t K) {
  GemmPlan p{};
  const PackedDims d = packed_dims(N, K);
  p.Np = d.Np;
  p.Kp = d.Kp;
  const int64_t KC = p.Kp / 128;
  const int64_t ntiles = p.Np / 16;
  if (M <= 32) {
    p.kind = 0;
    p.mt = M <= 16 ? 1 : 2;
    p.nt = 1;
    p.Mp = 16 * p.mt;
    const int64_t kcmax = 16 / p.mt;  // LDS cap: MT * 16 chunks * 4 KB / MT = 64 KB
    const int64_t groups = (ntiles + 4 * p.nt - 1) / (4 * p.nt);
    const int64_t s_lo = (KC + kcmax - 1) / kcmax;
    const double wb = 0.5625 * (double)p.Np * (double)p.Kp;
    const double pb = 4.0 * (double)M * (double)p.Np;
    int64_t s = pick_splits(groups, s_lo, std::max<int64_t>(s_lo, std::min<int64_t>(KC, 4 * s_lo + 8)),
                            3 * kCUs, wb, pb);
    p.kc_per_split = (int)((KC + s - 1) / s);
    p.splits = (int)((KC + p.kc_per_split - 1) / p.kc_per_split);
    p.kcmax = p.kc_per_split <= 4 ? 4 : p.kc_per_split <= 8 ? 8 : 16;
    p.groups = groups;
    p.xhat_bytes = 0;
  } else {
    p.kind = 1;
    p.mt = M <= 64 ? 4 : 8;
    p.nt = M <= 128 ? 1 : 4;
    p.Mp = round_up(M, 16 * p.mt);
    const int64_t ngroups = (ntiles + 4 * p.nt - 1) / (4 * p.nt);
    const int64_t mgroups = p.Mp / (16 * p.mt);
    const int64_t groups = ngroups * mgroups;
    int64_t s = 1;
    const double wb = 0.5625 * (double)p.Np * (double)p.Kp * (double)mgroups;
    const double pb = 4.0 * (double)M * (double)p.Np;
    if (groups < 2 * kCUs) s = pick_splits(groups, 1, std::min<int64_t>(KC, 16), 3 * kCUs, wb, pb);
    p.kc_per_split = (int)((KC + s - 1) / s);
    p.splits = (int)((KC + p.kc_per_split - 1) / p.kc_per_split);
    p.groups = groups;
    p.ngroups = ngroups;
    p.xhat_bytes = round_up(p.Mp * p.Kp * 2, 256);
  }
  const int64_t slab = (int64_t)p.splits * (16 * p.mt) * (64 * p.nt) * 4;
  p.partial_bytes = p.splits > 1 ? round_up(p.groups * slab, 256) : 0;
  p.counter_bytes = kCounterBytes;
  p.total_bytes = p.counter_bytes + p.xhat_bytes + p.partial_bytes;
  return p;
}

template <int MT, int NT, int HB, int KCMAX>
static void launch_small_t(const GemmPlan& p, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                           float g, bool aligned, const uint8_t* packed, int64_t N, float alpha,
                           const uint16_t* bias, uint16_t* y, int64_t ldy, float* partial,
                           uint32_t* counters, hipStream_t st) {
  const uint8_t* wcodes = packed;
  const uint8_t* wscales = packed + p.Np * p.Kp / 2;
  linear_small_kernel<MT, NT, HB, KCMAX><<<(unsigned)(p.groups * p.splits), 256, 0, st>>>(
      x, (int)M, (int)K, ldx, g, aligned ? 1 : 0, wcodes, wscales, (int)N, p.Kp, (int)(p.Np / 16),
      p.kc_per_split, p.splits, alpha, bias, y, ldy, partial, counters);
}

template <int MT, int NT, int HB>
static void launch_small_k(const GemmPlan& p, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                           float g, bool aligned, const uint8_t* packed, int64_t N, float alpha,
                           const uint16_t* bias, uint16_t* y, int64_t ldy, float* partial,
                           uint32_t* counters, hipStream_t st) {
  if (p.kcmax == 4)
    launch_small_t<MT, NT, HB, 4>(p, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st);
  else if (p.kcmax == 8 || MT == 2)
    launch_small_t<MT, NT, HB, 8>(p, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st);
  else
    launch_small_t<MT, NT, HB, 16 / MT>(p, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st);
}

template <int MT, int NT>
static hipError_t launch_small_hb(const GemmPlan& p, int hb, const uint16_t* x, int64_t M,
                                  int64_t K, int64_t ldx, float g, bool aligned,
                                  const uint8_t* packed, int64_t N, float alpha,
                                  const uint16_t* bias, uint16_t* y, int64_t ldy, float* partial,
                                  uint32_t* counters, hipStream_t st) {
  switch (hb) {
    case 0: launch_small_k<MT, NT, 0>(p, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st); break;
    case 16: launch_small_k<MT, NT, 16>(p, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st); break;
    case 32: launch_small_k<MT, NT, 32>(p, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st); break;
    case 64: launch_small_k<MT, NT, 64>(p, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st); break;
    case 128: launch_small_k<MT, NT, 128>(p, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int MT, int NT>
static hipError_t launch_tiled_t(const GemmPlan& p, const _Float16* xhat, const uint8_t* packed,
                                 int64_t M, int64_t N, float alpha, const uint16_t* bias,
                                 uint16_t* y, int64_t ldy, float* partial, uint32_t* counters,
                                 hipStream_t st) {
  const uint8_t* wcodes = packed;
  const uint8_t* wscales = packed + p.Np * p.Kp / 2;
  gemm_tiled_kernel<MT, NT><<<(unsigned)(p.groups * p.splits), 256, 0, st>>>(
      xhat, wcodes, wscales, (int)M, (int)N, p.Kp, (int)(p.Np / 16), (int)p.ngroups,
      p.kc_per_split, p.splits, alpha, bias, y, ldy, partial, counters);
  return hipGetLastError();
}

hipError_t launch_linear_nvfp4(const GemmPlan& p, const uint16_t* x, int64_t M, int64_t K,
                               int64_t ldx, float g, int hb, bool aligned, const uint8_t* packed,
                               int64_t N, float alpha, const uint16_t* bias, uint16_t* y,
                               int64_t ldy, uint8_t* workspace, hipStream_t st) {
  uint32_t* counters = reinterpret_cast<uint32_t*>(workspace);
  _Float16* xhat = reinterpret_cast<_Float16*>(workspace + p.counter_bytes);
  float* partial = reinterpret_cast<float*>(workspace + p.counter_bytes + p.xhat_bytes);
  if (p.groups > p.counter_bytes / 4) return hipErrorInvalidValue;
  if (p.kind == 0) {
    if (p.mt == 1) return launch_small_hb<1, 1>(p, hb, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st);
    if (p.mt == 2) return launch_small_hb<2, 1>(p, hb, x, M, K, ldx, g, aligned, packed, N, alpha, bias, y, ldy, partial, counters, st);
    return hipErrorInvalidValue;
  }
  hipError_t e = launch_quant_nvfp4_xhat(x, M, K, ldx, g, hb, aligned, p.Mp, p.Kp, xhat, st);
  if (e != hipSuccess) return e;
  if (p.mt == 4 && p.nt == 1) return launch_tiled_t<4, 1>(p, xhat, packed, M, N, alpha, bias, y, ldy, partial, counters, st);
  if (p.mt == 8 && p.nt == 1) return launch_tiled_t<8, 1>(p, xhat, packed, M, N, alpha, bias, y, ldy, partial, counters, st);
  if (p.mt == 4 && p.nt == 4) return launch_tiled_t<4, 4>(p, xhat, packed, M, N, alpha, bias, y, ldy, partial, counters, st);
  if (p.mt == 8 && p.nt == 4) return launch_tiled_t<8, 4>(p, xhat, packed, M, N, alpha, bias, y, ldy, partial, counters, st);
  return hipErrorInvalidValue;
}

}  // namespace fql
