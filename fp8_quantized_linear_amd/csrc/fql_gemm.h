// Pieces shared by the GEMM kernels: weight-fragment dequantization, direct
// global->LDS loads with explicit completion waits, the workgroup barrier
// used by the LDS rings, and the split-K epilogue.
#pragma once

#include "fql_device.h"
#include "fql_quant.h"

namespace fql {

// B fragment for one 32-deep K step of one 16-column tile: eight codes times
// their block scale (already float16).
__device__ __forceinline__ half8 b_fragment(uint32_t codes, _Float16 sh) {
  const half2v s2 = {sh, sh};
  uint32_t hw[4];
  dequant8_f16(codes, s2, hw);
  return __builtin_bit_cast(half8, uint4v{hw[0], hw[1], hw[2], hw[3]});
}

// The four K steps' scales of one chunk (one dword, byte j = step j) as float16.
struct ChunkScales {
  half2v lo, hi;
  __device__ __forceinline__ explicit ChunkScales(uint32_t w) { e4m3x4_to_f16(w, lo, hi); }
  __device__ __forceinline__ _Float16 operator[](int ks) const {
    return ks == 0 ? lo[0] : ks == 1 ? lo[1] : ks == 2 ? hi[0] : hi[1];
  }
};

__device__ __forceinline__ uint32_t dword_of(const uint4v& v, int i) {
  return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}

// Split-K partials are exchanged between workgroups that may sit on different
// XCDs (each with its own L2), so they are written and read with agent-scope
// relaxed atomics, which on gfx950 write through / read past the L2s to the
// device coherence point. Waiting for the stores to complete before the
// arrival increment orders them without any whole-cache write-back or
// invalidate. Each lane moves its accumulator fragment as two 8-byte words.
__device__ __forceinline__ void store_partial(float4v* frag, int lane, const float4v& v) {
  // A fragment's 64 float4 are stored as two 512-byte halves (words 0-1 of
  // every lane, then words 2-3), so each 8-byte store instruction writes whole
  // cache lines; interleaving the halves per lane would fill every other 8
  // bytes of the fragment and write each line to HBM twice.
  uint64_t* q = reinterpret_cast<uint64_t*>(frag);
  __hip_atomic_store(q + lane, __builtin_bit_cast(uint64_t, float2v{v[0], v[1]}), __ATOMIC_RELAXED,
                     __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(q + 64 + lane, __builtin_bit_cast(uint64_t, float2v{v[2], v[3]}),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float4v load_partial(const float4v* frag, int lane) {
  uint64_t* q = const_cast<uint64_t*>(reinterpret_cast<const uint64_t*>(frag));
  const float2v a = __builtin_bit_cast(float2v, __hip_atomic_load(q + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  const float2v b = __builtin_bit_cast(float2v, __hip_atomic_load(q + 64 + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
  return float4v{a[0], a[1], b[0], b[1]};
}

// Write the workgroup's output tile: directly (one split) or through the
// split-K slab and the last-arriver reduction. The lane's accumulators come
// as FR float4 fragments; fragment f element i is the output element at
// (m0 + row_of(f, i), n0 + col_of(f)).
//   slab: [splits][NW waves][FR][64 lanes] float4 for this workgroup's tile,
//   so every lane writes and later sums exactly its own fragments.
template <int FR, typename RowOf, typename ColOf, int NW = 4>
__device__ __forceinline__ void finish_frags(float4v (&frag)[FR], RowOf row_of, ColOf col_of, int M,
                                             int N, int m0, int n0, int split, int splits,
                                             float alpha, const uint16_t* __restrict__ bias,
                                             uint16_t* __restrict__ y, int64_t ldy,
                                             float4v* __restrict__ slab, uint32_t* counter,
                                             uint32_t* s_flag) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  auto emit = [&](int f, const float4v& s) {
    const int n = n0 + col_of(f);
    if (n >= N) return;
    const float bv = bias ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int m = m0 + row_of(f, i);
      if (m < M) y[(int64_t)m * ldy + n] = (uint16_t)f32_to_bf16_bits(alpha * s[i] + bv);
    }
  };
  if (splits == 1) {
#pragma unroll
    for (int f = 0; f < FR; ++f) emit(f, frag[f]);
    return;
  }
  float4v* mine = slab + wave * FR * 64;  // this wave's fragments (64 float4 each)
  const int64_t zstride = (int64_t)NW * FR * 64;
#pragma unroll
  for (int f = 0; f < FR; ++f) store_partial(mine + split * zstride + f * 64, lane, frag[f]);
  __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");  // partial stores have completed
  __syncthreads();
  if (tid == 0) {
    const uint32_t arrived =
        __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    *s_flag = arrived == (uint32_t)(splits - 1) ? 1u : 0u;
  }
  __syncthreads();
  if (*s_flag == 0u) return;
  // Sum in split order, FG fragments at a time. ZB splits' fragments are
  // loaded per round, all issued before any is used (clamped split index: a
  // static number of loads), so a round costs one memory round trip.
  constexpr int FG = FR < 8 ? FR : 8;
  constexpr int ZB = 16 / FG < 8 ? 16 / FG : 8;
#pragma unroll
  for (int f0 = 0; f0 < FR; f0 += FG) {
    float4v sum[FG];
#pragma unroll
    for (int f = 0; f < FG; ++f) sum[f] = float4v{0.f, 0.f, 0.f, 0.f};
    for (int z0 = 0; z0 < splits; z0 += ZB) {
      float4v v[ZB][FG];
#pragma unroll
      for (int j = 0; j < ZB; ++j) {
        const int z = z0 + j < splits ? z0 + j : splits - 1;
#pragma unroll
        for (int f = 0; f < FG; ++f) v[j][f] = load_partial(mine + z * zstride + (f0 + f) * 64, lane);
      }
#pragma unroll
      for (int j = 0; j < ZB; ++j)
        if (z0 + j < splits)
#pragma unroll
          for (int f = 0; f < FG; ++f) sum[f] += v[j][f];
    }
#pragma unroll
    for (int f = 0; f < FG; ++f) emit(f0 + f, sum[f]);
  }
  if (tid == 0) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// 16x16 accumulator tiles: the 4 waves form a WM x (4/WM) grid; wave (wm, wn)
// holds MT x NT tiles, rows m0 + (wm*MT + mt)*16 + 4*(lane/16) + i, columns
// n0 + (wn*NT + nt)*16 + lane%16.
template <int MT, int NT, int WM>
__device__ __forceinline__ void finish_tile(float4v (&acc)[MT][NT], int M, int N, int m0, int n0,
                                            int split, int splits, float alpha,
                                            const uint16_t* __restrict__ bias,
                                            uint16_t* __restrict__ y, int64_t ldy,
                                            float4v* __restrict__ slab, uint32_t* counter,
                                            uint32_t* s_flag) {
  constexpr int WN = 4 / WM;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;
  float4v frag[MT * NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) frag[mt * NT + nt] = acc[mt][nt];
  auto row_of = [&](int f, int i) { return (wm * MT + f / NT) * 16 + 4 * (lane >> 4) + i; };
  auto col_of = [&](int f) { return (wn * NT + f % NT) * 16 + (lane & 15); };
  finish_frags<MT * NT>(frag, row_of, col_of, M, N, m0, n0, split, splits, alpha, bias, y, ldy,
                        slab, counter, s_flag);
}

// 32x32 accumulator tiles (v_mfma_f32_32x32x16_f16 layout): the wave of
// column slice wn holds MT x NT tiles; register r of tile (a, b) is row m0 +
// a*32 + 8*(r/4) + 4*(lane/32) + r%4, column n0 + (wn*NT + b)*32 + lane%32.
// The workgroup has NW waves (m0 is the wave's own first row).
template <int MT, int NT, int NW = 4>
__device__ __forceinline__ void finish_tile32(float16v (&acc)[MT][NT], int M, int N, int m0, int n0,
                                              int wn, int split, int splits, float alpha,
                                              const uint16_t* __restrict__ bias,
                                              uint16_t* __restrict__ y, int64_t ldy,
                                              float4v* __restrict__ slab, uint32_t* counter,
                                              uint32_t* s_flag) {
  const int lane = threadIdx.x & 63;
  float4v frag[MT * NT * 4];
#pragma unroll
  for (int a = 0; a < MT; ++a)
#pragma unroll
    for (int b = 0; b < NT; ++b)
#pragma unroll
      for (int r4 = 0; r4 < 4; ++r4)
        frag[(a * NT + b) * 4 + r4] = float4v{acc[a][b][4 * r4], acc[a][b][4 * r4 + 1],
                                              acc[a][b][4 * r4 + 2], acc[a][b][4 * r4 + 3]};
  auto row_of = [&](int f, int i) { return (f / (NT * 4)) * 32 + 8 * (f % 4) + 4 * (lane >> 5) + i; };
  auto col_of = [&](int f) { return (wn * NT + (f / 4) % NT) * 32 + (lane & 31); };
  finish_frags<MT * NT * 4, decltype(row_of), decltype(col_of), NW>(
      frag, row_of, col_of, M, N, m0, n0, split, splits, alpha, bias, y, ldy, slab, counter, s_flag);
}

// Whole-tile write-out (one K split) through LDS. In the MFMA accumulator
// layouts a lane holds one column and 4-row runs of it, so direct stores are
// 2-byte scatters (64 per lane for a 128-row wave of 32x32 tiles). Instead
// each wave writes its bf16 results into a row-major copy of the workgroup's
// R x C tile in LDS (`lds`, at least R x (C + 8) halves, free of other use),
// and after a barrier every thread stores 16-byte row pieces: whole rows of
// consecutive addresses, an eighth of the store instructions. The value of
// each element is the direct path's (alpha * sum + bias, rounded to bf16
// once). Rows at or past M and columns at or past N are not stored; y needs
// 16-byte alignment and ldy a multiple of 8 for the 16-byte stores, else the
// pieces go out element by element. The caller has made sure that no LDS
// access or LDS-bound load of the workgroup is still in flight on `lds` (a
// wait and a barrier).
template <int C>
struct StagedPitch {
  // row pitch in halves: 16 bytes of padding keep the rows written by one
  // instruction's lane groups apart in the banks, and rows 16-byte aligned
  static constexpr int P = C + 8;
};

// the store half: 16-byte row pieces of the staged R x C tile, NW waves
template <int R, int C, int NW>
__device__ __forceinline__ void store_staged_tile(const uint16_t* lds, int M, int N, int m0, int n0,
                                                  uint16_t* __restrict__ y, int64_t ldy) {
  constexpr int P = StagedPitch<C>::P;
  const bool vec = (ldy & 7) == 0 && (reinterpret_cast<uintptr_t>(y) & 15) == 0;
  constexpr int PIECES = R * C / 8;
  static_assert(C % 8 == 0 && PIECES % (64 * NW) == 0, "whole pieces per thread");
#pragma unroll
  for (int q0 = 0; q0 < PIECES; q0 += 64 * NW) {
    const int q = q0 + threadIdx.x;
    const int row = q / (C / 8), c0 = (q % (C / 8)) * 8;
    const int m = m0 + row, n = n0 + c0;
    if (m >= M) continue;
    const uint4v v = *reinterpret_cast<const uint4v*>(&lds[row * P + c0]);
    uint16_t* dst = y + (int64_t)m * ldy + n;
    if (vec && n + 8 <= N) {
      *reinterpret_cast<uint4v*>(dst) = v;
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i)
        if (n + i < N) dst[i] = (uint16_t)(v[i / 2] >> (16 * (i % 2)));
    }
  }
}

// 32x32 accumulator tiles (the layout of finish_tile32): one row of NW
// column waves, each MT x NT tiles; R = 32 MT, C = 32 NW NT.
template <int MT, int NT, int NW>
__device__ __forceinline__ void write_tile32_staged(const float16v (&acc)[MT][NT], int M, int N, int m0,
                                                    int n0, int wn, float alpha,
                                                    const uint16_t* __restrict__ bias,
                                                    uint16_t* __restrict__ y, int64_t ldy,
                                                    uint16_t* lds) {
  constexpr int R = MT * 32, C = NW * NT * 32, P = StagedPitch<C>::P;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int b = 0; b < NT; ++b) {
    const int c = (wn * NT + b) * 32 + (lane & 31);
    const int n = n0 + c;
    const float bv = bias != nullptr && n < N ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int a = 0; a < MT; ++a)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int row = a * 32 + 8 * (r / 4) + 4 * (lane >> 5) + r % 4;
        lds[row * P + c] = (uint16_t)f32_to_bf16_bits(alpha * acc[a][b][r] + bv);
      }
  }
  __syncthreads();
  store_staged_tile<R, C, NW>(lds, M, N, m0, n0, y, ldy);
}

// 16x16 accumulator tiles (the layout of finish_tile): a WM x WN wave grid,
// each wave MT x NT tiles; R = 16 WM MT, C = 16 WN NT.
template <int MT, int NT, int WM, int WN>
__device__ __forceinline__ void write_tile16_staged(const float4v (&acc)[MT][NT], int M, int N, int m0,
                                                    int n0, int wm, int wn, float alpha,
                                                    const uint16_t* __restrict__ bias,
                                                    uint16_t* __restrict__ y, int64_t ldy,
                                                    uint16_t* lds) {
  constexpr int R = WM * MT * 16, C = WN * NT * 16, P = StagedPitch<C>::P;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int c = (wn * NT + nt) * 16 + (lane & 15);
    const int n = n0 + c;
    const float bv = bias != nullptr && n < N ? bf16_bits_to_f32(bias[n]) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = (wm * MT + mt) * 16 + 4 * (lane >> 4) + i;
        lds[row * P + c] = (uint16_t)f32_to_bf16_bits(alpha * acc[mt][nt][i] + bv);
      }
  }
  __syncthreads();
  store_staged_tile<R, C, WM * WN>(lds, M, N, m0, n0, y, ldy);
}

// Direct global -> LDS loads. The loads are issued with inline assembly and
// waited for with explicit s_waitcnt vmcnt(n): the compiler does not track
// LDS-DMA completion per ring stage and would otherwise wait for the whole
// ring before every LDS read.
typedef __attribute__((address_space(3))) void lds_void_t;
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
  return (uint32_t)(uintptr_t)(lds_void_t*)(p);
}
// 16 (or 4) bytes per lane from sbase + voff into LDS at lds + lane * 16 (or 4).
// sbase and lds must be wave-uniform. The LDS address travels in M0, passed
// as the asm statement's "{m0}" operand: the compiler writes M0 itself and
// knows the statement reads it, so no M0 value of its own can be disturbed.
// The compiler inserts no hazard wait states around inline assembly, and two
// GFX9 rules apply to these loads: an LDS-DMA load may read M0 only one wait
// state after a SALU write, and a vector memory instruction may read an SGPR
// (the base, M0) only five wait states after a VALU instruction (a
// v_readfirstlane, a 64-bit compare) wrote it. The statement's s_nop 0 keeps
// the first rule in any schedule; the second depends on the compiler's
// placement of those VALU instructions, and the build checks it on the
// generated assembly of every kernel that uses these loads (five wait states
// on every load cost 2% on the large GEMMs).
__device__ __forceinline__ void lds_load16(const void* sbase, uint32_t voff, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);  // uniform by contract; keeps it in an SGPR
  __asm__ volatile("s_nop 0\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds)
                   : "memory");
}
__device__ __forceinline__ void lds_load4(const void* sbase, uint32_t voff, uint32_t lds) {
  lds = __builtin_amdgcn_readfirstlane(lds);
  __asm__ volatile("s_nop 0\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(sbase), "{m0}"(lds)
                   : "memory");
}
// Output tile of workgroup `bid` (of `n`, one K split) in an XCD-grouped order.
// The workgroups of a launch are handed to the 8 XCDs round-robin (bid % 8),
// and each XCD has its own L2. Renumbering makes every XCD run a contiguous
// range of a band-major order: bands of `xg` row groups, walked column group
// by column group and row group by row group within a column, so the
// workgroups resident on one XCD at a time form an xg-row block that shares
// its activation rows and weight columns through that XCD's L2.
// Returns mgroup * ngroups + ngroup.
__device__ __forceinline__ int xcd_grouped_tile(int bid, int n, int ngroups, int xg) {
  const int q = n >> 3, r = n & 7, x = bid & 7;
  const int logical = x * q + (x < r ? x : r) + (bid >> 3);
  const int mgroups = n / ngroups;
  const int band = logical / (xg * ngroups);
  const int first_m = band * xg;
  const int gsize = mgroups - first_m < xg ? mgroups - first_m : xg;
  const int within = logical - first_m * ngroups;
  return (first_m + within % gsize) * ngroups + within / gsize;
}

// A wave-uniform address the compiler cannot prove uniform (e.g. formed inside
// a lane-dependent branch), moved to scalar registers for the loads above.
__device__ __forceinline__ const uint8_t* uniform_ptr(const uint8_t* p) {
  const uint64_t v = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return reinterpret_cast<const uint8_t*>(((uint64_t)hi << 32) | lo);
}
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  __asm__ volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Workgroup barrier without the compiler's release fence (which would wait
// for every outstanding load, including the ring's prefetches); LDS reads of
// the finished stage have completed (lgkmcnt) before any wave passes it.
__device__ __forceinline__ void stage_barrier() {
  __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ volatile("" ::: "memory");
}

}  // namespace fql
