// GEMM of the scaled-MFMA formats (MXFP4, MXFP8, per-tensor FP8, block FP8)
// on gfx950, plus the launch planner and the linear-layer launcher.
//
// One v_mfma_scale_f32_16x16x128_f8f6f4 computes a 16x16 output tile over a
// 128-deep chunk of K from the operands exactly as they sit in memory: E2M1 or
// E4M3 codes and, for the MX formats, one E8M0 byte per row and 32-block
// (lane 16j + r carries the scale of row r, block j). Nothing is
// dequantized. Per-tensor FP8 passes the unit scale and applies alpha in the
// epilogue; block FP8 computes each chunk into a fresh accumulator and adds
// it with the product of the row's and the column block's float32 scales
// (the per-128-group promotion).
//
// Workgroup: NW = WM x WN waves; wave (wm, wn) owns MTW x NTW output tiles of
// 16x16, so the workgroup tile is (WM*MTW*16) x (WN*NTW*16). The activation
// and weight tiles of one chunk go through an LDS ring of ST stages, filled by
// direct global->LDS loads that every wave issues for its share of the stage
// (item e of the stage is loaded by wave e % NW), spread between its MFMAs.
// The per-CU vector-memory path (about 64 B/clk) and LDS reads set the tile
// sizes: bytes per flop fall as 1/tile_rows + 1/tile_cols.
#include <algorithm>
#include <cstddef>
#include <cstdio>
#include <cstdlib>
#include <string>

#include "fql_device.h"
#include "fql_gemm.h"
#include "fql_internal.h"
#include "sc_quant.h"

namespace fql {

typedef int int8v __attribute__((ext_vector_type(8)));

ScDims sc_dims(int fmt, int64_t rows, int64_t K, bool weight) {
  ScDims d;
  d.rows_p = round_up(rows, 16);
  d.Kp = round_up(K, 128);
  d.KC = d.Kp / 128;
  d.quads = (d.rows_p + 63) / 64;
  d.code_bytes = fmt == SC_MXFP4 ? d.rows_p * d.Kp / 2 : d.rows_p * d.Kp;
  if (fmt == SC_MXFP4 || fmt == SC_MXFP8) d.scale_bytes = d.quads * d.KC * 256;
  else if (fmt == SC_FP8_BLOCK) d.scale_bytes = weight ? round_up((rows / 128) * d.KC * 4, 256) : d.quads * d.KC * 256;
  else d.scale_bytes = 0;
  return d;
}

template <int F>
struct ScTraits {
  static constexpr int H = F == SC_MXFP4 ? 1 : 2;            // 1 KiB halves per tile-chunk
  static constexpr int FMT = F == SC_MXFP4 ? 4 : 0;          // MFMA operand format (E2M1 / E4M3)
  static constexpr bool MX = F == SC_MXFP4 || F == SC_MXFP8;  // E8M0 scales in the operands
  static constexpr bool BLOCK = F == SC_FP8_BLOCK;
};

template <int F, int WM, int WN, int MTW, int NTW>
struct ScStage {
  static constexpr int H = ScTraits<F>::H;
  static constexpr int TA = WM * MTW, TB = WN * NTW;
  static_assert(TA == 1 || TA == 2 || TA % 4 == 0, "activation tiles within whole scale quads");
  static constexpr int QA = (TA + 3) / 4;
  static constexpr int QB = TB / 4;
  // block FP8: one float per 128-column block of the workgroup
  static constexpr int NBS = (TB * 16 + 127) / 128;
  static constexpr int SA = ScTraits<F>::MX || ScTraits<F>::BLOCK ? QA : 0;
  static constexpr int SB = ScTraits<F>::MX ? QB : (ScTraits<F>::BLOCK ? NBS : 0);
  uint4v a[TA][H][64];
  uint4v b[TB][H][64];
  uint32_t as[SA > 0 ? SA : 1][64];
  uint32_t bs[SB > 0 ? SB : 1][64];
};

// One scaled MFMA whose E8M0 scales are byte `BA` of `sa` and byte `BB` of
// `sb` (the instruction's scale byte select; it must be an immediate).
template <int FMT, int BA, int BB>
__device__ __forceinline__ float4v mfma_scale_bytes(const int8v& a, const int8v& b, const float4v& c, int sa,
                                                    int sb) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, FMT, FMT, BA, sa, BB, sb);
}
// The same with the bytes given as values that are constants once the
// caller's loops are unrolled (the switch folds to one call).
template <int FMT>
__device__ __forceinline__ float4v mfma_scale_sel(const int8v& a, const int8v& b, const float4v& c, int sa, int ba,
                                                  int sb, int bb) {
  switch (ba * 4 + bb) {
#define FQL_SC_SEL(I) \
  case I: return mfma_scale_bytes<FMT, I / 4, I % 4>(a, b, c, sa, sb);
    FQL_SC_SEL(0) FQL_SC_SEL(1) FQL_SC_SEL(2) FQL_SC_SEL(3) FQL_SC_SEL(4) FQL_SC_SEL(5) FQL_SC_SEL(6)
    FQL_SC_SEL(7) FQL_SC_SEL(8) FQL_SC_SEL(9) FQL_SC_SEL(10) FQL_SC_SEL(11) FQL_SC_SEL(12) FQL_SC_SEL(13)
    FQL_SC_SEL(14)
#undef FQL_SC_SEL
    default: return mfma_scale_bytes<FMT, 3, 3>(a, b, c, sa, sb);
  }
}

template <int F, int WM, int WN, int MTW, int NTW, int ST>
__global__ __launch_bounds__(64 * WM * WN) void gemm_sc_kernel(
    const uint8_t* __restrict__ xcodes, const uint8_t* __restrict__ xscales,
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales, int M, int N,
    int64_t KC, int ntiles_w, int64_t quads_w, int ngroups, int kc_per_split, int dp, int splits,
    float alpha, const float* __restrict__ alpha_dev, const uint16_t* __restrict__ bias,
    uint16_t* __restrict__ y, int64_t ldy, float4v* __restrict__ partial,
    uint32_t* __restrict__ counters) {
  if (alpha_dev != nullptr) alpha = *alpha_dev;  // output scale kept in device memory
  typedef ScTraits<F> T;
  typedef ScStage<F, WM, WN, MTW, NTW> Stage;
  constexpr int NW = WM * WN, H = T::H, TA = Stage::TA, TB = Stage::TB;
  constexpr int NA = TA * H, NB = TB * H, SA = Stage::SA, SB = Stage::SB;
  constexpr int ITEMS = NA + NB + SA + SB;
  constexpr int L = (ITEMS + NW - 1) / NW;  // loads per wave per chunk
  constexpr int P = MTW * NTW;              // MFMAs per wave per chunk
  constexpr int CHUNK = 64 * 16 * H;        // bytes of one tile-chunk
  // Fragment prefetch (the MFMAs of a chunk read registers filled during the
  // previous chunk) for MXFP4 and block FP8; per-tensor FP8 and MXFP8 read
  // their fragments just before the MFMAs, which measured faster for them
  // (their 3-stage rings lose a chunk of load lead time to the prefetch, and
  // they have no per-chunk VALU work for it to hide).
  constexpr bool PF = F == SC_MXFP4 || F == SC_FP8_BLOCK;
  static_assert(ST >= 3 && ST <= 8, "ring depth");
  static_assert(L * (PF ? ST - 1 : ST - 2) <= 63, "vmcnt range");
  static_assert(TB % 4 == 0, "weight tiles come in quads");
  static_assert(!T::BLOCK || (NTW * 16 <= 128 && 128 % (NTW * 16) == 0), "a wave's columns in one block");
  __shared__ Stage stage[ST];
  __shared__ uint32_t s_flag;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  // Workgroups [0, dp) compute whole tiles (tile = workgroup); after them
  // each remaining tile takes `splits` consecutive workgroups, one K range
  // each. Tiles are numbered row-major: mgroup * ngroups + ngroup.
  const int b = blockIdx.x;
  const bool whole = b < dp;
  const int tilegrp = whole ? b : dp + (b - dp) / splits;
  const int split = whole ? 0 : (b - dp) % splits;
  const int nsplit = whole ? 1 : splits;
  const int sslot = whole ? 0 : tilegrp - dp;  // partial slab and counter of a split tile
  const int ngroup = tilegrp % ngroups;
  const int mgroup = tilegrp / ngroups;
  const int64_t c_begin = whole ? 0 : (int64_t)split * kc_per_split;
  const int64_t c_last = whole ? KC : c_begin + kc_per_split;
  const int64_t c_end = c_last < KC ? c_last : KC;
  const int nch = (int)(c_end - c_begin);
  const int64_t a_tile0 = (int64_t)mgroup * TA;
  const int64_t a_quad0 = a_tile0 / 4;
  const int a_qoff = (int)(a_tile0 % 4);  // nonzero only when TA < 4
  const int64_t b_tile0 = (int64_t)ngroup * TB;

  // This wave's share of a stage: item e = wave + NW*j (waves past the last
  // item repeat the last item: same bytes, same place, and the same kind as
  // the other items of that slot). The item table is built once
  // (scalar registers: source base and per-chunk stride, LDS offset within
  // the stage, load width), so issuing a load in the loop costs a few scalar
  // instructions instead of re-deriving the item's address.
  const uint8_t* it_src[L];
  uint32_t it_stride[L], it_lds[L], it_voff[L];
  bool it_wide[L];
#pragma unroll
  for (int j = 0; j < L; ++j) {
    int e = wave + NW * j;
    e = e < ITEMS ? e : ITEMS - 1;
    if (e < NA) {
      const int t = e / H, h = e % H;
      it_src[j] = xcodes + (a_tile0 + t) * KC * CHUNK + h * 1024;
      it_stride[j] = CHUNK;
      it_lds[j] = (uint32_t)offsetof(Stage, a) + (t * H + h) * 1024;
      it_wide[j] = true;
    } else if (e < NA + NB) {
      const int t = (e - NA) / H, h = (e - NA) % H;
      const int64_t gt = b_tile0 + t < ntiles_w ? b_tile0 + t : 0;  // past N: tile 0, never stored
      it_src[j] = wcodes + gt * KC * CHUNK + h * 1024;
      it_stride[j] = CHUNK;
      it_lds[j] = (uint32_t)offsetof(Stage, b) + (t * H + h) * 1024;
      it_wide[j] = true;
    } else if (e < NA + NB + SA) {
      const int q = e - NA - NB;
      it_src[j] = xscales + (a_quad0 + q) * KC * 256;
      it_stride[j] = 256;
      it_lds[j] = (uint32_t)offsetof(Stage, as) + q * 256;
      it_wide[j] = false;
    } else {
      const int q = e - NA - NB - SA;
      it_lds[j] = (uint32_t)offsetof(Stage, bs) + q * 256;
      it_wide[j] = false;
      if (T::MX) {
        const int64_t gq = b_tile0 / 4 + q < quads_w ? b_tile0 / 4 + q : 0;
        it_src[j] = wscales + gq * KC * 256;
        it_stride[j] = 256;
      } else {  // block FP8: the column block's scale, broadcast to all 64 slots
        int64_t nb = (b_tile0 * 16) / 128 + q;
        const int64_t nbs = ((int64_t)ntiles_w * 16) / 128;
        nb = nb < nbs ? nb : 0;
        it_src[j] = wscales + nb * KC * 4;
        it_stride[j] = 4;
      }
    }
    it_voff[j] = it_wide[j] ? (uint32_t)lane * 16 : (T::BLOCK && e >= NA + NB + SA ? 0u : (uint32_t)lane * 4);
  }
  // Which kind of item slot j holds is known at compile time once the loops
  // are unrolled whenever all waves' item j are code tiles (or all MX scale
  // quads): then width and stride are constants and no branch is emitted.
  // For those the chunk's offset rides in the per-lane offset (one vector add
  // per chunk and stride, see ChunkOffsets) instead of a 64-bit scalar add per
  // load; a tile's KC chunks stay far below 4 GiB.
  struct ChunkOffsets {
    uint32_t code, scale;  // lane*16 + c*CHUNK, lane*4 + c*256
  };
  auto offsets_of = [&](int64_t c) -> ChunkOffsets {
    return ChunkOffsets{(uint32_t)lane * 16u + (uint32_t)c * (uint32_t)CHUNK, (uint32_t)lane * 4u + (uint32_t)c * 256u};
  };
  auto issue_item = [&](Stage& sg, int64_t c, const ChunkOffsets& o, int j) {
    const uint32_t lds = lds_offset(&sg) + it_lds[j];
    if (NW * j + NW <= NA + NB) {
      lds_load16(it_src[j], o.code, lds);
    } else if (NW * j >= NA + NB && T::MX) {
      lds_load4(it_src[j], o.scale, lds);
    } else {
      const uint8_t* src = it_src[j] + (uint32_t)c * it_stride[j];
      if (it_wide[j]) lds_load16(src, it_voff[j], lds);
      else lds_load4(src, it_voff[j], lds);
    }
  };

  float4v acc[MTW][NTW];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};

  if constexpr (PF) {
    // This wave's operand fragments of one chunk, in two register sets: the
    // MFMAs of chunk i read set i % 2 while the LDS reads of chunk i+1 fill the
    // other, so no MFMA waits on an LDS read issued just before it. Each
    // fragment of chunk i+1 is read once the last MFMA of chunk i that reads
    // the same slot is issued, so only about one set is live at a time.
    // Fragments are kept as 16-byte halves: an FP4 operand fills only the
    // first half of the MFMA's 32-byte operand, so no zero half is held across
    // the loop. The E8M0 scales stay packed as loaded, four tiles' bytes per dword: the
    // wave's row tiles start at tile a_first of the loaded quads and its column
    // tiles at b_first (MTW and NTW divide 4 or are multiples of it, so the
    // first tile's byte offset is the only runtime part: the words are shifted
    // by it once, and tile mt's byte is mt % 4 of word mt / 4).
    constexpr int AW = (MTW + 3) / 4, BW = (NTW + 3) / 4;
    static_assert((MTW % 4 == 0 || 4 % MTW == 0) && (NTW % 4 == 0 || 4 % NTW == 0), "tiles per wave");
    const int a_first = a_qoff + wm * MTW, b_first = wn * NTW;
    const int a_shift = 8 * (a_first % 4), b_shift = 8 * (b_first % 4);
    uint4v fa[2][MTW][H];  // activation tiles
    int fsa[2][AW];        // their E8M0 scale words (MX)
    float4v fs4[2][MTW];   // block FP8: row scales x the column block's scale
    uint4v fb[2][NTW][H];  // weight tiles
    int fsb[2][BW];        // their E8M0 scale words (MX)
    float fsw[2];          // block FP8: the wave's column block scale
    auto operand = [&](const uint4v (&f)[H]) -> int8v {
      const uint4v q0 = f[0];
      if (H == 1) return int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, 0, 0, 0, 0};
      const uint4v q1 = f[H - 1];
      return int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
    };
    auto read_sw = [&](const Stage& sg, int q) {
      fsw[q] = T::BLOCK ? __uint_as_float(sg.bs[(wn * NTW * 16) / 128][0]) : 0.0f;
    };
    auto read_b = [&](const Stage& sg, int q, int nt) {
      const int t = wn * NTW + nt;
#pragma unroll
      for (int h = 0; h < H; ++h) fb[q][nt][h] = sg.b[t][h][lane];
      if (T::MX && nt % 4 == 0) fsb[q][nt / 4] = (int)(sg.bs[(b_first + nt) / 4][lane] >> b_shift);
    };
    auto read_a = [&](const Stage& sg, int q, int mt) {
      const int t = wm * MTW + mt;
#pragma unroll
      for (int h = 0; h < H; ++h) fa[q][mt][h] = sg.a[t][h][lane];
      const int at = a_qoff + t;  // tile index within the loaded scale quads
      if (T::MX && mt % 4 == 0) fsa[q][mt / 4] = (int)(sg.as[(a_first + mt) / 4][lane] >> a_shift);
      if (T::BLOCK) {
        // row scales of the lane's four accumulator rows 16*at + 4*(lane/16) + i
        const float* rs = reinterpret_cast<const float*>(&sg.as[at / 4][0]) + 16 * (at % 4) + 4 * (lane >> 4);
        fs4[q][mt] = float4v{rs[0] * fsw[q], rs[1] * fsw[q], rs[2] * fsw[q], rs[3] * fsw[q]};
      }
    };
    auto mfma = [&](int q, int mt, int nt) {
      if (T::BLOCK) {
        const float4v z = float4v{0.f, 0.f, 0.f, 0.f};
        const float4v part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(fa[q][mt]), operand(fb[q][nt]), z,
                                                                              0, 0, 0, 127, 0, 127);
        acc[mt][nt] += part * fs4[q][mt];
      } else if (T::MX) {
        acc[mt][nt] = mfma_scale_sel<T::FMT>(operand(fa[q][mt]), operand(fb[q][nt]), acc[mt][nt], fsa[q][mt / 4], mt % 4,
                                             fsb[q][nt / 4], nt % 4);
      } else {
        acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(operand(fa[q][mt]), operand(fb[q][nt]), acc[mt][nt],
                                                                       T::FMT, T::FMT, 0, 127, 0, 127);
      }
    };

    // Ring: chunk i lives in stage i % ST. The first ST chunks are loaded up
    // front and chunk 0's fragments read. Chunk i then waits for the wave's
    // own loads of chunk i+1, passes the barrier (every
    // wave's loads of chunk i+1 have landed, and every wave has read chunk i's
    // fragments out of stage i % ST) and issues its MFMAs from registers; after
    // each row tile's MFMAs it reads that row tile of chunk i+1, during the last
    // row tile's the weight tiles of chunk i+1, and it refills stage i % ST with
    // chunk i+ST between the MFMAs. Chunk indices past the end are clamped to
    // the last chunk, so every chunk issues the same loads, reads and barrier
    // (the last chunk's reads of a "next" chunk are in-bounds and unused).
#pragma unroll
    for (int p0 = 0; p0 < ST; ++p0) {
      const int64_t c = c_begin + p0 < c_end ? c_begin + p0 : c_end - 1;
      const ChunkOffsets o = offsets_of(c);
#pragma unroll
      for (int j = 0; j < L; ++j) issue_item(stage[p0], c, o, j);
    }
    wait_vmcnt<L * (ST - 1)>();  // this wave's loads of chunk 0
    stage_barrier();
    read_sw(stage[0], 0);
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) read_b(stage[0], 0, nt);
#pragma unroll
    for (int mt = 0; mt < MTW; ++mt) read_a(stage[0], 0, mt);

    auto chunk = [&](int i, int s, int q) {
      wait_vmcnt<L * (ST - 2)>();  // this wave's loads of chunk i+1
      stage_barrier();
      const Stage& next = stage[(s + 1) % ST];
      read_sw(next, q ^ 1);
      int64_t rc = c_begin + i + ST;
      rc = rc < c_end ? rc : c_end - 1;
      const ChunkOffsets ro = offsets_of(rc);
      int p = 0;
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
          for (int j = 0; j < L; ++j)
            if ((j * P) / L == p) issue_item(stage[s], rc, ro, j);
          mfma(q, mt, nt);
          ++p;
          if (mt == MTW - 1) read_b(next, q ^ 1, nt);  // the tile's last MFMA of this chunk is issued
        }
        read_a(next, q ^ 1, mt);
        // keep the reads behind the MFMAs that free their registers
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    // unrolled so that the stage and the fragment set of every chunk are static
    constexpr int U = ST % 2 == 0 ? ST : 2 * ST;
    for (int i0 = 0; i0 < nch; i0 += U) {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (i0 + u < nch) chunk(i0 + u, u % ST, u % 2);
    }
  } else {
    // one chunk: fragments from stage sg, MFMAs, and the refill loads of the
    // stage `refill` (chunk rc) spread between the MFMAs
    auto compute = [&](const Stage& sg, Stage& refill, int64_t rc) {
      const ChunkOffsets ro = offsets_of(rc);
      int8v b[NTW];
      int sb[NTW];
#pragma unroll
      for (int nt = 0; nt < NTW; ++nt) {
        const int t = wn * NTW + nt;
        const uint4v q0 = sg.b[t][0][lane];
        if (H == 1) {
          b[nt] = int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, 0, 0, 0, 0};
        } else {
          const uint4v q1 = sg.b[t][H - 1][lane];
          b[nt] = int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
        }
        sb[nt] = T::MX ? (int)((sg.bs[t / 4][lane] >> (8 * (t % 4))) & 0xFFu) : 127;
      }
      float swv = 0.0f;
      if (T::BLOCK) swv = __uint_as_float(sg.bs[(wn * NTW * 16) / 128][0]);
      int p = 0;
#pragma unroll
      for (int mt = 0; mt < MTW; ++mt) {
        const int t = wm * MTW + mt;
        const uint4v q0 = sg.a[t][0][lane];
        int8v a;
        if (H == 1) {
          a = int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, 0, 0, 0, 0};
        } else {
          const uint4v q1 = sg.a[t][H - 1][lane];
          a = int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
        }
        const int at = a_qoff + t;  // tile index within the loaded scale quads
        int sa = 127;
        if (T::MX) sa = (int)((sg.as[at / 4][lane] >> (8 * (at % 4))) & 0xFFu);
        float4v s4 = float4v{0.f, 0.f, 0.f, 0.f};
        if (T::BLOCK) {
          // row scales of the lane's four accumulator rows 16*at + 4*(lane/16) + i
          const float* rs = reinterpret_cast<const float*>(&sg.as[at / 4][0]) + 16 * (at % 4) + 4 * (lane >> 4);
          s4 = float4v{rs[0] * swv, rs[1] * swv, rs[2] * swv, rs[3] * swv};
        }
#pragma unroll
        for (int nt = 0; nt < NTW; ++nt) {
#pragma unroll
          for (int j = 0; j < L; ++j)
            if ((j * P) / L == p) issue_item(refill, rc, ro, j);
          if (T::BLOCK) {
            const float4v z = float4v{0.f, 0.f, 0.f, 0.f};
            const float4v part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[nt], z, 0, 0, 0, 127, 0, 127);
            acc[mt][nt] += part * s4;
          } else {
            acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[nt], acc[mt][nt], T::FMT,
                                                                           T::FMT, 0, sa, 0, sb[nt]);
          }
          ++p;
        }
      }
    };

    // Ring: chunk i lives in stage i % ST. Before computing chunk i a wave
    // waits for its own loads of chunk i, passes the barrier (everyone's have
    // landed and everyone has finished chunk i-1), then refills stage
    // (i-1) % ST with chunk i+ST-1 while computing (clamped chunk index past
    // the end: a static number of loads per chunk).
#pragma unroll
    for (int p0 = 0; p0 < ST - 1; ++p0) {
      const int64_t c = c_begin + p0 < c_end ? c_begin + p0 : c_end - 1;
      const ChunkOffsets o = offsets_of(c);
#pragma unroll
      for (int j = 0; j < L; ++j) issue_item(stage[p0], c, o, j);
    }
    for (int i0 = 0; i0 < nch; i0 += ST) {
#pragma unroll
      for (int j = 0; j < ST; ++j) {
        if (i0 + j < nch) {
          wait_vmcnt<L * (ST - 2)>();
          stage_barrier();
          int64_t rc = c_begin + i0 + j + ST - 1;
          rc = rc < c_end ? rc : c_end - 1;
          compute(stage[j], stage[(j + ST - 1) % ST], rc);
        }
      }
    }
  }
  wait_vmcnt<0>();  // no LDS load may still be in flight when the workgroup ends

  const int m0 = mgroup * TA * 16, n0 = ngroup * TB * 16;
  // a whole tile goes out through the ring's LDS when the staged tile fits it
  // (and its 16-byte pieces divide evenly among the threads)
  constexpr bool kStaged = sizeof(stage) >= (size_t)TA * 16 * StagedPitch<TB * 16>::P * 2 &&
                           (TA * 16 * TB * 16 / 8) % (64 * NW) == 0;
  if constexpr (kStaged) {
    if (nsplit == 1) {
      __syncthreads();  // every wave's loads have landed: the ring is free
      write_tile16_staged<MTW, NTW, WM, WN>(acc, M, N, m0, n0, wm, wn, alpha, bias, y, ldy,
                                            reinterpret_cast<uint16_t*>(&stage[0]));
      return;
    }
  }
  float4v frag[P];
#pragma unroll
  for (int mt = 0; mt < MTW; ++mt)
#pragma unroll
    for (int nt = 0; nt < NTW; ++nt) frag[mt * NTW + nt] = acc[mt][nt];
  auto row_of = [&](int f, int i) { return (wm * MTW + f / NTW) * 16 + 4 * (lane >> 4) + i; };
  auto col_of = [&](int f) { return (wn * NTW + f % NTW) * 16 + (lane & 15); };
  float4v* slab = partial + (int64_t)sslot * splits * (NW * P * 64);
  finish_frags<P, decltype(row_of), decltype(col_of), NW>(
      frag, row_of, col_of, M, N, m0, n0, split, nsplit, alpha, bias, y, ldy, slab, counters + sslot,
      &s_flag);
}

// ---------------------------------------------------------------------------
// small-M GEMV: per-wave LDS rings, no workgroup barrier in the loop
// ---------------------------------------------------------------------------
//
// For M <= 32 the call is a stream over the weight: every weight byte is used
// once. W waves of a workgroup share NT 16-column tiles and split the K range;
// each wave streams its own chunks (activation tiles, weight tiles, scales)
// into a private LDS ring of D stages with direct global->LDS loads and waits
// only for its own loads (explicit vmcnt; no barrier until the end), so D
// chunks per wave are always in flight. The W partial sums are added in wave
// order through LDS at the end (deterministic, no global atomics).

// Wait until at most k chunks of L loads each are still in flight (k <= K).
template <int L, int K>
struct WaitChunks {
  static __device__ __forceinline__ void run(int k) {
    if (k >= K) wait_vmcnt<L * K>();
    else WaitChunks<L, K - 1>::run(k);
  }
};
template <int L>
struct WaitChunks<L, 0> {
  static __device__ __forceinline__ void run(int) { wait_vmcnt<0>(); }
};

template <int F, int MT, int NT, int FQ = 0>
struct ScvStage {
  static constexpr int H = ScTraits<F>::H;
  uint4v a[MT][H][64];
  uint4v b[NT][H][64];
  uint32_t sa[64];  // MX: A scale quad dword; block FP8: A row scales (float bits)
  uint32_t sb[64];  // MX: B scale quad dword; block FP8: the column block's scale (broadcast)
};
// With the activation quantized inside the workgroup (FQ = 1) the ring
// carries only the weight.
template <int F, int MT, int NT>
struct ScvStage<F, MT, NT, 1> {
  static constexpr int H = ScTraits<F>::H;
  uint4v b[NT][H][64];
  uint32_t sb[64];
};

// FQ = 1: the workgroup first quantizes rows 0 .. M-1 of x itself, with the
// standalone quantizer's block arithmetic, into a compact LDS copy of the
// activation operand for the whole K range (dynamic LDS, rows 0 .. M-1 only:
// codes [KC][H][4 lane groups][M] x 16 B, then the scales: MX [KC][4][M]
// dwords (byte 0), block FP8 [KC][M] floats); blocks past K are zero. Lanes
// of rows >= M read row 0 (an output row depends only on its own activation
// row and rows >= M are never stored). The ring then carries only the
// weight. This removes the separate quantizer launch for decode sizes.
template <int F, int W, int MT, int NT, int D, int FQ>
__global__ __launch_bounds__(64 * W) void gemv_sc_kernel(
    const uint8_t* __restrict__ xcodes, const uint8_t* __restrict__ xscales,
    const uint8_t* __restrict__ wcodes, const uint8_t* __restrict__ wscales, int M, int N,
    int64_t KC, int ntiles_w, int64_t quads_w, float alpha, const float* __restrict__ alpha_dev,
    const uint16_t* __restrict__ bias, uint16_t* __restrict__ y, int64_t ldy,
    const uint16_t* __restrict__ x, int64_t ldx, int aligned, float inv_scale, int64_t K) {
  if (alpha_dev != nullptr) alpha = *alpha_dev;  // output scale kept in device memory
  typedef ScTraits<F> T;
  typedef ScvStage<F, MT, NT, FQ> Stage;
  constexpr int H = T::H;
  constexpr int64_t CHUNK = 1024 * H;
  // loads per chunk
  constexpr int L = (FQ ? 0 : MT * H) + NT * H + (T::MX || T::BLOCK ? (FQ ? 1 : 2) : 0);
  static_assert(MT >= 1 && MT <= 4 && (NT == 1 || NT == 2 || NT == 4), "tiles within one scale quad");
  static_assert(L * (D - 1) <= 63, "vmcnt range");
  __shared__ Stage ring[W][D];
  static_assert(sizeof(ring) >= sizeof(float4v) * W * MT * NT * 64, "reduction buffer aliases the ring");
  float4v(*red)[MT * NT][64] = reinterpret_cast<float4v(*)[MT * NT][64]>(&ring[0][0]);
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int64_t tile0 = (int64_t)blockIdx.x * NT;
  const int64_t cpw = (KC + W - 1) / W;
  const int64_t c0 = (int64_t)wave * cpw < KC ? (int64_t)wave * cpw : KC;
  const int64_t c1 = c0 + cpw < KC ? c0 + cpw : KC;
  const int n = (int)(c1 - c0);

  int64_t bt[NT];
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) bt[nt] = tile0 + nt < ntiles_w ? tile0 + nt : ntiles_w - 1;  // past N: never stored
  const int64_t bquad = tile0 / 4 < quads_w ? tile0 / 4 : quads_w - 1;
  const int64_t nbs = ((int64_t)ntiles_w * 16) / 128;
  const int64_t nb = (tile0 * 16) / 128 < nbs ? (tile0 * 16) / 128 : (nbs > 0 ? nbs - 1 : 0);

  extern __shared__ __attribute__((aligned(16))) uint8_t sc_xop[];
  const uint32_t* xsd = reinterpret_cast<const uint32_t*>(sc_xop + KC * H * 4 * M * 16);

  // (called after the first weight chunks are issued, so they load meanwhile)
  auto quantize_activation = [&]() {
    const int64_t nblk = KC * 4;              // 32-blocks per row of the padded operand
    const int64_t total = (int64_t)M * nblk;  // rows >= M are never stored: not quantized
    for (int64_t base = 0; base < total; base += 64 * W) {
      // consecutive lanes take consecutive blocks of a row, so the four blocks
      // of a 128-group (block FP8) sit in lanes l, l^1, l^2, l^3
      const int64_t i = base + tid;
      const bool inside = i < total;
      const int64_t m = inside ? i / nblk : 0, b = inside ? i - m * nblk : 0;
      const bool valid = inside && b * 32 < K;
      float v[32];
      if (valid) load32(x + m * ldx + b * 32, aligned != 0, v);
      else
#pragma unroll
        for (int j = 0; j < 32; ++j) v[j] = 0.0f;
      uint32_t w[8], sbyte = 0;
      float gs = 0.0f;
      quant_block32<F>(v, valid, inv_scale, w, sbyte, gs);
      if (inside) {
        if (!valid) {
#pragma unroll
          for (int j = 0; j < 8; ++j) w[j] = 0u;
          sbyte = 0;
          gs = 0.0f;
        }
        const int64_t c = b / 4;
        const int kg = (int)(b % 4);
        // FP4: the 16-byte piece of row m is lane group kg; FP8: pieces h16 =
        // 2kg + j go to half h16/4, lane group h16%4
        if (F == SC_MXFP4) {
          *reinterpret_cast<uint4v*>(sc_xop + ((c * 4 + kg) * M + m) * 16) = uint4v{w[0], w[1], w[2], w[3]};
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const int h16 = 2 * kg + j;
            *reinterpret_cast<uint4v*>(sc_xop + (((c * H + h16 / 4) * 4 + h16 % 4) * M + m) * 16) =
                uint4v{w[4 * j], w[4 * j + 1], w[4 * j + 2], w[4 * j + 3]};
          }
        }
        uint8_t* sbase = sc_xop + KC * H * 4 * M * 16;
        if (T::MX) reinterpret_cast<uint32_t*>(sbase)[(c * 4 + kg) * M + m] = sbyte;
        if (T::BLOCK && kg == 0) reinterpret_cast<float*>(sbase)[c * M + m] = gs;
      }
    }
    __syncthreads();
  };

  auto issue = [&](Stage& sg, int64_t c) {
    const uint32_t base = lds_offset(&sg);
    if constexpr (!FQ) {
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int h = 0; h < H; ++h)
          lds_load16(xcodes + (mt * KC + c) * CHUNK + h * 1024, lane * 16,
                     base + (uint32_t)offsetof(Stage, a) + (mt * H + h) * 1024);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int h = 0; h < H; ++h)
        lds_load16(wcodes + (bt[nt] * KC + c) * CHUNK + h * 1024, lane * 16,
                   base + (uint32_t)offsetof(Stage, b) + (nt * H + h) * 1024);
    if constexpr (!FQ) {
      if (T::MX || T::BLOCK) lds_load4(xscales + c * 256, lane * 4, base + (uint32_t)offsetof(Stage, sa));
    }
    if (T::MX) lds_load4(wscales + (bquad * KC + c) * 256, lane * 4, base + (uint32_t)offsetof(Stage, sb));
    else if (T::BLOCK) lds_load4(wscales + (nb * KC + c) * 4, 0u, base + (uint32_t)offsetof(Stage, sb));
  };

  float4v acc[MT][NT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) acc[mt][nt] = float4v{0.f, 0.f, 0.f, 0.f};

  // the lane's activation row of row tile mt in the compact copy (rows >= M
  // read row 0)
  auto fq_row = [&](int mt) -> int {
    const int row = 16 * mt + (lane & 15);
    return row < M ? row : 0;
  };
  // the activation's code words of row tile mt, half h, chunk c
  auto a_word = [&](const Stage& sg, int mt, int h, int64_t c) -> uint4v {
    if constexpr (FQ)
      return *reinterpret_cast<const uint4v*>(sc_xop + (((c * H + h) * 4 + (lane >> 4)) * M + fq_row(mt)) * 16);
    else return sg.a[mt][h][lane];
  };
  // MX: the E8M0 scale byte of row tile mt for this lane's row and block
  auto a_scale_byte = [&](const Stage& sg, int mt, int64_t c) -> int {
    if constexpr (FQ) return (int)(xsd[(c * 4 + (lane >> 4)) * M + fq_row(mt)] & 0xFFu);
    else return (int)((sg.sa[lane] >> (8 * mt)) & 0xFFu);
  };
  // block FP8: the float32 scale of row 16mt + 4(lane/16) + i
  auto a_row_scale = [&](const Stage& sg, int mt, int i, int64_t c) -> float {
    const int row = 16 * mt + 4 * (lane >> 4) + i;
    if constexpr (FQ) return reinterpret_cast<const float*>(xsd)[c * M + (row < M ? row : 0)];
    else return reinterpret_cast<const float*>(&sg.sa[0])[row];
  };
  auto compute = [&](const Stage& sg, int64_t c) {
    int8v b[NT];
    int sb[NT];
    const uint32_t sbw = sg.sb[lane];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
      const uint4v q0 = sg.b[nt][0][lane];
      if (H == 1) {
        b[nt] = int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, 0, 0, 0, 0};
      } else {
        const uint4v q1 = sg.b[nt][H - 1][lane];
        b[nt] = int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
      }
      sb[nt] = T::MX ? (int)((sbw >> (8 * ((tile0 + nt) % 4))) & 0xFFu) : 127;
    }
    const float swv = T::BLOCK ? __uint_as_float(sbw) : 0.0f;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      const uint4v q0 = a_word(sg, mt, 0, c);
      int8v a;
      if (H == 1) {
        a = int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, 0, 0, 0, 0};
      } else {
        const uint4v q1 = a_word(sg, mt, H - 1, c);
        a = int8v{(int)q0.x, (int)q0.y, (int)q0.z, (int)q0.w, (int)q1.x, (int)q1.y, (int)q1.z, (int)q1.w};
      }
      const int sa = T::MX ? a_scale_byte(sg, mt, c) : 127;
      float4v s4 = float4v{0.f, 0.f, 0.f, 0.f};
      if (T::BLOCK)
        s4 = float4v{a_row_scale(sg, mt, 0, c) * swv, a_row_scale(sg, mt, 1, c) * swv,
                     a_row_scale(sg, mt, 2, c) * swv, a_row_scale(sg, mt, 3, c) * swv};
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        if (T::BLOCK) {
          const float4v z = float4v{0.f, 0.f, 0.f, 0.f};
          const float4v part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[nt], z, 0, 0, 0, 127, 0, 127);
          acc[mt][nt] += part * s4;
        } else {
          acc[mt][nt] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b[nt], acc[mt][nt], T::FMT,
                                                                         T::FMT, 0, sa, 0, sb[nt]);
        }
      }
    }
  };

  // chunk idx of this wave lives in stage idx % D; before computing it the
  // wave waits until at most min(D-1, n-1-idx) later chunks are in flight
  Stage* mine = ring[wave];
  const int pre = n < D ? n : D;
#pragma unroll
  for (int j = 0; j < D; ++j)
    if (j < pre) issue(mine[j], c0 + j);
  if constexpr (FQ) quantize_activation();
  for (int i0 = 0; i0 < n; i0 += D) {
#pragma unroll
    for (int j = 0; j < D; ++j) {
      const int idx = i0 + j;
      if (idx < n) {
        const int later = n - 1 - idx;
        WaitChunks<L, D - 1>::run(later < D - 1 ? later : D - 1);
        compute(mine[j], c0 + idx);
        if (idx + D < n) {
          __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");  // stage reads done before the refill
          issue(mine[j], c0 + idx + D);
        }
      }
    }
  }
  wait_vmcnt<0>();
  __syncthreads();  // every wave is done with the ring, which now holds the partial sums

  // wave-order reduction of the W partial sums, then the epilogue: fragment
  // f (row tile f / NT, column tile f % NT) is finished by wave f % W
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
// configurations, plan, launcher
// ---------------------------------------------------------------------------

// (WM, WN, MTW, NTW, ST) GEMM configurations built (the planner's choices:
// 64 x 128 tiles up to M = 128, 128 x 128 for 8-bit formats up to M = 512,
// then 256 x 128 for 8-bit formats and 256 x 256 for FP4, whose ring alone
// fits in LDS; 16 x 128 tiles as the fallback).
#define FQL_SC_CONFIGS_ANY(X, F) \
  X(F, 1, 4, 4, 2, 4) X(F, 2, 2, 4, 4, 3) X(F, 4, 2, 4, 4, 3) X(F, 1, 4, 1, 2, 4)
#define FQL_SC_CONFIGS_FP4(X, F) FQL_SC_CONFIGS_ANY(X, F) X(F, 2, 4, 8, 4, 4)
#define FQL_SC_CONFIGS_ALL(X) \
  FQL_SC_CONFIGS_FP4(X, SC_MXFP4) FQL_SC_CONFIGS_ANY(X, SC_MXFP8) FQL_SC_CONFIGS_ANY(X, SC_FP8) \
  FQL_SC_CONFIGS_ANY(X, SC_FP8_BLOCK)

// (W, MT, NT, D) GEMV configurations built: 4 waves, one row tile with four
// (FP4) or two (8-bit) column tiles, two row tiles with two column tiles.
#define FQL_SCV_CONFIGS_FP4(X, F) X(F, 4, 1, 4, 3) X(F, 4, 2, 2, 3)
#define FQL_SCV_CONFIGS_FP8(X, F) X(F, 4, 1, 2, 3) X(F, 4, 2, 2, 3)
#define FQL_SCV_CONFIGS_ALL(X) \
  FQL_SCV_CONFIGS_FP4(X, SC_MXFP4) FQL_SCV_CONFIGS_FP8(X, SC_MXFP8) FQL_SCV_CONFIGS_FP8(X, SC_FP8) \
  FQL_SCV_CONFIGS_FP8(X, SC_FP8_BLOCK)

// The GEMV configurations also built with the activation quantized in the
// workgroup (FQ = 1): the one-row-tile decode defaults.
#define FQL_SCV_FUSED_CONFIGS_ALL(X) \
  X(SC_MXFP4, 4, 1, 4, 3) X(SC_MXFP8, 4, 1, 2, 3) X(SC_FP8, 4, 1, 2, 3) X(SC_FP8_BLOCK, 4, 1, 2, 3)

template <int F, int W, int MT, int NT, int D>
static constexpr bool scv_config_fits() {
  return sizeof(ScvStage<F, MT, NT>) * W * D <= 160 * 1024;
}

static bool scv_config_built(int fmt, int w, int mt, int nt, int d) {
#define FQL_X(F0, A, B, C, E) \
  if (fmt == F0 && w == A && mt == B && nt == C && d == E) return scv_config_fits<F0, A, B, C, E>();
  FQL_SCV_CONFIGS_ALL(FQL_X)
#undef FQL_X
  return false;
}

// Dynamic LDS of the fused GEMV (the compact activation operand, M rows), or
// 0 when the fused kernel is not built for this configuration or the operand
// and the weight ring do not fit in 160 KiB together.
static int64_t scv_fused_lds(int fmt, int w, int mt, int nt, int d, int64_t KC, int64_t M) {
  const int H = fmt == SC_MXFP4 ? 1 : 2;
  const int64_t dyn = KC * M * (H * 64 + 16);  // codes, then scales, rows 0 .. M-1
#define FQL_X(F0, A, B, C, E)                                                                     \
  if (fmt == F0 && w == A && mt == B && nt == C && d == E)                                         \
    return (int64_t)sizeof(ScvStage<F0, B, C, 1>) * A * E + dyn <= 160 * 1024 ? dyn : 0;
  FQL_SCV_FUSED_CONFIGS_ALL(FQL_X)
#undef FQL_X
  return 0;
}

static constexpr size_t kLdsLimit = 160 * 1024;

template <int F, int WM, int WN, int MTW, int NTW, int ST>
static constexpr bool sc_config_fits() {
  return sizeof(ScStage<F, WM, WN, MTW, NTW>) * ST + 16 <= kLdsLimit;
}

static bool sc_config_built(int fmt, int wm, int wn, int mtw, int ntw, int st) {
#define FQL_X(F0, A, B, C, D, E)                                                                 \
  if (fmt == F0 && wm == A && wn == B && mtw == C && ntw == D && st == E)                        \
    return sc_config_fits<F0, A, B, C, D, E>();
  FQL_SC_CONFIGS_ALL(FQL_X)
#undef FQL_X
  return false;
}

static const char* sc_fmt_name(int f) {
  return f == SC_MXFP4 ? "mxfp4" : f == SC_MXFP8 ? "mxfp8" : f == SC_FP8 ? "fp8" : "fp8_block";
}

ScPlan plan_sc_gemm(int fmt, int64_t M, int64_t N, int64_t K) {
  ScPlan p{};
  p.fmt = fmt;
  const ScDims w = sc_dims(fmt, N, K, true);
  const int64_t KC = w.KC, ntiles = w.rows_p / 16;
  const bool fp4 = fmt == SC_MXFP4;
  // defaults (MI355X sweeps at K = 4096, N = 14336, M = 1 .. 4096): one row
  // tile and two column tiles per wave for decode sizes (more workgroups in
  // flight), 64 x 128 workgroup tiles up to M = 128, 128 x 128 for 8-bit
  // formats up to M = 512, then the 8-wave tiles (256 x 256 for FP4, whose
  // ring fits in LDS; 256 x 128 for FP8).
  int wm = 1, wn = 4, mtw = 1, ntw = 2, st = 4;
  if (M <= 32) { wm = 1; wn = 4; mtw = 1; ntw = 2; st = 4; }
  else if (M <= 128 || (fp4 && M <= 512)) { wm = 1; wn = 4; mtw = 4; ntw = 2; st = 4; }
  else if (M <= 512) { wm = 2; wn = 2; mtw = 4; ntw = 4; st = 3; }
  else if (fp4) { wm = 2; wn = 4; mtw = 8; ntw = 4; st = 4; }
  else { wm = 4; wn = 2; mtw = 4; ntw = 4; st = 3; }
  // register-streaming GEMV for small M: W waves split K, NT tiles per workgroup
  {
    int gw = 0, gnt = 0, gd = 0;
    const int mt = (int)((M + 15) / 16);
    bool gemv = M <= 32;
    if (M <= 16) { gw = 4; gnt = fmt == SC_MXFP4 ? 4 : 2; gd = 3; }
    else { gw = 4; gnt = 2; gd = 3; }
    bool forced = false;
    int fq = -1;  // -1: fused when built and it fits
    const std::string gemv_spec = plan_override(kOverrideScGemv);
    const std::string gemm_spec = plan_override(kOverrideScGemm);
    if (!gemv_spec.empty()) {  // benchmarking aid: "W,NT,D[,FQ]" (0 = off)
      int a = 0, b = 0, c = 0, f = -1;
      const int k = std::sscanf(gemv_spec.c_str(), "%d,%d,%d,%d", &a, &b, &c, &f);
      if (k >= 1 && a == 0) gemv = false;
      else if (k >= 3 && M <= 64 && scv_config_built(fmt, a, mt, b, c)) {
        gemv = true; gw = a; gnt = b; gd = c; forced = true;
        if (k == 4) fq = f;
      }
    }
    if (!gemm_spec.empty()) gemv = forced;
    if (gemv && scv_config_built(fmt, gw, mt, gnt, gd)) {
      p.kind = 1;
      p.wm = 1; p.wn = gw; p.mtw = mt; p.ntw = gnt; p.st = gd;
      // decode sizes quantize the activation inside the workgroups (one launch)
      const int64_t dyn = M <= 16 && fq != 0 ? scv_fused_lds(fmt, gw, mt, gnt, gd, KC, M) : 0;
      p.fq = dyn > 0 ? 1 : 0;
      p.dyn_lds = dyn;
      p.Mp = 16 * mt;
      p.ngroups = (ntiles + gnt - 1) / gnt;
      p.groups = p.ngroups;
      p.splits = 1;
      p.kc_per_split = (int)KC;
      const ScDims x = sc_dims(fmt, p.Mp, K, false);
      p.xcode_bytes = round_up(x.code_bytes, 256);
      p.xscale_bytes = round_up(x.scale_bytes, 256);
      p.partial_bytes = 0;
      p.counter_bytes = 64 * 1024;
      p.total_bytes = p.counter_bytes + p.xcode_bytes + p.xscale_bytes;
      return p;
    }
  }
  int splits_override = 0, tail_override = 0;
  const std::string gemm_spec = plan_override(kOverrideScGemm);
  if (!gemm_spec.empty()) {  // benchmarking aid: "wm,wn,mtw,ntw,st,splits[,tail]"
    int a = 0, b = 0, c = 0, d = 0, f = 0, s = 0, t = 0;
    if (std::sscanf(gemm_spec.c_str(), "%d,%d,%d,%d,%d,%d,%d", &a, &b, &c, &d, &f, &s, &t) >= 5 &&
        sc_config_built(fmt, a, b, c, d, f)) {
      wm = a; wn = b; mtw = c; ntw = d; st = f; splits_override = s; tail_override = t;
    }
  }
  if (!sc_config_built(fmt, wm, wn, mtw, ntw, st)) { wm = 1; wn = 4; mtw = 1; ntw = 2; st = 4; }
  p.wm = wm; p.wn = wn; p.mtw = mtw; p.ntw = ntw; p.st = st;
  const int tile_rows = 16 * wm * mtw, tile_cols = 16 * wn * ntw;
  p.Mp = round_up(M, std::max(tile_rows, 16));
  p.ngroups = (ntiles * 16 + tile_cols - 1) / tile_cols;
  const int64_t groups = p.ngroups * (p.Mp / tile_rows);
  // split K until about 256 workgroups are in flight (at most 4 ways)
  int64_t s = std::max<int64_t>(1, std::min<int64_t>(std::min<int64_t>(4, KC), (256 + groups / 2) / groups));
  if (splits_override > 0) s = std::min<int64_t>(splits_override, KC);
  p.kc_per_split = (int)((KC + s - 1) / s);
  p.splits = (int)((KC + p.kc_per_split - 1) / p.kc_per_split);
  p.groups = groups;
  // The 8-wave tiles hold one workgroup per CU (their rings fill the LDS).
  // When their tiles leave the last round of the 256 CUs at most half full
  // and K is long (at least 64 chunks), that round's tiles are split along K
  // (up to 4 ways, through the split-K partial sums) instead. With short K
  // the partial sums cost more than the round saves: MXFP4 at M = 4096,
  // N = 14336, K = 4096 (896 tiles, 3.5 rounds, 32 chunks) took 180 us split
  // against 163 us whole. tail_override: 1 = never, 2..4 = that many ways.
  p.dp_groups = p.splits > 1 ? 0 : groups;
  if (p.splits == 1 && wm * wn == 8 && tail_override != 1 && groups >= 256) {
    const int64_t r = groups % 256;
    int64_t ts = r > 0 && r <= 128 && KC >= 64 ? std::min<int64_t>(4, 256 / r) : 1;
    if (tail_override >= 2 && tail_override <= 4 && r > 0) ts = tail_override;
    if (ts > 1 && KC >= 4 * ts) {
      p.dp_groups = groups - r;
      p.kc_per_split = (int)((KC + ts - 1) / ts);
      p.splits = (int)((KC + p.kc_per_split - 1) / p.kc_per_split);
    }
  }
  const ScDims x = sc_dims(fmt, p.Mp, K, false);
  p.xcode_bytes = round_up(x.code_bytes, 256);
  p.xscale_bytes = round_up(std::max<int64_t>(x.scale_bytes, 0), 256);
  const int64_t slab = (int64_t)p.splits * wm * wn * mtw * ntw * 64 * 16;
  p.partial_bytes = p.splits > 1 ? round_up((groups - p.dp_groups) * slab, 256) : 0;
  p.counter_bytes = 64 * 1024;
  p.total_bytes = p.counter_bytes + p.xcode_bytes + p.xscale_bytes + p.partial_bytes;
  return p;
}

std::string describe_sc_plan(const ScPlan& p) {
  char b[240];
  if (p.kind == 1 && p.fq) {
    std::snprintf(b, sizeof(b), "gemv_sc_kernel<%s,W=%d,MT=%d,NT=%d,D=%d,FQ=1> grid=%lld splits=1",
                  sc_fmt_name(p.fmt), p.wn, p.mtw, p.ntw, p.st, (long long)p.groups);
    return std::string(b);
  }
  if (p.kind == 1) {
    std::snprintf(b, sizeof(b), "sc_quant_operand_kernel<%s> + gemv_sc_kernel<%s,W=%d,MT=%d,NT=%d,D=%d> grid=%lld splits=1",
                  sc_fmt_name(p.fmt), sc_fmt_name(p.fmt), p.wn, p.mtw, p.ntw, p.st, (long long)p.groups);
    return std::string(b);
  }
  // whole tiles first; a split tail reads "tail=<tiles>x<splits>"
  const bool tail = p.dp_groups > 0 && p.splits > 1;
  const std::string extra =
      tail ? " tail=" + std::to_string(p.groups - p.dp_groups) + "x" + std::to_string(p.splits) : "";
  std::snprintf(b, sizeof(b),
                "sc_quant_operand_kernel<%s> + gemm_sc_kernel<%s,WM=%d,WN=%d,MTW=%d,NTW=%d,ST=%d> grid=%lld splits=%d%s",
                sc_fmt_name(p.fmt), sc_fmt_name(p.fmt), p.wm, p.wn, p.mtw, p.ntw, p.st,
                (long long)(p.dp_groups + (p.groups - p.dp_groups) * p.splits), tail ? 1 : p.splits,
                extra.c_str());
  return std::string(b);
}

template <int F, int WM, int WN, int MTW, int NTW, int ST>
static hipError_t launch_sc_t(const ScPlan& p, const uint8_t* xc, const uint8_t* xs,
                              const uint8_t* packed, const ScDims& w, int64_t M, int64_t N,
                              float alpha, const float* alpha_dev, const uint16_t* bias, uint16_t* y,
                              int64_t ldy, float4v* partial, uint32_t* counters, hipStream_t st) {
  if constexpr (!sc_config_fits<F, WM, WN, MTW, NTW, ST>()) {
    return hipErrorInvalidValue;
  } else {
    const int64_t grid = p.dp_groups + (p.groups - p.dp_groups) * p.splits;
    gemm_sc_kernel<F, WM, WN, MTW, NTW, ST><<<(unsigned)grid, 64 * WM * WN, 0, st>>>(
        xc, xs, packed, packed + w.code_bytes, (int)M, (int)N, w.KC, (int)(w.rows_p / 16), w.quads,
        (int)p.ngroups, p.kc_per_split, (int)p.dp_groups, p.splits, alpha, alpha_dev, bias, y, ldy,
        partial, counters);
    return hipGetLastError();
  }
}

template <int F, int W, int MT, int NT, int D>
static hipError_t launch_scv_t(const ScPlan& p, const uint8_t* xc, const uint8_t* xs,
                               const uint8_t* packed, const ScDims& w, int64_t M, int64_t N,
                               float alpha, const float* alpha_dev, const uint16_t* bias,
                               uint16_t* y, int64_t ldy, hipStream_t st) {
  if constexpr (!scv_config_fits<F, W, MT, NT, D>()) {
    return hipErrorInvalidValue;
  } else {
    gemv_sc_kernel<F, W, MT, NT, D, 0><<<(unsigned)p.groups, 64 * W, 0, st>>>(
        xc, xs, packed, packed + w.code_bytes, (int)M, (int)N, w.KC, (int)(w.rows_p / 16), w.quads,
        alpha, alpha_dev, bias, y, ldy, nullptr, 0, 0, 0.0f, 0);
    return hipGetLastError();
  }
}

template <int F, int W, int MT, int NT, int D>
static hipError_t launch_scv_fused_t(const ScPlan& p, const uint16_t* x, int64_t ldx, bool aligned,
                                     float inv_scale, int64_t K, const uint8_t* packed,
                                     const ScDims& w, int64_t M, int64_t N, float alpha,
                                     const float* alpha_dev, const uint16_t* bias, uint16_t* y,
                                     int64_t ldy, hipStream_t st) {
  if (p.dyn_lds <= 0 || M > 16 * MT) return hipErrorInvalidValue;
  gemv_sc_kernel<F, W, MT, NT, D, 1><<<(unsigned)p.groups, 64 * W, (size_t)p.dyn_lds, st>>>(
      nullptr, nullptr, packed, packed + w.code_bytes, (int)M, (int)N, w.KC, (int)(w.rows_p / 16),
      w.quads, alpha, alpha_dev, bias, y, ldy, x, ldx, aligned ? 1 : 0, inv_scale, K);
  return hipGetLastError();
}

hipError_t launch_sc_linear(const ScPlan& p, const uint16_t* x, int64_t M, int64_t K, int64_t ldx,
                            bool aligned, float inv_scale, const uint8_t* packed, int64_t N,
                            float alpha, const float* alpha_dev, const uint16_t* bias, uint16_t* y,
                            int64_t ldy, uint8_t* workspace, hipStream_t st) {
  const ScDims w = sc_dims(p.fmt, N, K, true);
  uint32_t* counters = reinterpret_cast<uint32_t*>(workspace);
  uint8_t* xc = workspace + p.counter_bytes;
  uint8_t* xs = xc + p.xcode_bytes;
  float4v* partial = reinterpret_cast<float4v*>(xs + p.xscale_bytes);
  if (p.splits > 1 && p.groups - p.dp_groups > p.counter_bytes / 4) return hipErrorInvalidValue;  // counter per split tile
  if (p.kind == 1 && p.fq) {
#define FQL_X(F0, A, B, C, E)                                                                      \
  if (p.fmt == F0 && p.wn == A && p.mtw == B && p.ntw == C && p.st == E)                           \
    return launch_scv_fused_t<F0, A, B, C, E>(p, x, ldx, aligned, inv_scale, K, packed, w, M, N,    \
                                              alpha, alpha_dev, bias, y, ldy, st);
    FQL_SCV_FUSED_CONFIGS_ALL(FQL_X)
#undef FQL_X
    return hipErrorInvalidValue;
  }
  hipError_t e = launch_sc_quant_operand(p.fmt, x, M, K, ldx, aligned, inv_scale, p.Mp, xc, xs, st);
  if (e != hipSuccess) return e;
  if (p.kind == 1) {
#define FQL_X(F0, A, B, C, E)                                                                      \
  if (p.fmt == F0 && p.wn == A && p.mtw == B && p.ntw == C && p.st == E)                           \
    return launch_scv_t<F0, A, B, C, E>(p, xc, xs, packed, w, M, N, alpha, alpha_dev, bias, y, ldy, \
                                        st);
    FQL_SCV_CONFIGS_ALL(FQL_X)
#undef FQL_X
    return hipErrorInvalidValue;
  }
#define FQL_X(F0, A, B, C, D, E)                                                                  \
  if (p.fmt == F0 && p.wm == A && p.wn == B && p.mtw == C && p.ntw == D && p.st == E)             \
    return launch_sc_t<F0, A, B, C, D, E>(p, xc, xs, packed, w, M, N, alpha, alpha_dev, bias, y, ldy, \
                                          partial, counters, st);
  FQL_SC_CONFIGS_ALL(FQL_X)
#undef FQL_X
  return hipErrorInvalidValue;
}

}  // namespace fql
