// Device helpers shared by the grouped expert GEMMs (gemm_big.hip, bf16 and
// MXFP4-dequantising; gemm_mxw.hip, MXFP4 codes in LDS):
// buffer resources and direct-to-LDS copies, the swizzled LDS row layouts,
// the block -> (expert, row tile, column tile, K split) map and the f32
// epilogue of the down projection.
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {
namespace gemm {

// Waves per block (4 = one per SIMD, 8 = two per SIMD), arranged 2 x NW/2.
#ifndef MOE_BIG_WAVES
#define MOE_BIG_WAVES 8
#endif
constexpr int kNW = MOE_BIG_WAVES;
constexpr int kNT = kNW * 64;

constexpr uint32_t kOOB = 0x80000000u;  // offset bit past every record count
constexpr uint32_t kRsrcFlags = 0x00020000u;

typedef __attribute__((address_space(3))) void lds_void;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void *base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)bytes,
                                           kRsrcFlags);
}

// Direct-to-LDS copies: lane i of the instruction writes bytes
// [16 i, 16 i + 16) (dma16) or [4 i, 4 i + 4) (dma4) of the run at lds_run.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint8_t *lds_run, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_run, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void dma4(__amdgpu_buffer_rsrc_t r, uint8_t *lds_run, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void *)lds_run, 4, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(N) with the other counters left alone (gfx9 encoding:
// vmcnt bits [3:0] and [15:14], expcnt [6:4], lgkmcnt [11:8]).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS tile rows, 16-B chunks swizzled so that the 16 consecutive rows read
// by one 16-lane pass of ds_read_b128 fall in 16 distinct groups of 4 banks:
//   512- and 256-B rows: chunk c of row r at c ^ (r % 16)
//   128-B rows: chunk c of row r at c ^ ((r / 2) % 8)
//    64-B rows: chunk c of row r at c ^ ((r / 4) % 4)
//    32-B rows: chunk c of row r at c ^ ((r / 8) % 2)
template <int ROWB>
__device__ __forceinline__ int swz_key(int row) {
  static_assert(ROWB == 512 || ROWB == 256 || ROWB == 128 || ROWB == 64 || ROWB == 32,
                "row bytes");
  if constexpr (ROWB >= 256) return row & 15;
  if constexpr (ROWB == 128) return (row >> 1) & 7;
  if constexpr (ROWB == 64) return (row >> 2) & 3;
  return (row >> 3) & 1;
}
template <int ROWB>
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * ROWB + ((chunk ^ swz_key<ROWB>(row)) << 4);
}
// Global chunk that lane `lane` of the 1 KB direct-to-LDS run `run` (rows
// run * 1024 / ROWB onwards) must fetch so that the run lands swizzled.
template <int ROWB>
__device__ __forceinline__ int run_chunk(int run, int lane) {
  constexpr int CPR = ROWB / 16, RPR = 1024 / ROWB;
  return (lane % CPR) ^ swz_key<ROWB>(run * RPR + lane / CPR);
}

// Global chunk a lane must fetch so that a 1 KB direct-to-LDS run of wave
// `wave` lands in the swizzled layout (run j of wave w is rows
// (kNW j + w) * 1024 / ROWB onwards; kNW is even, so the key depends on the
// wave's parity only).
template <int ROWB>
__device__ __forceinline__ int dma_chunk(int wave, int lane) {
  if constexpr (ROWB == 128) return (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
  return (lane & 3) ^ (lane >> 4);
}

// Where a block works: pile e, rows [row0, row0 + rows), column tile nt,
// work item (tile index * S + split), row-tile size bm.  Run by wave 0;
// e = -1 when the block has no work.  A pile of m rows has ceil(m / bm(m))
// row tiles, bm(m) given by the caller (a constant, or a choice by pile
// size).  Tiles are ordered expert-major, then column tile, then row tile,
// the S splits of a tile adjacent; the ordered list is cut into 8
// contiguous chunks, one per XCD (block b runs on XCD b mod 8), so the tiles
// that share an expert's weights share one L2.
struct TileSlot {
  int e, row0, rows, nt, item, bm;
  int split;  // K split of this block (item % its list's split count)
  int tail;   // LPT: the block is in the list of last row tiles
};

// LPT (longest first): the tile list is cut in two, the full row tiles of
// every pile (all but its last) and then the last row tile of each pile,
// which is the ragged one; each XCD gets a contiguous eighth of each list
// and runs its full tiles before its last tiles, so the short tiles fill the
// last round.  The grid needs 16 blocks beyond the tile count (each list's
// eighths round up separately).
// BAL (balanced rows): the ceil(m / bm) row tiles of a pile share its 32-row
// groups evenly (tile i takes groups [i G / t, (i + 1) G / t) of G), instead
// of bm-row tiles and a ragged last one, so that a pile's tiles take about
// the same time and the blocks running on an XCD stay in step through K.
// S1 (LPT only; 0 = S): K splits of each tile of the last-row-tile list, so
// that a tail round of few tiles can be spread over more blocks.
// RG (list 0 only; 0 = off): a pile's tiles are taken in groups of RG row
// tiles, column tile by column tile within a group, so that the blocks
// running together on an XCD share both the group's pile rows (across
// column tiles) and each column tile's weights (across the group's row
// tiles) in L2; without it a large pile's rows are streamed again for every
// column tile.
template <bool LPT = false, typename RowTile, bool BAL = false>
__device__ __forceinline__ void map_block_fn(const int32_t *offsets, int E, int n_tiles, int S,
                                             int lane, TileSlot *out, RowTile bm_of,
                                             std::integral_constant<bool, BAL> = {}, int S1 = 0,
                                             int RG = 0) {
  if (S1 <= 0) S1 = S;
  const int per = (E + MOE_WAVE - 1) / MOE_WAVE;
  const int eb = lane * per, ee = min(E, eb + per);
  // With one expert per lane (E <= 64) its offsets are loaded once.
  const int o0 = per == 1 && eb < E ? offsets[eb] : 0;
  const int o1 = per == 1 && eb < E ? offsets[eb + 1] : 0;
  auto tiles_of = [&](int m) { const int bm = bm_of(m); return (m + bm - 1) / bm; };
  // Row tiles of a pile in list 0 (LPT: all but the last) and list 1.
  auto in_list = [&](int te, bool last) {
    return LPT ? (last ? (te > 0 ? 1 : 0) : max(te - 1, 0)) : (last ? 0 : te);
  };
  int loc0 = 0, loc1 = 0;
  if (per == 1) {
    const int te = tiles_of(o1 - o0);
    loc0 = in_list(te, false);
    loc1 = in_list(te, true);
  } else {
    for (int x = eb; x < ee; ++x) {
      const int te = tiles_of(offsets[x + 1] - offsets[x]);
      loc0 += in_list(te, false);
      loc1 += in_list(te, true);
    }
  }
  const int incl0 = wave_incl_scan(loc0), incl1 = LPT ? wave_incl_scan(loc1) : 0;
  const int tot0 = __builtin_amdgcn_readlane(incl0, MOE_WAVE - 1) * n_tiles * S;
  const int tot1 = LPT ? __builtin_amdgcn_readlane(incl1, MOE_WAVE - 1) * n_tiles * S1 : 0;
  const int b = blockIdx.x;
  const int xcd = b & 7, slot = b >> 3;
  int base0 = 0, base1 = 0;
  for (int x = 0; x < xcd; ++x) {
    base0 += (tot0 - x + 7) >> 3;
    base1 += (tot1 - x + 7) >> 3;
  }
  const int cnt0 = (tot0 - xcd + 7) >> 3, cnt1 = (tot1 - xcd + 7) >> 3;
  if (slot >= cnt0 + cnt1) {
    if (lane == 0) out->e = -1;
    return;
  }
  const bool last = slot >= cnt0;
  const int item = last ? base1 + slot - cnt0 : base0 + slot;
  const int SS = last ? S1 : S;
  const int L = item / SS;
  if (lane == 0) {
    out->item = item;
    out->split = item % SS;
    out->tail = last ? 1 : 0;
  }
  const int incl = last ? incl1 : incl0, mine = last ? loc1 : loc0;
  const int lo = (incl - mine) * n_tiles, hi = incl * n_tiles;
  if (L >= lo && L < hi) {
    int acc = lo;
    for (int x = eb; x < ee; ++x) {
      const int ox = per == 1 ? o0 : offsets[x];
      const int m = (per == 1 ? o1 : offsets[x + 1]) - ox;
      const int bm = bm_of(m), te = (m + bm - 1) / bm, c = in_list(te, last);
      if (L < acc + c * n_tiles) {
        const int loc = L - acc;
        int mloc = last ? te - 1 : loc % c;
        out->e = x;
        out->nt = last ? loc : loc / c;
        if (RG > 0 && !last) {
          const int grp = loc / (RG * n_tiles), within = loc - grp * RG * n_tiles;
          const int gr = min(RG, c - grp * RG);  // row tiles in this group
          out->nt = within / gr;
          mloc = grp * RG + within % gr;
        }
        if constexpr (BAL) {
          const int G = (m + 31) / 32;
          const int g0 = (int)((long long)mloc * G / te), g1 = (int)((long long)(mloc + 1) * G / te);
          out->row0 = ox + 32 * g0;
          out->rows = min(m, 32 * g1) - 32 * g0;
        } else {
          out->row0 = ox + mloc * bm;
          out->rows = min(bm, m - mloc * bm);
        }
        out->bm = bm;
        break;
      }
      acc += c * n_tiles;
    }
  }
}

template <int BM, bool LPT = false, bool BAL = false>
__device__ __forceinline__ void map_block(const int32_t *offsets, int E, int n_tiles, int S,
                                          int lane, TileSlot *out, int S1 = 0, int RG = 0) {
  map_block_fn<LPT>(offsets, E, n_tiles, S, lane, out, [](int) { return BM; },
                    std::integral_constant<bool, BAL>{}, S1, RG);
}

// f32 stores of a block's accumulators: acc[tm][tn] of wave (wm, wn) holds
// pile row wm*WM + tm*32 + lane%32 and columns wn*WN + tn*32 + (i/4)*8 +
// (lane/32)*4 + i%4 (the MFMA takes the weight rows as its first operand),
// so each lane stores 16-B runs of four columns.  dst is [R][N] f32 (N a
// multiple of 8); rows past `rows` and columns past N are skipped.
template <int TM, int TN, int WM, int WN>
__device__ __forceinline__ void store_f32_tile(const f32x16 (&acc)[TM][TN], float *dst, int N,
                                               int row0, int rows, int n0, int wm, int wn,
                                               int lane) {
  const int lr = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int r = wm * WM + tm * 32 + lr;
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn * WN + tn * 32 + g * 8 + lg * 4;
        if (r < rows && col < N) {
          const f32x4 v = {acc[tm][tn][g * 4], acc[tm][tn][g * 4 + 1], acc[tm][tn][g * 4 + 2],
                           acc[tm][tn][g * 4 + 3]};
          *(f32x4 *)(dst + (size_t)(row0 + r) * N + col) = v;
        }
      }
  }
}

// Register epilogues: acc[tm][tn] holds pile row l % 32 of its 32-row group
// and columns (i/4)*8 + (l/32)*4 + i%4 of its 32-column group in lane l,
// element i (the MFMA takes the weight rows as its first operand).  Runs of
// lanes l and l + 32 are exchanged with v_permlane32_swap so that each lane
// stores 16-B pieces of eight consecutive columns; every store is issued
// (lanes outside the tile carry an offset past the record count).
// Four f32 pairs packed to bf16 (lo = columns 8g + 4lg + {0,1}, hi = +{2,3})
// for g = 2h, 2h+1 -> the 16-B piece of eight consecutive columns this lane
// stores.
__device__ __forceinline__ u32x4 swap_halves(uint32_t x_lo, uint32_t x_hi, uint32_t y_lo,
                                             uint32_t y_hi) {
  const auto lo = __builtin_amdgcn_permlane32_swap(x_lo, y_lo, false, false);
  const auto hi = __builtin_amdgcn_permlane32_swap(x_hi, y_hi, false, false);
  return u32x4{lo[0], hi[0], lo[1], hi[1]};
}

// Down: bf16 rows [0, rows) of a tile in ro (row pitch N bf16), each value
// the f32 result rounded once.
template <int TM, int TN, int WM, int WN>
__device__ __forceinline__ void store_bf16_regs(const f32x16 (&acc)[TM][TN],
                                                __amdgpu_buffer_rsrc_t ro, int N, int rows, int n0,
                                                int wm, int wn) {
  // (the lane id is read afresh: lane-derived values of the K loop are
  // not kept live across it for the epilogue)
  const int lane = __lane_id(), lr = lane & 31, lg = lane >> 5;
  const uint32_t rowoff = (uint32_t)(wm * WM + lr) * (uint32_t)N;  // row r's first element
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int r = wm * WM + tm * 32 + lr;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      uint32_t pk[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        pk[g][0] = pack_bf16x2(acc[tm][j][g * 4], acc[tm][j][g * 4 + 1]);
        pk[g][1] = pack_bf16x2(acc[tm][j][g * 4 + 2], acc[tm][j][g * 4 + 3]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 o = swap_halves(pk[2 * h][0], pk[2 * h][1], pk[2 * h + 1][0], pk[2 * h + 1][1]);
        const int col = n0 + wn * WN + j * 32 + 16 * h + lg * 8;
        const uint32_t off =
            (r < rows && col < N) ? (rowoff + (uint32_t)(tm * 32 * N) + col) * 2u : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(o, ro, off, 0, 0);
      }
    }
  }
}

// SwiGLU epilogue of an up tile with bf16 output: acc[tm][j] (j < TN/2) are
// the gate columns and acc[tm][j + TN/2] the matching value columns of the
// tile's OC outputs.  Values are staged through LDS (8-B writes of four
// columns) so that global stores are 16-B pieces of rows; the caller has
// made the stages free (barrier).  out is [R][N] bf16 with N % 8 == 0.
template <int TM, int TN, int WM, int WN, int BM, int OC, int NT = kNT>
__device__ __forceinline__ void store_swiglu_bf16_tile(const f32x16 (&acc)[TM][TN], uint8_t *smem,
                                                       uint16_t *out, int N, int row0, int rows,
                                                       int n0, int wm, int wn, int lane, int tid) {
  constexpr int PITCH = OC * 2 + 16;  // bytes per staged row (padded)
  const int lr = lane & 31, lg = lane >> 5;
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int r = wm * WM + tm * 32 + lr;
#pragma unroll
    for (int j = 0; j < TN / 2; ++j)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * (WN / 2) + j * 32 + g * 8 + lg * 4;
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) v[q] = silu(acc[tm][j][g * 4 + q]) * acc[tm][j + TN / 2][g * 4 + q];
        const u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
        *(u32x2 *)(smem + r * PITCH + col * 2) = pk;
      }
  }
  __syncthreads();
  constexpr int CH = OC / 8;  // 16-B chunks per row
  for (int idx = tid; idx < BM * CH; idx += NT) {
    const int r = idx / CH, ch = idx % CH;
    const int col = n0 + ch * 8;
    if (r < rows && col < N)  // N % 8 == 0: a chunk is all in or all out
      *(u32x4 *)(out + (size_t)(row0 + r) * N + col) = *(const u32x4 *)(smem + r * PITCH + ch * 16);
  }
}

}  // namespace gemm
}  // namespace moe
