// Large-tile grouped expert GEMMs for gfx950 (the prefill path of the
// expert FFN; see ffn.hip for the operation and its sources).
//
//   up:   H[r]  = silu(A[r] . W1_e^T) * (A[r] . W3_e^T)   (bf16 out)
//   down: Yp[r] = H[r] . W2_e^T                            (f32 out), or, when
//         every token has one expert, Y[tok(r)] = w(tok) * (H[r] . W2_e^T)
//         written straight into the layer output (combine fused).
//
// Block = 8 waves (two per SIMD, so one wave's MFMAs cover the other's
// barrier and LDS waits) arranged 2 x 4.  Block tile BM rows x BNB B-rows
// (the up kernel's B-rows are BNB/2 rows of W1 followed by the same BNB/2
// rows of W3, so each wave holds matching gate and value accumulators).
// Wave tile (BM/2) x (BNB/4) on v_mfma_f32_32x32x16_bf16.  At 256 x 256 the
// block moves 64 KB from L2 per 64-deep K step for 8.4 MFLOP, i.e. 32 B per
// clock per CU at the MFMA peak, about what L2 delivers to a CU: this tile
// size is the smallest that is not load-bound.
//
// bf16 operands reach LDS by direct buffer loads (buffer_load_dwordx4 ...
// lds): lane i of an instruction fills bytes [16 i, 16 i + 16) of a 1 KB run,
// so the global address each lane fetches is chosen to produce the swizzled
// layout (see swz()).  Loads past a buffer's record count return zero, which
// fills ragged rows and the K tail.  K advances by 64 through two LDS
// stages: one step of loads is in flight while the other is multiplied.
//
// Tiles are ordered expert-major, then N-tile, then M-tile, and the ordered
// list is cut into 8 contiguous chunks, one per XCD (workgroup i runs on XCD
// i mod 8), so the tiles that share an expert's weights share one L2.
//
// bf16 weights: big_gemm_kernel (K loop rotated against its barriers, see
// there).  Both kernels store their epilogues from registers.
// MXFP4 weights with K past what the GEMM with codes in LDS keeps
// (mxdq_gemm_kernel): 32 E2M1 codes and their E8M0 scale are converted to
// bf16 in registers (v_cvt_scalef32_pk_bf16_fp4) and written to LDS, so the
// MFMA loop is the same.
#include <atomic>
#include <type_traits>

#include "gemm_big.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace gemm;

constexpr int kBK = 64;  // K step of both kernels

template <int BM, int BNB, int BK>
struct Tile {
  static constexpr int WM = BM / 2, WN = BNB / (kNW / 2);
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int ROWB = BK * 2, CPR = BK / 8, RPR = 1024 / ROWB;
  static constexpr int A_BYTES = BM * ROWB, B_BYTES = BNB * ROWB;
  static constexpr int STAGE = A_BYTES + B_BYTES;
  static constexpr int A_RUNS = BM / RPR / kNW;  // 1 KB DMA runs per wave per stage
  static constexpr int B_RUNS = BNB / RPR / kNW;
  static constexpr int SLICES = BK / 16;
  static constexpr int MX_ALL = BNB * (BK / 32);               // (row, 32-K block) units
  static constexpr int MX_UNITS = (MX_ALL + kNT - 1) / kNT;      // per thread
};

// Row tiles per group in the tile order (map_block_fn RG): on the
// Mixtral-shaped up GEMM (7 row tiles per pile) groups of four cut the bytes
// fetched past L2 from 15.2 to 8.0 GB per launch and the kernel by 1%;
// groups of two were 3% slower.  Its down GEMM (6 full row tiles per pile,
// K = 14336) takes a pile's full row tiles in one group: 0.4% off the layer
// against groups of four (groups of two: 0.6% slower).
constexpr int kBigRowGroup = 4;
constexpr int kDownRowGroup = 8;

// ---- epilogues from registers ----------------------------------------------
// The MFMA takes the weight rows as its first operand, so accumulator
// element i of lane l is pile row l % 32 of the 32-row group and output
// column (i/4)*8 + (l/32)*4 + i%4 of the 32-column group: every lane holds
// runs of four consecutive columns of one row.  Two such runs of lanes l and
// l + 32 (columns 8h..8h+7 of a 16-column half h) are exchanged with
// v_permlane32_swap so that lane l stores columns 16h..16h+7 and lane l + 32
// columns 16h+8..16h+15, as 16-B stores.  Every store is issued (lanes
// outside the tile carry an offset past the record count), so an epilogue
// issues a fixed number of vector memory operations per wave.

// s_waitcnt lgkmcnt(0) with the other counters left alone.
__device__ __forceinline__ void lgkm_wait0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}

// Up: H rows [row0, row0 + rows) in ro (row pitch N bf16) = silu(gate) * value,
// gate = acc[tm][j], value = acc[tm][j + TN/2].  TM * TN stores per wave.
template <int TM, int TN, int WM, int WN>
__device__ __forceinline__ void store_swiglu_regs(const f32x16 (&acc)[TM][TN],
                                                  __amdgpu_buffer_rsrc_t ro, int N, int rows,
                                                  int n0, int wm, int wn) {
  // (the lane id is read afresh: lane-derived values of the K loop are
  // not kept live across it for the epilogue)
  const int lane = __lane_id(), lr = lane & 31, lg = lane >> 5;
  const uint32_t rowoff = (uint32_t)(wm * WM + lr) * (uint32_t)N;  // row r's first element
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int r = wm * WM + tm * 32 + lr;
#pragma unroll
    for (int j = 0; j < TN / 2; ++j) {
      uint32_t pk[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float v[4];
#pragma unroll
        for (int q = 0; q < 4; ++q)
          v[q] = silu(acc[tm][j][g * 4 + q]) * acc[tm][j + TN / 2][g * 4 + q];
        pk[g][0] = pack_bf16x2(v[0], v[1]);
        pk[g][1] = pack_bf16x2(v[2], v[3]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 o = swap_halves(pk[2 * h][0], pk[2 * h][1], pk[2 * h + 1][0], pk[2 * h + 1][1]);
        const int col = n0 + wn * (WN / 2) + j * 32 + 16 * h + lg * 8;
        const uint32_t off =
            (r < rows && col < N) ? (rowoff + (uint32_t)(tm * 32 * N) + col) * 2u : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(o, ro, off, 0, 0);
      }
    }
  }
}

// Down: f32 rows [0, rows) of a tile in ro (row pitch N floats), 16-B stores
// of four columns.  TM * TN * 4 stores per wave.
template <int TM, int TN, int WM, int WN>
__device__ __forceinline__ void store_f32_regs(const f32x16 (&acc)[TM][TN],
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
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = n0 + wn * WN + tn * 32 + g * 8 + lg * 4;
        const uint32_t off =
            (r < rows && col < N) ? (rowoff + (uint32_t)(tm * 32 * N) + col) * 4u : kOOB;
        const f32x4 v = {acc[tm][tn][g * 4], acc[tm][tn][g * 4 + 1], acc[tm][tn][g * 4 + 2],
                         acc[tm][tn][g * 4 + 3]};
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), ro, off, 0, 0);
      }
  }
}

// Down with the combine fused (one expert per token): y[token] = w(token) *
// row, bf16, in ro = the layer output (row pitch N bf16).
template <int TM, int TN, int WM, int WN>
__device__ __forceinline__ void store_scaled_rows_regs(const f32x16 (&acc)[TM][TN],
                                                       __amdgpu_buffer_rsrc_t ro, int N,
                                                       const int32_t *perm_out,
                                                       const float *comb_w, int row0, int rows,
                                                       int n0, int wm, int wn) {
  const int lane = __lane_id(), lr = lane & 31, lg = lane >> 5;
  int tok[TM];
  float scale[TM];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) tok[tm] = perm_out[row0 + min(wm * WM + tm * 32 + lr, rows - 1)];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) scale[tm] = comb_w[tok[tm]];
#pragma unroll
  for (int tm = 0; tm < TM; ++tm) {
    const int r = wm * WM + tm * 32 + lr;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
      uint32_t pk[4][2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        pk[g][0] = pack_bf16x2(acc[tm][j][g * 4] * scale[tm], acc[tm][j][g * 4 + 1] * scale[tm]);
        pk[g][1] = pack_bf16x2(acc[tm][j][g * 4 + 2] * scale[tm], acc[tm][j][g * 4 + 3] * scale[tm]);
      }
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const u32x4 o = swap_halves(pk[2 * h][0], pk[2 * h][1], pk[2 * h + 1][0], pk[2 * h + 1][1]);
        const int col = n0 + wn * WN + j * 32 + 16 * h + lg * 8;
        const uint32_t off =
            (r < rows && col < N) ? ((uint32_t)tok[tm] * (uint32_t)N + col) * 2u : kOOB;
        __builtin_amdgcn_raw_buffer_store_b128(o, ro, off, 0, 0);
      }
    }
  }
}

// ---- bf16 weights ------------------------------------------------------------
// One K step is SLICES MFMA k-slices of 16.  The K loop is rotated by one
// slice against the barriers: after the barrier that publishes stage s + 1,
// a wave reads its fragments of slice 0 of s + 1 and then runs the MFMAs of
// the last slice of step s, whose fragments it read before the barrier, so
// the LDS latency after a barrier is covered by MFMAs instead of stalling
// both waves of a SIMD; then it issues the copies of step s + 2 into the
// stage every wave has just finished.  Scheduling groups pin the order
// "MFMA, LDS read, MFMA, LDS read, ..." inside a slice, and slices do not
// mix.  The last step is peeled off the loop, so the loop body has no
// branch: with one, the compiler's LDS counter at the join made the
// slice-3 MFMAs wait for the new reads.
//
// ACT (a compile-time count) is the number of this wave's 32-row groups that
// hold pile rows: the last row tile of a pile is usually ragged, and its
// empty groups are neither read from LDS nor multiplied.  A wave with
// ACT = 0 still issues its share of the copies and meets every barrier.
//
// LPT: longest-first tile order (map_block_fn), for unsplit down GEMMs of
// three or more rounds of blocks, where the ragged last row tiles then fill
// the last round.  FUSE is the combine-fused down pass.
template <bool UP, bool GATHER, bool FUSE, int BM, int BNB, bool LPT>
__global__ __launch_bounds__(kNT, 1) void big_gemm_kernel(BigGemmParams p) {
  constexpr int BK = kBK;
  using T = Tile<BM, BNB, BK>;
  static_assert(!(UP && FUSE), "the fused combine is a down epilogue");
  static_assert(T::SLICES % 2 == 0, "slices alternate between two fragment buffers");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ TileSlot s_t;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA bases
  const int N = p.N, K = p.K;
  const int S = UP ? 1 : (p.splits > 1 ? p.splits : 1);

  // ---- block -> tile ------------------------------------------------------
  // The up projection takes balanced row tiles: a pile's blocks then take
  // about the same time, and the blocks of an XCD that share operands stay
  // closer in K (measured: L2 hit rate 45% -> 50% on the Mixtral-shaped up).
  const int S1 = (LPT && !UP && p.tail_splits > 1) ? p.tail_splits : S;
  if (wave == 0)
    map_block<BM, LPT, UP>(p.offsets, p.E, p.n_tiles, S, lane, &s_t, S1,
                           UP ? kBigRowGroup : kDownRowGroup);
  __syncthreads();
  const int e = s_t.e;
  if (e < 0) return;
  const int row0 = s_t.row0, rows = s_t.rows;
  const int n0 = s_t.nt * (UP ? BNB / 2 : BNB);
  const int split = s_t.split;
  const bool tail_split = LPT && !UP && S1 > 1 && s_t.tail;
  // K range of this block: [kbeg, kend), a whole multiple of BK but the end.
  const int kbeg = S > 1 ? split * p.ksplit : (tail_split ? split * p.tail_ksplit : 0);
  const int kend = S > 1 ? min(K, kbeg + p.ksplit) : (tail_split ? min(K, kbeg + p.tail_ksplit) : K);
  const int nk = (kend - kbeg + BK - 1) / BK;

  // ---- per-lane DMA offsets -----------------------------------------------
  // Run j of wave w fills LDS chunks q = (8 j + w) * 64 + lane, i.e. row
  // rbase + j * RUN_ROWS (rbase = w * RPR + lane / CPR < RUN_ROWS), stored
  // chunk lane % CPR, which must hold global chunk c = stored ^ key(row)
  // (the same for every run of a wave).  Valid offsets are < 2^31 (checked
  // on the host); an invalid row carries bit 31 and the K tail ORs it in, so
  // such lanes read zeros.
  constexpr int RUN_ROWS = kNW * T::RPR;
  const int c = dma_chunk<BK * 2>(wave, lane);
  const int rbase = wave * T::RPR + lane / T::CPR;
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.a, p.a_bytes);
  // A rows: one offset per run when gathered (the pile-row -> token loads are
  // issued together, the row index clamped into the tile so that every load
  // is in bounds), else the first run's offset (run j is RUN_ROWS rows
  // further); B rows: the first run's offset (likewise).
  uint32_t a_off[GATHER ? T::A_RUNS : 1];
  if constexpr (GATHER) {
    int a_src[T::A_RUNS];
#pragma unroll
    for (int j = 0; j < T::A_RUNS; ++j) a_src[j] = p.perm[row0 + min(rbase + j * RUN_ROWS, rows - 1)];
#pragma unroll
    for (int j = 0; j < T::A_RUNS; ++j)
      a_off[j] = rbase + j * RUN_ROWS < rows
                     ? ((uint32_t)a_src[j] * (uint32_t)K + (uint32_t)c * 8u) * 2u
                     : kOOB;
  } else {
    a_off[0] = ((uint32_t)(row0 + rbase) * (uint32_t)K + (uint32_t)c * 8u) * 2u;
  }
  const int pe = phys_slot(p.slot, p.n_slots, e);  // physical weight slot
  const size_t mat_elems = (size_t)N * K;
  const __amdgpu_buffer_rsrc_t rb0 =
      rsrc((const uint16_t *)p.b0 + (size_t)pe * mat_elems, (uint32_t)(mat_elems * 2));
  const __amdgpu_buffer_rsrc_t rb1 =
      UP ? rsrc((const uint16_t *)p.b1 + (size_t)pe * mat_elems, (uint32_t)(mat_elems * 2)) : rb0;
  const uint32_t b_off0 = ((uint32_t)(n0 + rbase) * (uint32_t)K + (uint32_t)c * 8u) * 2u;
  const int b_lim = N - n0;  // valid B rows: rbase + j * RUN_ROWS < b_lim
  static_assert(!UP || (BNB / 2) % RUN_ROWS == 0, "W1/W3 halves of whole runs");

  // Copies of K step kt into LDS stage `stage` (a step past the end issues
  // zero loads).
  auto issue = [&](int kt, int stage) {
    const int k0 = kbeg + kt * BK;
    const uint32_t kpen = (k0 + c * 8 < kend) ? 0u : kOOB;
    const uint32_t k0b = (uint32_t)k0 * 2u;
    const uint32_t rstep = (uint32_t)RUN_ROWS * (uint32_t)K * 2u;  // bytes per run of rows
    uint8_t *sa = smem + stage * T::STAGE;
    uint8_t *sb = sa + T::A_BYTES;
#pragma unroll
    for (int j = 0; j < T::A_RUNS; ++j) {
      const uint32_t off =
          GATHER ? a_off[j] : (rbase + j * RUN_ROWS < rows ? a_off[0] + j * rstep : kOOB);
      dma16(ra, sa + (kNW * j + wave) * 1024, (off + k0b) | kpen);
    }
#pragma unroll
    for (int j = 0; j < T::B_RUNS; ++j) {
      const bool second = UP && j * RUN_ROWS >= BNB / 2;
      const int jj = UP ? (j * RUN_ROWS) % (BNB / 2) / RUN_ROWS : j;  // run within W1 or W3
      const uint32_t off = rbase + jj * RUN_ROWS < b_lim ? b_off0 + jj * rstep : kOOB;
      dma16(second ? rb1 : rb0, sb + (kNW * j + wave) * 1024, (off + k0b) | kpen);
    }
  };

  const int wm = wave / (kNW / 2), wn = wave % (kNW / 2);
  const int lr = lane & 31, lg = lane >> 5;
  f32x16 acc[T::TM][T::TN];
#pragma unroll
  for (int a = 0; a < T::TM; ++a)
#pragma unroll
    for (int b = 0; b < T::TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  // B-row of wave-subtile j: up = gate rows then the matching value rows.
  auto brow = [&](int j) {
    if (UP)
      return j < T::TN / 2 ? wn * (T::WN / 2) + j * 32 + lr
                           : BNB / 2 + wn * (T::WN / 2) + (j - T::TN / 2) * 32 + lr;
    return wn * T::WN + j * 32 + lr;
  };
  auto read_frags = [&](auto actc, const uint8_t *sa, int kk, bf16x8 *af, bf16x8 *bfr) {
    constexpr int ACT = decltype(actc)::value;
    const uint8_t *sb = sa + T::A_BYTES;
    const int ch = kk * 2 + lg;
#pragma unroll
    for (int tm = 0; tm < ACT; ++tm)
      af[tm] = *(const bf16x8 *)(sa + swz<BK * 2>(wm * T::WM + tm * 32 + lr, ch));
    if constexpr (ACT > 0) {
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn) bfr[tn] = *(const bf16x8 *)(sb + swz<BK * 2>(brow(tn), ch));
    }
  };
  auto mfmas = [&](auto actc, const bf16x8 *af, const bf16x8 *bfr) {
    constexpr int ACT = decltype(actc)::value;
#pragma unroll
    for (int tm = 0; tm < ACT; ++tm)
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[tn], af[tm], acc[tm][tn], 0, 0, 0);
  };

  auto kloop = [&](auto actc) {
    constexpr int ACT = decltype(actc)::value;
    constexpr int NF = ACT > 0 ? ACT + T::TN : 0;  // fragment reads per slice
    constexpr int NM = ACT * T::TN;                // MFMAs per slice
    wait_vmcnt<0>();
    __syncthreads();
    bf16x8 a0[T::TM], b0[T::TN], a1[T::TM], b1[T::TN];
    read_frags(actc, smem, 0, a0, b0);
    issue(1, 1);
    __builtin_amdgcn_sched_barrier(0);
    // Slices 0 .. SLICES-2 of the step in stage st: each reads the next
    // slice's fragments while its MFMAs run.
    auto slices = [&](int st) {
      const uint8_t *sa = smem + st * T::STAGE;
#pragma unroll
      for (int kk = 0; kk + 1 < T::SLICES; ++kk) {
        bf16x8 *ac = (kk & 1) ? a1 : a0, *bc = (kk & 1) ? b1 : b0;
        bf16x8 *an = (kk & 1) ? a0 : a1, *bn = (kk & 1) ? b0 : b1;
        read_frags(actc, sa, kk + 1, an, bn);
        mfmas(actc, ac, bc);
#pragma unroll
        for (int i = 0; i < NM; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          if (i < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_barrier(0);
      }
    };
    for (int kt = 0; kt + 1 < nk; ++kt) {
      const int st = kt & 1;
      slices(st);
      // This stage's copies have landed and slice 3's fragments are in
      // registers on every wave before anyone copies into this stage again.
      wait_vmcnt<0>();
      lgkm_wait0();
      __syncthreads();
      // Slice 0 of step kt + 1, read while the MFMAs of slice 3 run.
      read_frags(actc, smem + (st ^ 1) * T::STAGE, 0, a0, b0);
      mfmas(actc, a1, b1);
#pragma unroll
      for (int i = 0; i < NF; ++i) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
#pragma unroll
      for (int i = 0; i < NM; ++i) __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_barrier(0);
      issue(kt + 2, st);
    }
    slices((nk - 1) & 1);
    mfmas(actc, a1, b1);
  };
  issue(0, 0);
  const int act = __builtin_amdgcn_readfirstlane(min(T::TM, max(0, (rows - wm * T::WM + 31) / 32)));
  static_assert(T::TM >= 2 && T::TM <= 5, "row groups per wave");
  if (act == T::TM) {
    kloop(std::integral_constant<int, T::TM>{});
  } else if (act == 0) {
    kloop(std::integral_constant<int, 0>{});
  } else if (act == 1) {
    kloop(std::integral_constant<int, 1>{});
  } else if constexpr (T::TM >= 3) {
    if (act == 2) {
      kloop(std::integral_constant<int, 2>{});
    } else if constexpr (T::TM >= 4) {
      if (act == 3) {
        kloop(std::integral_constant<int, 3>{});
      } else if constexpr (T::TM >= 5) {
        kloop(std::integral_constant<int, 4>{});
      }
    }
  }

  // ---- epilogue (stores from registers) --------------------------------------
  if constexpr (UP) {
    store_swiglu_regs<T::TM, T::TN, T::WM, T::WN>(
        acc, rsrc((uint16_t *)p.out + (size_t)row0 * N, (uint32_t)rows * (uint32_t)N * 2u), N, rows,
        n0, wm, wn);
  } else if constexpr (FUSE) {
    store_scaled_rows_regs<T::TM, T::TN, T::WM, T::WN>(
        acc, rsrc(p.out, (uint32_t)p.fuse_rows * (uint32_t)N * 2u), N, p.perm_out, p.comb_w, row0,
        rows, n0, wm, wn);
  } else if (p.out_bf16 && !tail_split && S == 1) {
    // bf16 pile outputs.
    store_bf16_regs<T::TM, T::TN, T::WM, T::WN>(
        acc, rsrc((uint16_t *)p.out + (size_t)row0 * N, (uint32_t)rows * (uint32_t)N * 2u), N, rows,
        n0, wm, wn);
  } else {
    // Tail split: this split's partial sums of the pile's last row tile,
    // compactly at row e * BM + (pile row - row0) of plane `split`; split K:
    // plane `split` of the partial sums, added later in split order; else
    // the f32 pile outputs.
    float *dst = tail_split ? p.tail_part + (size_t)split * p.tail_plane + (size_t)e * BM * N
                            : (S > 1 ? p.part + (size_t)split * p.R * N : (float *)p.out) +
                                  (size_t)row0 * N;
    store_f32_regs<T::TM, T::TN, T::WM, T::WN>(
        acc, rsrc(dst, (uint32_t)rows * (uint32_t)N * 4u), N, rows, n0, wm, wn);
  }
}

// ---- MXFP4 weights, dequantised in registers ---------------------------------
// Each thread owns (B-row, 32-K block) units u = tid + kNT i; their codes
// and scales are loaded into registers one step ahead of the activation
// copies (two register slots, by step parity), so a load has about two
// steps of compute to land before it is converted into the B tile of the
// stage.  One tile per block.
template <bool UP, bool GATHER, bool FUSE, int BM, int BNB>
__global__ __launch_bounds__(kNT, 1) void mxdq_gemm_kernel(BigGemmParams p) {
  constexpr int BK = kBK, NST = 2;
  using T = Tile<BM, BNB, BK>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ TileSlot s_t;

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // uniform: LDS DMA bases
  const int N = p.N, K = p.K;
  const int S = UP ? 1 : (p.splits > 1 ? p.splits : 1);

  if (wave == 0) map_block<BM, false, UP>(p.offsets, p.E, p.n_tiles, S, lane, &s_t, S, kBigRowGroup);
  __syncthreads();
  const int e = s_t.e;
  if (e < 0) return;
  const int row0 = s_t.row0, rows = s_t.rows;
  const int n0 = s_t.nt * (UP ? BNB / 2 : BNB);
  const int split = s_t.split;
  const int kbeg = S > 1 ? split * p.ksplit : 0;
  const int kend = S > 1 ? min(K, kbeg + p.ksplit) : K;

  const int c = dma_chunk<BK * 2>(wave, lane);
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.a, p.a_bytes);
  uint32_t a_off[T::A_RUNS];
  int a_src[T::A_RUNS];
#pragma unroll
  for (int j = 0; j < T::A_RUNS; ++j) {
    const int r = (kNW * j + wave) * T::RPR + lane / T::CPR;
    a_src[j] = GATHER ? p.perm[row0 + min(r, rows - 1)] : row0 + r;
  }
#pragma unroll
  for (int j = 0; j < T::A_RUNS; ++j) {
    const int r = (kNW * j + wave) * T::RPR + lane / T::CPR;
    a_off[j] = r < rows ? ((uint32_t)a_src[j] * (uint32_t)K + (uint32_t)c * 8u) * 2u : kOOB;
  }
  const int pe = phys_slot(p.slot, p.n_slots, e);  // physical weight slot
  // Codes and scales read with buffer loads (32-bit offsets; an invalid unit
  // carries kOOB and reads zeros).  Whether a unit is in W1 or W3 (up)
  // depends on its wave only.
  const size_t qn = (size_t)N * (K / 2), sn = (size_t)N * (K / 32);
  const __amdgpu_buffer_rsrc_t rq0 = rsrc((const uint8_t *)p.b0 + (size_t)pe * qn, (uint32_t)qn);
  const __amdgpu_buffer_rsrc_t rs0 = rsrc(p.s0 + (size_t)pe * sn, (uint32_t)sn);
  const __amdgpu_buffer_rsrc_t rq1 =
      UP ? rsrc((const uint8_t *)p.b1 + (size_t)pe * qn, (uint32_t)qn) : rq0;
  const __amdgpu_buffer_rsrc_t rs1 = UP ? rsrc(p.s1 + (size_t)pe * sn, (uint32_t)sn) : rs0;
  uint32_t q_off[T::MX_UNITS], s_off[T::MX_UNITS];
#pragma unroll
  for (int i = 0; i < T::MX_UNITS; ++i) {
    const int u = tid + kNT * i;
    const int br = u / (BK / 32), half = u % (BK / 32);
    const int n = UP ? n0 + (br % (BNB / 2)) : n0 + br;
    const bool ok = n < N && u < T::MX_ALL;
    q_off[i] = ok ? (uint32_t)n * (uint32_t)(K / 2) + half * 16u : kOOB;
    s_off[i] = ok ? (uint32_t)n * (uint32_t)(K / 32) + half : kOOB;
  }
  u32x4 mq[2][T::MX_UNITS];
  uint32_t ms[2][T::MX_UNITS];
  auto load_b = [&](int kt, u32x4 *q, uint32_t *sv) {
    const int k0 = kbeg + kt * BK;
#pragma unroll
    for (int i = 0; i < T::MX_UNITS; ++i) {
      const int half = (tid + kNT * i) % (BK / 32);
      const uint32_t pen = (k0 + half * 32 < kend) ? 0u : kOOB;
      // Units u >= (BNB / 2) * (BK / 32) (a multiple of 64) are W3 rows, so
      // the choice follows the wave index (uniform: one buffer resource).
      static_assert((BNB / 2) * (BK / 32) % 64 == 0, "W1/W3 split at a wave boundary");
      const bool second = UP && (wave * 64 + kNT * i) >= (BNB / 2) * (BK / 32);
      q[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                            second ? rq1 : rq0, (q_off[i] + k0 / 2) | pen, 0, 0));
      sv[i] = __builtin_amdgcn_raw_buffer_load_b8(second ? rs1 : rs0, (s_off[i] + k0 / 32) | pen, 0, 0);
    }
  };
  // Copies of activation step kt into stage `stage`, then the register loads
  // of weight step kt + 1 into slot SL (a compile-time index: the K loop is
  // unrolled by two).
  auto issue = [&](int kt, int stage, auto slc) {
    constexpr int SL = decltype(slc)::value;
    const int k0 = kbeg + kt * BK;
    const uint32_t kpen = (k0 + c * 8 < kend) ? 0u : kOOB;
    const uint32_t k0b = (uint32_t)k0 * 2u;
    uint8_t *sa = smem + stage * T::STAGE;
#pragma unroll
    for (int j = 0; j < T::A_RUNS; ++j) dma16(ra, sa + (kNW * j + wave) * 1024, (a_off[j] + k0b) | kpen);
    load_b(kt + 1, mq[SL], ms[SL]);
  };
  // Convert the codes of one step (a register slot) into the B tile of a stage.
  auto store_slot = [&](int stage, const u32x4 *mqs, const uint32_t *mss) {
    uint8_t *sb = smem + stage * T::STAGE + T::A_BYTES;
#pragma unroll
    for (int i = 0; i < T::MX_UNITS; ++i) {
      const int u = tid + kNT * i;
      if (T::MX_ALL % kNT != 0 && u >= T::MX_ALL) continue;
      const int br = u / (BK / 32), half = u % (BK / 32);
      const float sc = e8m0_to_f32(mss[i]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t wv = mqs[i][q];
        const bf16x2 p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 0);
        const bf16x2 p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 1);
        const bf16x2 p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 2);
        const bf16x2 p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 3);
        const u32x4 o = {__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1),
                         __builtin_bit_cast(uint32_t, p2), __builtin_bit_cast(uint32_t, p3)};
        *(u32x4 *)(sb + swz<BK * 2>(br, half * 4 + q)) = o;
      }
    }
  };

  const int wm = wave / (kNW / 2), wn = wave % (kNW / 2);
  const int lr = lane & 31, lg = lane >> 5;
  f32x16 acc[T::TM][T::TN];
#pragma unroll
  for (int a = 0; a < T::TM; ++a)
#pragma unroll
    for (int b = 0; b < T::TN; ++b)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[a][b][i] = 0.f;

  auto brow = [&](int j) {
    if (UP)
      return j < T::TN / 2 ? wn * (T::WN / 2) + j * 32 + lr
                           : BNB / 2 + wn * (T::WN / 2) + (j - T::TN / 2) * 32 + lr;
    return wn * T::WN + j * 32 + lr;
  };
  auto read_frags = [&](auto actc, const uint8_t *sa, const uint8_t *sb, int kk, bf16x8 *af,
                        bf16x8 *bfr) {
    constexpr int ACT = decltype(actc)::value;
    const int ch = kk * 2 + lg;
#pragma unroll
    for (int tm = 0; tm < ACT; ++tm)
      af[tm] = *(const bf16x8 *)(sa + swz<BK * 2>(wm * T::WM + tm * 32 + lr, ch));
    if constexpr (ACT > 0) {
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn) bfr[tn] = *(const bf16x8 *)(sb + swz<BK * 2>(brow(tn), ch));
    }
  };
  auto mfmas = [&](auto actc, const bf16x8 *af, const bf16x8 *bfr) {
    constexpr int ACT = decltype(actc)::value;
#pragma unroll
    for (int tm = 0; tm < ACT; ++tm)
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn)
        acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[tn], af[tm], acc[tm][tn], 0, 0, 0);
  };
  constexpr int NV = T::A_RUNS;  // DMA issues per step
  auto step = [&](auto actc, int stage, int kt_issue, int stage_issue, auto slc) {
    constexpr int ACT = decltype(actc)::value;
    constexpr int NF = ACT > 0 ? ACT + T::TN : 0;
    constexpr int NM = ACT * T::TN;
    const uint8_t *sa = smem + stage * T::STAGE;
    const uint8_t *sb = sa + T::A_BYTES;
    bf16x8 a0[T::TM], b0[T::TN], a1[T::TM], b1[T::TN];
    read_frags(actc, sa, sb, 0, a0, b0);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < T::SLICES; ++kk) {
      bf16x8 *ac = (kk & 1) ? a1 : a0, *bc = (kk & 1) ? b1 : b0;
      bf16x8 *an = (kk & 1) ? a0 : a1, *bn = (kk & 1) ? b0 : b1;
      if (kk + 1 < T::SLICES) read_frags(actc, sa, sb, kk + 1, an, bn);
      if (kk == 0) issue(kt_issue, stage_issue, slc);
      mfmas(actc, ac, bc);
#pragma unroll
      for (int i = 0; i < NM; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        if (kk + 1 < T::SLICES && i < NF) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        if (kk == 0 && i < NV) __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  const int nk = (kend - kbeg + BK - 1) / BK;
  // Step kt (parity P = kt & 1): its copies are done once only the register
  // loads of the following step are pending; it issues step kt + 1 (and the
  // registers of step kt + 2, slot P) and converts step kt + 1 (slot 1 - P).
  auto kstep = [&](auto actc, int kt, auto parc) {
    constexpr int P = decltype(parc)::value;
    wait_vmcnt<2 * T::MX_UNITS>();
    __syncthreads();
    step(actc, kt % NST, kt + 1, (kt + 1) % NST, parc);
    if (kt + 1 < nk) store_slot((kt + 1) % NST, mq[1 - P], ms[1 - P]);
  };
  auto kloop = [&](auto actc) {
    for (int kt = 0; kt < nk; kt += 2) {
      kstep(actc, kt, std::integral_constant<int, 0>{});
      if (kt + 1 < nk) kstep(actc, kt + 1, std::integral_constant<int, 1>{});
    }
  };
  load_b(0, mq[0], ms[0]);
  issue(0, 0, std::integral_constant<int, 1>{});
  store_slot(0, mq[0], ms[0]);
  const int act = __builtin_amdgcn_readfirstlane(min(T::TM, max(0, (rows - wm * T::WM + 31) / 32)));
  static_assert(T::TM >= 2 && T::TM <= 4, "row groups per wave");
  if (act == T::TM) {
    kloop(std::integral_constant<int, T::TM>{});
  } else if (act == 0) {
    kloop(std::integral_constant<int, 0>{});
  } else if (act == 1) {
    kloop(std::integral_constant<int, 1>{});
  } else if constexpr (T::TM >= 3) {
    if (act == 2) {
      kloop(std::integral_constant<int, 2>{});
    } else if constexpr (T::TM >= 4) {
      kloop(std::integral_constant<int, 3>{});
    }
  }
  wait_vmcnt<0>();

  if constexpr (!UP) {
    if (S > 1) {
      // Split K: this block's partial sums go to plane `split`; a later
      // kernel adds the planes in split order.
      store_f32_regs<T::TM, T::TN, T::WM, T::WN>(
          acc, rsrc(p.part + (size_t)split * p.R * N + (size_t)row0 * N, (uint32_t)rows * N * 4u), N,
          rows, n0, wm, wn);
      return;
    }
  }
  if constexpr (UP) {
    store_swiglu_regs<T::TM, T::TN, T::WM, T::WN>(
        acc, rsrc((uint16_t *)p.out + (size_t)row0 * N, (uint32_t)rows * N * 2u), N, rows, n0, wm,
        wn);
  } else if constexpr (FUSE) {
    store_scaled_rows_regs<T::TM, T::TN, T::WM, T::WN>(
        acc, rsrc(p.out, (uint32_t)p.fuse_rows * (uint32_t)N * 2u), N, p.perm_out, p.comb_w, row0, rows,
        n0, wm, wn);
  } else {
    store_f32_regs<T::TM, T::TN, T::WM, T::WN>(
        acc, rsrc((float *)p.out + (size_t)row0 * N, (uint32_t)rows * N * 4u), N, rows, n0, wm, wn);
  }
}

// Dynamic LDS above 64 KB must be allowed once per device and kernel.
template <typename Kern>
hipError_t allow_lds(Kern kern, int lds, std::atomic<uint64_t> &done) {
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(done.load(std::memory_order_acquire) & bit)) {
    err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    done.fetch_or(bit, std::memory_order_release);
  }
  return hipSuccess;
}

template <bool UP, bool GATHER, bool FUSE, int BM, int BNB, bool LPT>
hipError_t launch_bf16(const BigGemmParams &p, int blocks, hipStream_t st) {
  using T = Tile<BM, BNB, kBK>;
  constexpr int lds = 2 * T::STAGE;
  auto kern = big_gemm_kernel<UP, GATHER, FUSE, BM, BNB, LPT>;
  static std::atomic<uint64_t> attr_done{0};
  hipError_t err = allow_lds(kern, lds, attr_done);
  if (err != hipSuccess) return err;
  kern<<<blocks, kNT, lds, st>>>(p);
  return hipGetLastError();
}

template <bool UP, bool GATHER, bool FUSE, int BM, int BNB>
hipError_t launch_mxdq(const BigGemmParams &p, int blocks, hipStream_t st) {
  using T = Tile<BM, BNB, kBK>;
  constexpr int lds = 2 * T::STAGE;
  auto kern = mxdq_gemm_kernel<UP, GATHER, FUSE, BM, BNB>;
  static std::atomic<uint64_t> attr_done{0};
  hipError_t err = allow_lds(kern, lds, attr_done);
  if (err != hipSuccess) return err;
  kern<<<blocks, kNT, lds, st>>>(p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_big_gemm(const BigGemmParams &p, bool up, bool mx, bool gather, bool fuse,
                           int bm, int bnb, hipStream_t st) {
  const int m_tiles = (p.R + bm - 1) / bm + (p.E < p.R ? p.E : p.R);
  const int blocks = m_tiles * p.n_tiles * (up ? 1 : (p.splits > 1 ? p.splits : 1));
  // Longest first for unsplit bf16 down GEMMs of three or more rounds (16
  // spare blocks: the two tile lists' per-XCD shares round up separately).
  // A tail split (p.tail_splits > 1) runs longest first too; its tail list
  // has tail_splits blocks per tile.
  const bool lpt =
      !up && !mx && p.splits <= 1 && (p.tail_splits > 1 || blocks > 2 * cu_count());
  if (p.tail_splits > 1 && (up || mx || p.splits > 1 || fuse)) return hipErrorInvalidValue;
  const int spare = 16 + (p.tail_splits > 1 ? (p.tail_splits - 1) * (p.E < p.R ? p.E : p.R) *
                                                  p.n_tiles
                                            : 0);
#define MOE_BF16(U, G, F, A, B)                                                     \
  if (!mx && up == U && gather == G && fuse == F && bm == A && bnb == B) {         \
    if constexpr (!U && !F)                                                         \
      if (lpt) return launch_bf16<U, G, F, A, B, true>(p, blocks + spare, st);      \
    return launch_bf16<U, G, F, A, B, false>(p, blocks, st);                        \
  }
#define MOE_MXDQ(U, G, F, A, B)                                                     \
  if (mx && up == U && gather == G && fuse == F && bm == A && bnb == B)            \
    return launch_mxdq<U, G, F, A, B>(p, blocks, st);
  // up: gather from X or contiguous rows
  MOE_BF16(true, true, false, 256, 256)
  MOE_BF16(true, false, false, 256, 256)
  MOE_BF16(true, true, false, 320, 256)
  MOE_BF16(true, false, false, 320, 256)
  // down: f32 pile outputs, or the combine fused for one expert per token
  MOE_BF16(false, false, false, 320, 256)
  MOE_BF16(false, false, true, 320, 256)
  MOE_BF16(false, false, false, 256, 256)
  MOE_BF16(false, false, false, 256, 128)
  MOE_BF16(false, false, false, 128, 128)
  MOE_BF16(false, false, true, 256, 256)
  MOE_BF16(false, false, true, 256, 128)
  MOE_BF16(false, false, true, 128, 128)
  // MXFP4 with K past the GEMM with codes in LDS
  MOE_MXDQ(true, true, false, 256, 256)
  MOE_MXDQ(true, false, false, 256, 256)
  MOE_MXDQ(false, false, false, 256, 256)
  MOE_MXDQ(false, false, false, 256, 128)
  MOE_MXDQ(false, false, false, 128, 128)
  MOE_MXDQ(false, false, true, 256, 256)
  MOE_MXDQ(false, false, true, 256, 128)
  MOE_MXDQ(false, false, true, 128, 128)
#undef MOE_BF16
#undef MOE_MXDQ
  return hipErrorInvalidValue;
}

}  // namespace moe
