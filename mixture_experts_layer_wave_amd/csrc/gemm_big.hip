// Large-tile grouped expert GEMM for gfx950 (the prefill path of the
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
// fills ragged rows and the K tail.  K advances by BK (MOE_BF16_BK) through
// NST (MOE_BF16_NST) LDS stages: NST - 1 steps of loads are in flight while
// one is multiplied.
// MXFP4 weights go through registers instead: 32 E2M1 codes and their E8M0
// scale are converted to bf16 (v_cvt_scalef32_pk_bf16_fp4) and written to
// LDS (BK = 64, two stages), so the MFMA loop is the same.
//
// Tiles are ordered expert-major, then N-tile, then M-tile, and the ordered
// list is cut into 8 contiguous chunks, one per XCD (workgroup i runs on XCD
// i mod 8), so the tiles that share an expert's weights share one L2.
#include <atomic>
#include <type_traits>

#include "gemm_big.h"
#include "gemm_common.h"
#include "kernels.h"

namespace moe {
namespace {

using namespace gemm;

// K step and LDS stage count of the bf16 path (MXFP4 uses 64 and 2).
#ifndef MOE_BF16_BK
#define MOE_BF16_BK 64
#endif
#ifndef MOE_BF16_NST
#define MOE_BF16_NST 2
#endif

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
// groups of two were 3% slower.
constexpr int kBigRowGroup = 4;

// LPT: longest-first tile order (map_block_fn), for unsplit down GEMMs of
// three or more rounds of blocks, where the ragged last row tiles then fill
// the last round.
template <bool UP, bool MX, bool GATHER, bool FUSE, int BM, int BNB, bool LPT>
__global__ __launch_bounds__(kNT, 1) void big_gemm_kernel(BigGemmParams p) {
  constexpr int BK = MX ? 64 : MOE_BF16_BK;
  constexpr int NST = MX ? 2 : MOE_BF16_NST;
  using T = Tile<BM, BNB, BK>;
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
  if (wave == 0) map_block<BM, LPT, UP>(p.offsets, p.E, p.n_tiles, S, lane, &s_t, S1, kBigRowGroup);
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

  // ---- per-lane DMA offsets -----------------------------------------------
  // Run j of wave w fills LDS chunks q = (4 j + w) * 64 + lane, i.e. row
  // (4 j + w) * RPR + lane / CPR, stored chunk lane % CPR, which must hold
  // global chunk c = stored ^ key(row).  key(row) is the same for every run
  // of a wave: BK = 64: (4 (w % 2) + lane / 16) % 8;  BK = 32: lane / 16.
  const int c = dma_chunk<BK * 2>(wave, lane);
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.a, p.a_bytes);
  // Valid offsets are < 2^31 (checked on the host); an invalid row carries
  // bit 31 and the K tail ORs it in, so such lanes read zeros.
  // The pile-row -> token loads are issued together (row index clamped into
  // the tile, so every load is in bounds) and awaited once.
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
  const size_t mat_elems = (size_t)N * K;
  __amdgpu_buffer_rsrc_t rb0, rb1;
  uint32_t b_off[MX ? 1 : T::B_RUNS];
  if constexpr (!MX) {
    rb0 = rsrc((const uint16_t *)p.b0 + (size_t)pe * mat_elems, (uint32_t)(mat_elems * 2));
    rb1 = UP ? rsrc((const uint16_t *)p.b1 + (size_t)pe * mat_elems, (uint32_t)(mat_elems * 2))
             : rb0;
#pragma unroll
    for (int j = 0; j < T::B_RUNS; ++j) {
      const int br = (kNW * j + wave) * T::RPR + lane / T::CPR;
      const int n = UP ? n0 + (br % (BNB / 2)) : n0 + br;
      b_off[j] = n < N ? ((uint32_t)n * (uint32_t)K + (uint32_t)c * 8u) * 2u : kOOB;
    }
  }
  // MXFP4 units: thread owns (B-row, 32-K block) pairs u = tid + kNT i, read
  // with buffer loads from the expert's code and scale matrices (32-bit
  // offsets; an invalid unit carries kOOB and reads zeros).  Whether a unit
  // is in W1 or W3 (up) depends on its wave only.
  __amdgpu_buffer_rsrc_t rq0, rq1, rs0, rs1;
  uint32_t q_off[MX ? T::MX_UNITS : 1], s_off[MX ? T::MX_UNITS : 1];
  if constexpr (MX) {
    const size_t qn = (size_t)N * (K / 2), sn = (size_t)N * (K / 32);
    rq0 = rsrc((const uint8_t *)p.b0 + (size_t)pe * qn, (uint32_t)qn);
    rs0 = rsrc(p.s0 + (size_t)pe * sn, (uint32_t)sn);
    rq1 = UP ? rsrc((const uint8_t *)p.b1 + (size_t)pe * qn, (uint32_t)qn) : rq0;
    rs1 = UP ? rsrc(p.s1 + (size_t)pe * sn, (uint32_t)sn) : rs0;
#pragma unroll
    for (int i = 0; i < T::MX_UNITS; ++i) {
      const int u = tid + kNT * i;
      const int br = u / (BK / 32), half = u % (BK / 32);
      const int n = UP ? n0 + (br % (BNB / 2)) : n0 + br;
      const bool ok = n < N && u < T::MX_ALL;
      q_off[i] = ok ? (uint32_t)n * (uint32_t)(K / 2) + half * 16u : kOOB;
      s_off[i] = ok ? (uint32_t)n * (uint32_t)(K / 32) + half : kOOB;
    }
  }
  // MXFP4 codes and scales are loaded into registers one step ahead of the
  // activation copies (two register slots, by step parity), so a load has
  // about two steps of compute to land before it is dequantised.
  u32x4 mq[2][MX ? T::MX_UNITS : 1];
  uint32_t ms[2][MX ? T::MX_UNITS : 1];
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

  // Issue the loads of K step kt into LDS stage `stage` (a step at or past
  // the end issues only zero loads, which keeps the count per step fixed),
  // then (MXFP4) the register loads of step kt + 1 into slot SL = (kt+1) & 1
  // (a compile-time index: the K loop is unrolled by two).
  auto issue = [&](int kt, int stage, auto slc) {
    constexpr int SL = decltype(slc)::value;
    const int k0 = kbeg + kt * BK;
    const uint32_t kpen = (k0 + c * 8 < kend) ? 0u : kOOB;
    const uint32_t k0b = (uint32_t)k0 * 2u;
    uint8_t *sa = smem + stage * T::STAGE;
#pragma unroll
    for (int j = 0; j < T::A_RUNS; ++j) dma16(ra, sa + (kNW * j + wave) * 1024, (a_off[j] + k0b) | kpen);
    if constexpr (!MX) {
      uint8_t *sb = sa + T::A_BYTES;
#pragma unroll
      for (int j = 0; j < T::B_RUNS; ++j) {
        const bool second = UP && (kNW * j + wave) * T::RPR >= BNB / 2;
        dma16(second ? rb1 : rb0, sb + (kNW * j + wave) * 1024, (b_off[j] + k0b) | kpen);
      }
    } else {
      load_b(kt + 1, mq[SL], ms[SL]);
    }
  };
  // MXFP4: dequantise the codes of step kt (register slot kt & 1) into the
  // B tile of LDS stage `stage`.
  auto mx_store_slot = [&](int stage, const u32x4 *mqs, const uint32_t *mss) {
    if constexpr (MX) {
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

  // One K step = SLICES MFMA k-slices of 16.  Fragments of slice kk + 1 are
  // read while the MFMAs of slice kk run; scheduling groups pin the order
  // "MFMA, LDS read, MFMA, LDS read, ..." inside a slice (and spread the DMA
  // issue of a later step over slice 0), and slices do not mix.
  //
  // ACT (a compile-time count) is the number of this wave's 32-row groups
  // that hold pile rows: the last row tile of a pile is usually ragged, and
  // its empty groups are neither read from LDS nor multiplied.  A wave with
  // ACT = 0 still issues its share of the copies and meets every barrier.
  constexpr int NV = T::A_RUNS + (MX ? 0 : T::B_RUNS);  // DMA issues per step
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
  auto step = [&](auto actc, int stage, int kt_issue, int stage_issue, auto slc) {
    constexpr int ACT = decltype(actc)::value;
    constexpr int NF = ACT > 0 ? ACT + T::TN : 0;  // fragment reads per slice
    constexpr int NM = ACT * T::TN;                // MFMAs per slice
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
  // Vector memory operations issued after a step's copies: NST - 2 later
  // steps of copies, or (MXFP4) the register loads of the following step.
  constexpr int NAFTER = MX ? 2 * T::MX_UNITS : (NST - 2) * NV;
  // Step kt (parity P = kt & 1): its copies are done once only the later
  // operations are pending; it issues step kt + 1 (and the MXFP4 registers
  // of step kt + 2, slot P) and dequantises step kt + 1 (slot 1 - P).
  auto kstep = [&](auto actc, int kt, auto parc) {
    constexpr int P = decltype(parc)::value;
    wait_vmcnt<NAFTER>();
    __syncthreads();
    step(actc, kt % NST, kt + NST - 1, (kt + NST - 1) % NST, parc);
    if (MX && kt + 1 < nk) mx_store_slot((kt + 1) % NST, mq[1 - P], ms[1 - P]);
  };
  auto kloop = [&](auto actc) {
    if constexpr (MX) {
      for (int kt = 0; kt < nk; kt += 2) {
        kstep(actc, kt, std::integral_constant<int, 0>{});
        if (kt + 1 < nk) kstep(actc, kt + 1, std::integral_constant<int, 1>{});
      }
    } else {
      for (int kt = 0; kt < nk; ++kt) kstep(actc, kt, std::integral_constant<int, 0>{});
    }
  };
  static_assert(NST == 2 || !MX, "MXFP4 register slots assume two LDS stages");
  if constexpr (MX) load_b(0, mq[0], ms[0]);
  issue(0, 0, std::integral_constant<int, 1>{});
#pragma unroll
  for (int s = 1; s < NST - 1; ++s) issue(s, s, std::integral_constant<int, 0>{});
  mx_store_slot(0, mq[0], ms[0]);
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
  wait_vmcnt<0>();

  // ---- epilogue --------------------------------------------------------------
  // The MFMA takes the weight rows as its first operand, so accumulator
  // element i of lane l is pile row l % 32 of the 32-row group and output
  // column (i/4)*8 + (l/32)*4 + i%4 of the 32-column group: every lane holds
  // runs of four consecutive columns of one row.
  if constexpr (!UP) {
    if (tail_split) {
      // This split's partial sums of the pile's last row tile, compactly:
      // row e * BM + (pile row - row0) of plane `split`.
      store_f32_tile<T::TM, T::TN, T::WM, T::WN>(
          acc, p.tail_part + (size_t)split * p.tail_plane + (size_t)e * BM * N, N, 0, rows, n0, wm,
          wn, lane);
      return;
    }
    if (S > 1) {
      // Split K: this block's partial sums go to plane `split` (16-B stores of
      // four columns); a later kernel adds the planes in split order.
      store_f32_tile<T::TM, T::TN, T::WM, T::WN>(acc, p.part + (size_t)split * p.R * N, N, row0,
                                                 rows, n0, wm, wn, lane);
      return;
    }
  }
  if constexpr (UP) {
    __syncthreads();  // every wave is done reading the stages
    store_swiglu_bf16_tile<T::TM, T::TN, T::WM, T::WN, BM, BNB / 2>(acc, smem, (uint16_t *)p.out, N,
                                                                    row0, rows, n0, wm, wn, lane, tid);
  } else if constexpr (FUSE) {
    // Combine fused (one expert per token): y[token] = w(token) * row, bf16,
    // staged through LDS (8-B writes of four columns) so that global stores
    // are 16-B pieces of rows.
    constexpr int OC = BNB;             // output columns of the tile
    constexpr int PITCH = OC * 2 + 16;  // bytes per staged row (padded)
    __syncthreads();  // every wave is done reading the stages
    uint8_t *so = smem;
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      const int r = wm * T::WM + tm * 32 + lr;
      const float scale = p.comb_w[p.perm_out[row0 + min(r, rows - 1)]];
#pragma unroll
      for (int j = 0; j < T::TN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int col = wn * T::WN + j * 32 + g * 8 + lg * 4;
          float v[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) v[q] = acc[tm][j][g * 4 + q] * scale;
          const u32x2 pk = {pack_bf16x2(v[0], v[1]), pack_bf16x2(v[2], v[3])};
          *(u32x2 *)(so + r * PITCH + col * 2) = pk;
        }
      }
    }
    __syncthreads();
    constexpr int CH = OC / 8;  // 16-B chunks per row; N % 8 == 0
    for (int idx = tid; idx < BM * CH; idx += kNT) {
      const int r = idx / CH, ch = idx % CH;
      const int col = n0 + ch * 8;
      if (r < rows && col < N)
        *(u32x4 *)((uint16_t *)p.out + (size_t)p.perm_out[row0 + r] * N + col) =
            *(const u32x4 *)(so + r * PITCH + ch * 16);
    }
  } else {
    // f32 pile outputs.
    store_f32_tile<T::TM, T::TN, T::WM, T::WN>(acc, (float *)p.out, N, row0, rows, n0, wm, wn,
                                               lane);
  }
}

template <bool UP, bool MX, bool GATHER, bool FUSE, int BM, int BNB, bool LPT>
hipError_t launch_one(const BigGemmParams &p, int blocks, hipStream_t st) {
  using T = Tile<BM, BNB, MX ? 64 : MOE_BF16_BK>;
  constexpr int NST = MX ? 2 : MOE_BF16_NST;
  constexpr int OC = UP ? BNB / 2 : BNB;
  constexpr int EPI = (UP || FUSE) ? BM * (OC * 2 + 16) : 0;
  constexpr int lds = NST * T::STAGE > EPI ? NST * T::STAGE : EPI;
  auto kern = big_gemm_kernel<UP, MX, GATHER, FUSE, BM, BNB, LPT>;
  // Dynamic LDS above 64 KB must be allowed once per device.
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load(std::memory_order_acquire) & bit)) {
    err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (err != hipSuccess) return err;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
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
#define MOE_BIG(U, M, G, F, A, B)                                                    \
  if (up == U && mx == M && gather == G && fuse == F && bm == A && bnb == B) {      \
    if constexpr (!U && !M)                                                          \
      if (lpt) return launch_one<U, M, G, F, A, B, true>(p, blocks + spare, st);     \
    return launch_one<U, M, G, F, A, B, false>(p, blocks, st);                       \
  }
  // up: gather from X or contiguous rows; bf16 or MXFP4 weights
  MOE_BIG(true, false, true, false, 256, 256)
  MOE_BIG(true, false, false, false, 256, 256)
  MOE_BIG(true, false, true, false, 320, 256)
  MOE_BIG(true, false, false, false, 320, 256)
  MOE_BIG(false, false, false, false, 320, 256)
  MOE_BIG(false, false, false, true, 320, 256)
  MOE_BIG(true, true, true, false, 256, 256)
  MOE_BIG(true, true, false, false, 256, 256)
  // down: f32 pile outputs, or the combine fused for one expert per token
  MOE_BIG(false, false, false, false, 256, 256)
  MOE_BIG(false, false, false, false, 256, 128)
  MOE_BIG(false, false, false, false, 128, 128)
  MOE_BIG(false, false, false, true, 256, 256)
  MOE_BIG(false, false, false, true, 256, 128)
  MOE_BIG(false, false, false, true, 128, 128)
  MOE_BIG(false, true, false, false, 256, 256)
  MOE_BIG(false, true, false, false, 256, 128)
  MOE_BIG(false, true, false, false, 128, 128)
  MOE_BIG(false, true, false, true, 256, 256)
  MOE_BIG(false, true, false, true, 256, 128)
  MOE_BIG(false, true, false, true, 128, 128)
#undef MOE_BIG
  return hipErrorInvalidValue;
}

}  // namespace moe
