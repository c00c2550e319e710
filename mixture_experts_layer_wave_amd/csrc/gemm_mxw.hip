// Grouped expert GEMM with the MXFP4 weights kept as E2M1 codes in LDS (the
// expert FFN; ffn.hip states the operation and its sources).
//
//   up:   H[r]  = silu(A[r] . W1_e^T) * (A[r] . W3_e^T)   (W4A8: MXFP8 out,
//                                                          W4A16: bf16 out)
//   down: Yp[r] = H[r] . W2_e^T                            (f32 out)
//
// W4A8 (A8): MXFP8 activations, both operands in stored form on the scaled
// MFMA (below).  W4A16: bf16 activations on v_mfma_f32_32x32x16_bf16; each
// lane converts the 32 codes of one weight block from LDS with
// v_cvt_scalef32_pk_bf16_fp4 (exact in bf16) into four 8-deep fragments,
// lane half h taking K [32 h, 32 h + 32) of each 64-deep chunk and slice s
// of it K [32 h + 8 s, 32 h + 8 s + 8); the activation fragments are read
// in the same K order (any fixed order is valid when both operands agree).
//
// v_mfma_scale_f32_32x32x64_f8f6f4 multiplies E2M1 weight codes (first
// operand, format 4) by E4M3 activation codes (second operand, format 0),
// each with one E8M0 scale per 32 K.  Its operand layout on gfx950:
//   - FP4 operand: lane l holds row l % 32 and the 32 consecutive K
//     [32 h, 32 h + 32) of the 64-K step (h = l / 32), two per byte with the
//     even K in the low nibble: a 16-B piece of a stored MXFP4 row.
//   - FP8 operand: lane l holds row l % 32; bytes 0-15 are K [16 h, 16 h + 16)
//     and bytes 16-31 are K [32 + 16 h, 48 + 16 h).
//   - Scales: lane l gives the scale of block h (K [32 h, 32 h + 32)) of its
//     row, from the byte of its scale register that op_sel names.
// The output layout is that of the bf16 MFMA: with the weight rows as the
// first operand, accumulator element i of lane l is pile row l % 32 and
// output column (i/4)*8 + (l/32)*4 + i%4 of the 32 x 32 tile.
//
// Block = 8 waves (2 x 4); tile BM pile rows x 256 weight rows; K step BK =
// 128 or 256 (two or four MFMA k-steps) through two LDS stages.  A stage
// holds BM x BK B of activation codes, 256 x BK/2 B of weight codes (both
// in swizzled rows) and the BM rows' activation scales (BK/32 bytes per row
// and step), all copied by direct-to-LDS buffer loads.  A 256-deep step
// reads 128 contiguous bytes of each weight row, which streams from HBM
// about a quarter faster than 64-byte pieces of as many rows.  The weight scales of
// the tile's 256 rows over the whole K range are one contiguous run per
// matrix and are copied once per tile.  At BM = 256 a step moves 50 KB for
// 16.8 MFLOP (the bf16 GEMM: 64 KB for 8.4 MFLOP), and the MFMA runs at
// twice the bf16 rate.
//
// The up epilogue encodes the hidden as MXFP8 (OCP MX v1.0 rule): per row
// and 32 columns, shared exponent X = floor(log2 amax) - 8 read from the
// exponent bits of the float32 amax, elements v * 2^-X (exact) converted by
// v_cvt_pk_fp8_f32 (round to nearest even) after a clamp to +-448.
#include <algorithm>
#include <atomic>
#include <type_traits>

#include "gemm_common.h"
#include "gemm_mxw.h"

namespace moe {
namespace {

using namespace gemm;

typedef int v8i __attribute__((ext_vector_type(8)));

// Tile of BM pile rows x 256 weight rows, K step BK (64, 128 or 256: 32, 64
// or 128 bytes of each weight row per step), NST LDS stages, NW waves per
// block arranged 2 x NW/2.  WSS: the weight scales travel with each step
// (an aligned pair of 4-B words per weight row holding the step's BK/32 = 4
// scale bytes) instead of one run over the whole K range per tile, which
// makes the LDS of a tile independent of K.
template <int BM_, int NST_, int BK_, bool A8_, int NW_ = kNW, bool WSS_ = false>
struct T8 {
  static constexpr int BM = BM_, BNB = 256, BK = BK_, NST = NST_, NW = NW_, NT = NW_ * 64;
  static constexpr bool A8 = A8_, WSS = WSS_;
  static constexpr int WM = BM / 2, WN = BNB / (NW / 2);
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int EA = A8 ? 1 : 2;  // bytes per activation element
  static constexpr int ROWA = BK * EA, ROWB = BK / 2;  // LDS bytes per row and step
  static constexpr int RPA = 1024 / ROWA, RPB = 1024 / ROWB;  // rows per 1 KB run
  static constexpr int A_BYTES = BM * ROWA, B_BYTES = BNB * ROWB, AS_BYTES = A8 ? NW * 256 : 0;
  static constexpr int WS_BYTES = WSS ? BNB * 8 : 0;  // per-step weight scales
  static constexpr int STAGE = A_BYTES + B_BYTES + AS_BYTES + WS_BYTES;
  static constexpr int A_RUNS = A_BYTES / 1024 / NW;  // 1 KB runs per wave per stage
  static constexpr int B_RUNS = B_BYTES / 1024 / NW;
  static constexpr int NKK = BK / 64;                  // 64-deep chunks per K step
  static constexpr int SB = BK / 32;                   // scale bytes per row and step
  static constexpr int RW = BM / NW;  // activation-scale rows copied by each wave
  static constexpr int WS_RUNS = WS_BYTES / 256 / NW;  // 4-B copies of 64 lanes per wave
  static constexpr int NV = A_RUNS + B_RUNS + (A8 ? 1 : 0) + WS_RUNS;  // copies per wave per step
  static_assert(A_RUNS >= 1 && B_RUNS >= 1 && RW * SB <= 256, "tile shape");
  static_assert(!WSS || (!A8 && SB == 4 && WS_RUNS >= 1 && WS_BYTES % (256 * NW) == 0),
                "per-step scales: four bytes a row, whole runs per wave");
  static_assert(NST >= 2 && (NST - 2) * NV < 64, "stages");
};

// Weight-scale bytes of a tile kept in LDS: per matrix, rows x K/32 padded
// to a whole 256-B run.
__host__ __device__ constexpr int ws_region(int rows, int K) {
  return (rows * (K / 32) + 255) / 256 * 256;
}

// One scaled MFMA: weights (E2M1, scale byte 0 of sw) times activations
// (E4M3, scale byte OPA of sa).
template <int OPA>
__device__ __forceinline__ f32x16 mma(const v8i &w, const v8i &a, const f32x16 &c, int sw, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, a, c, 4, 0, 0, sw, OPA, sa);
}

// One block tile (the work of a block once its tile is known).
template <bool UP, bool GATHER, int BM, int NST, int BK_, bool A8, int NW = kNW, bool WSS = false>
__device__ __forceinline__ void mxw_tile(const MxwParams &p, const TileSlot &t, uint8_t *smem,
                                         int tid, int lane, int wave) {
  using T = T8<BM, NST, BK_, A8, NW, WSS>;
  constexpr int BNB = T::BNB, BK = T::BK;
  static_assert(BK == 64 || BK == 128 || BK == 256, "K step");
  constexpr int NR = UP ? BNB / 2 : BNB;  // weight rows per matrix in the tile
  const int N = p.N, K = p.K, KB = K / 32;
  const int S = UP ? 1 : (p.splits > 1 ? p.splits : 1);
  const int e = t.e;
  const int row0 = t.row0, rows = t.rows;
  const int n0 = t.nt * NR;
  const int split = t.split;
  const int kbeg = S > 1 ? split * p.ksplit : 0;
  const int kend = S > 1 ? min(K, kbeg + p.ksplit) : K;
  const int sp = (KB + 3) / 4 * 4;  // activation scale pitch

  // ---- copy offsets ---------------------------------------------------------
  // Activation codes: wave w copies the 1 KB runs w * A_RUNS + j (RPA rows
  // each).  The pile-row -> token loads are issued together (index clamped
  // into the tile, so every load is in bounds) and awaited once.  Valid
  // offsets are < 2^31 (checked on the host); an invalid row carries bit 31,
  // and so does a chunk past the K range, so such lanes read zeros.  With two
  // stages (every step waits for all copies) a run wholly past the pile's
  // rows is not issued at all: the rows it would fill feed only outputs that
  // are never stored.
  constexpr int CPA = T::ROWA / 16, CPB = T::ROWB / 16;  // 16-B chunks per row and step
  constexpr int SD = T::SB / 4;                            // scale words per row and step
  constexpr int EA = T::EA, EPC = 16 / EA;                 // bytes and elements per chunk
  const __amdgpu_buffer_rsrc_t ra = rsrc(p.a, p.a_bytes), ras = rsrc(p.as, p.as_bytes);
  uint32_t a_off[T::A_RUNS];
  int a_src[T::A_RUNS], a_chk[T::A_RUNS];
#pragma unroll
  for (int j = 0; j < T::A_RUNS; ++j) {
    const int run = wave * T::A_RUNS + j, r = run * T::RPA + lane / CPA;
    a_chk[j] = run_chunk<T::ROWA>(run, lane);
    a_src[j] = GATHER ? p.perm[row0 + min(r, rows - 1)] : row0 + r;
  }
  // Activation scales: lane l of wave w copies word l % SD of row
  // RW w + l / SD (lanes past the wave's RW rows read zeros).
  const int srow = T::RW * wave + lane / SD;
  const int s_src = GATHER ? p.perm[row0 + min(srow, rows - 1)] : row0 + srow;
#pragma unroll
  for (int j = 0; j < T::A_RUNS; ++j) {
    const int r = (wave * T::A_RUNS + j) * T::RPA + lane / CPA;
    a_off[j] = r < rows ? (uint32_t)a_src[j] * (uint32_t)(K * EA) + (uint32_t)a_chk[j] * 16u : kOOB;
  }
  const int a_live =
      NST > 2 ? T::A_RUNS
              : __builtin_amdgcn_readfirstlane(
                    min(T::A_RUNS, max(0, (rows - wave * T::A_RUNS * T::RPA + T::RPA - 1) / T::RPA)));
  const uint32_t as_off = (lane < T::RW * SD && srow < rows)
                              ? (uint32_t)s_src * (uint32_t)sp + 4u * (uint32_t)(lane % SD)
                              : kOOB;

  // Weight codes: run j of wave w fills rows (NW j + w) * RPB + lane / CPB;
  // up rows [0, 128) are W1 rows n0.., rows [128, 256) the same rows of W3.
  const int pe = phys_slot(p.slot, p.n_slots, e);
  const size_t qn = (size_t)N * (K / 2), sn = (size_t)N * KB;
  const __amdgpu_buffer_rsrc_t rq0 = rsrc(p.b0 + (size_t)pe * qn, (uint32_t)qn);
  const __amdgpu_buffer_rsrc_t rq1 = UP ? rsrc(p.b1 + (size_t)pe * qn, (uint32_t)qn) : rq0;
  const __amdgpu_buffer_rsrc_t rs0 = rsrc(p.s0 + (size_t)pe * sn, (uint32_t)sn);
  const __amdgpu_buffer_rsrc_t rs1 = UP ? rsrc(p.s1 + (size_t)pe * sn, (uint32_t)sn) : rs0;
  uint32_t b_off[T::B_RUNS];
  int b_chk[T::B_RUNS];
#pragma unroll
  for (int j = 0; j < T::B_RUNS; ++j) {
    const int run = NW * j + wave, br = run * T::RPB + lane / CPB;
    const int n = n0 + (UP ? br % NR : br);
    b_chk[j] = run_chunk<T::ROWB>(run, lane);
    b_off[j] = n < N ? (uint32_t)n * (uint32_t)(K / 2) + (uint32_t)b_chk[j] * 16u : kOOB;
  }
  // Per-step weight scales (WSS): lane l of run j (of wave w) copies word
  // l % 2 of the aligned pair holding row 32 (NW j + w) + l / 2's four
  // scale bytes of the step (rows [NR, 2 NR) of an up tile are W3's); the
  // pair starts at the byte address rounded down to 4, so the step's bytes
  // sit at offset (n KB + first K block) % 4 of the 8, the same every step.
  uint32_t ws_off[T::WS_RUNS > 0 ? T::WS_RUNS : 1];
  if constexpr (WSS) {
#pragma unroll
    for (int j = 0; j < T::WS_RUNS; ++j) {
      const int br = 32 * (NW * j + wave) + (lane >> 1);
      const int n = n0 + (UP ? br % NR : br);
      ws_off[j] = n < N ? ((uint32_t)n * (uint32_t)KB + (uint32_t)(kbeg / 32)) & ~3u : kOOB;
      ws_off[j] += 4u * (uint32_t)(lane & 1);
    }
  }

  // Weight scales of rows [n0, n0 + NR) over all K: one contiguous run of
  // NR * K/32 bytes per matrix (4-B aligned: checked on the host), copied
  // in 256-B pieces; bytes past the matrix read as zero.
  uint8_t *wscl = smem + NST * T::STAGE;
  const int RB = NR * KB, RBP = WSS ? 0 : ws_region(NR, K);
  if constexpr (!WSS) {
    const uint32_t base = (uint32_t)n0 * (uint32_t)KB;
#pragma unroll
    for (int g = 0; g < (UP ? 2 : 1); ++g)
      for (int q = wave; q < RBP / 256; q += NW) {
        const uint32_t o = (uint32_t)q * 256u + (uint32_t)lane * 4u;
        dma4(g ? rs1 : rs0, wscl + g * RBP + q * 256, o < (uint32_t)RB ? base + o : kOOB);
      }
  }

  // Copies of K step kt into LDS stage `stage`.  A step at or past the end
  // issues only zero loads, which keeps the count per step fixed.
  auto issue = [&](int kt, int stage) {
    const int k0 = kbeg + kt * BK;
    uint8_t *sa = smem + stage * T::STAGE;
    uint8_t *sb = sa + T::A_BYTES;
    uint8_t *ss = sb + T::B_BYTES;
#pragma unroll
    for (int j = 0; j < T::A_RUNS; ++j)
      if (j < a_live)
        dma16(ra, sa + (wave * T::A_RUNS + j) * 1024,
              (a_off[j] + (uint32_t)(k0 * EA)) | ((k0 + a_chk[j] * EPC < kend) ? 0u : kOOB));
#pragma unroll
    for (int j = 0; j < T::B_RUNS; ++j) {
      const bool second = UP && (NW * j + wave) * T::RPB >= NR;
      dma16(second ? rq1 : rq0, sb + (NW * j + wave) * 1024,
            (b_off[j] + (uint32_t)k0 / 2u) | ((k0 + b_chk[j] * 32 < kend) ? 0u : kOOB));
    }
    if constexpr (A8) dma4(ras, ss + wave * 256, (as_off + (uint32_t)k0 / 32u) | (k0 < kend ? 0u : kOOB));
    if constexpr (WSS) {
#pragma unroll
      for (int j = 0; j < T::WS_RUNS; ++j) {
        const bool second = UP && 32 * (NW * j + wave) >= NR;  // 32 rows a run
        dma4(second ? rs1 : rs0, ss + T::AS_BYTES + (NW * j + wave) * 256,
             (ws_off[j] + (uint32_t)(kt * T::SB)) | (k0 < kend ? 0u : kOOB));
      }
    }
  };

  const int wm = wave / (NW / 2), wn = wave % (NW / 2);
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
                           : NR + wn * (T::WN / 2) + (j - T::TN / 2) * 32 + lr;
    return wn * T::WN + j * 32 + lr;
  };
  // LDS address of this lane's weight-scale row for subtile j.
  int ws_row[T::TN];
#pragma unroll
  for (int j = 0; j < T::TN; ++j) {
    const int b = brow(j);
    if constexpr (WSS)  // within a stage: the row's word pair, at the step's first byte
      ws_row[j] = T::A_BYTES + T::B_BYTES + T::AS_BYTES + b * 8 +
                  (int)(((uint32_t)(n0 + b % NR) * (uint32_t)KB + (uint32_t)(kbeg / 32)) & 3u);
    else
      ws_row[j] = (b >= NR ? RBP : 0) + (b % NR) * KB;
  }

  // Weight scales of K step kt (the whole-K run is in LDS from the tile's
  // start, so they are read before the step's barrier, off the critical
  // path).  A block past the K range multiplies zero codes; its byte
  // (another row's) is replaced by 1.0 so that a NaN scale cannot leak in.
  const int kbend = (kend + 31) / 32;
  auto load_wsc = [&](auto actc, int kt, uint32_t (&wsc)[T::TN][T::NKK]) {
    constexpr int ACT = decltype(actc)::value;
    if constexpr (ACT > 0) {
      const int blk0 = kbeg / 32 + kt * T::SB + lg;
      const uint8_t *st_ws = smem + (kt % NST) * T::STAGE;  // WSS: this step's stage
#pragma unroll
      for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
        for (int kk = 0; kk < T::NKK; ++kk) {
          const int blk = blk0 + 2 * kk;
          const uint32_t v = WSS ? st_ws[ws_row[tn] + lg + 2 * kk]
                                 : wscl[ws_row[tn] + min(blk, kbend - 1)];
          wsc[tn][kk] = blk < kbend ? v : 127u;
        }
    }
  };
  // One K step: activation scales (W4A8), then the fragments of each 64-K MFMA step (those of
  // step kk + 1 read while step kk multiplies; the copies of a later K step
  // are issued after the first reads).  ACT (a compile-time count) is the
  // number of this wave's 32-row groups that hold pile rows; the empty groups
  // of a ragged last row tile are neither read nor multiplied.  A wave with
  // ACT = 0 still copies and meets every barrier.
  auto step = [&](auto actc, int kt, int stage, int kt_issue, int stage_issue,
                  const uint32_t (&wsc)[T::TN][T::NKK]) {
    constexpr int ACT = decltype(actc)::value;
    constexpr int NKK = T::NKK;
    const uint8_t *sa = smem + stage * T::STAGE;
    const uint8_t *sb = sa + T::A_BYTES;
    const uint8_t *ss = sb + T::B_BYTES;
    const int blk0 = kbeg / 32 + kt * T::SB + lg;  // K block of this lane's half, k-step 0
    // activation scales: word kk / 2 of the row, this half's byte moved to
    // byte 0 (k-step kk even) or 2 (odd)
    uint32_t asc[T::TM][SD];
    if constexpr (A8) {
#pragma unroll
      for (int tm = 0; tm < ACT; ++tm) {
        const int r = wm * T::WM + tm * 32 + lr;
        const uint8_t *q = ss + (r / T::RW) * 256 + (r % T::RW) * T::SB;
#pragma unroll
        for (int w = 0; w < SD; ++w) asc[tm][w] = ((const uint32_t *)q)[w] >> (8 * lg);
      }
    }
    auto frags = [&](int kk, v8i *af, v8i *bf) {
#pragma unroll
      for (int tm = 0; tm < ACT; ++tm) {
        const int r = wm * T::WM + tm * 32 + lr;
        const u32x4 lo = *(const u32x4 *)(sa + swz<T::ROWA>(r, 4 * kk + lg));
        const u32x4 hi = *(const u32x4 *)(sa + swz<T::ROWA>(r, 4 * kk + 2 + lg));
        af[tm] = v8i{(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w,
                     (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
      }
      if constexpr (ACT > 0) {
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) {
          const u32x4 w = *(const u32x4 *)(sb + swz<T::ROWB>(brow(tn), 2 * kk + lg));
          bf[tn] = v8i{(int)w.x, (int)w.y, (int)w.z, (int)w.w, 0, 0, 0, 0};
        }
      }
    };
    if constexpr (!A8) {
      // W4A16: per 64-deep chunk, the lane's 32 weight codes (one block) and
      // the four 16-B activation pieces of its K, then four bf16 MFMA slices
      u32x4 wq[2][T::TN], aq[2][T::TM][4];
      float wsf[T::TN][NKK];
      if constexpr (ACT > 0) {
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn)
#pragma unroll
          for (int kk = 0; kk < NKK; ++kk) wsf[tn][kk] = e8m0_to_f32(wsc[tn][kk]);
      }
      auto frags16 = [&](int kk, u32x4 *wv, u32x4 (*av)[4]) {
#pragma unroll
        for (int tm = 0; tm < ACT; ++tm) {
          const int r = wm * T::WM + tm * 32 + lr;
#pragma unroll
          for (int sl = 0; sl < 4; ++sl)
            av[tm][sl] = *(const u32x4 *)(sa + swz<T::ROWA>(r, 8 * kk + 4 * lg + sl));
        }
        if constexpr (ACT > 0) {
#pragma unroll
          for (int tn = 0; tn < T::TN; ++tn)
            wv[tn] = *(const u32x4 *)(sb + swz<T::ROWB>(brow(tn), 2 * kk + lg));
        }
      };
      frags16(0, wq[0], aq[0]);
      issue(kt_issue, stage_issue);
#pragma unroll
      for (int kk = 0; kk < NKK; ++kk) {
        if (kk + 1 < NKK) frags16(kk + 1, wq[(kk + 1) & 1], aq[(kk + 1) & 1]);
#pragma unroll
        for (int sl = 0; sl < 4; ++sl) {
          bf16x8 wf[T::TN];
#pragma unroll
          for (int tn = 0; tn < T::TN; ++tn) {
            const uint32_t word = wq[kk & 1][tn][sl];
            const float sc = wsf[tn][kk];
            const u32x4 u = {
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 0)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 1)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 2)),
                __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, sc, 3))};
            wf[tn] = __builtin_bit_cast(bf16x8, u);
          }
#pragma unroll
          for (int tm = 0; tm < ACT; ++tm)
#pragma unroll
            for (int tn = 0; tn < T::TN; ++tn)
              acc[tm][tn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                  wf[tn], __builtin_bit_cast(bf16x8, aq[kk & 1][tm][sl]), acc[tm][tn], 0, 0, 0);
        }
      }
      return;
    }
    v8i af[2][T::TM], bf[2][T::TN];
    frags(0, af[0], bf[0]);
    issue(kt_issue, stage_issue);
#pragma unroll
    for (int kk = 0; kk < NKK; ++kk) {
      if (kk + 1 < NKK) frags(kk + 1, af[(kk + 1) & 1], bf[(kk + 1) & 1]);
#pragma unroll
      for (int tm = 0; tm < ACT; ++tm)
#pragma unroll
        for (int tn = 0; tn < T::TN; ++tn) {
          const v8i &wv = bf[kk & 1][tn], &av = af[kk & 1][tm];
          // past the K range the row's scale word may hold another row's
          // bytes: 127 puts 2^0 or 2^-127 (never NaN) in the selected byte
          const int sa = blk0 + 2 * kk < kbend ? (int)asc[tm][kk / 2] : 127;
          if (kk & 1)
            acc[tm][tn] = mma<2>(wv, av, acc[tm][tn], (int)wsc[tn][kk], sa);
          else
            acc[tm][tn] = mma<0>(wv, av, acc[tm][tn], (int)wsc[tn][kk], sa);
        }
    }
  };

  // Step kt's copies are done once only the NST - 2 later steps' copies
  // are pending (loads complete in order); it then issues step kt + NST - 1
  // into the stage that step kt - 1 used.
  const int nk = (kend - kbeg + BK - 1) / BK;
  auto kloop = [&](auto actc) {
    for (int kt = 0; kt < nk; ++kt) {
      // the scale run lands with step 0's copies (per-step scales, WSS,
      // with every step's): read it after that barrier
      uint32_t wsc[T::TN][T::NKK];
      if (kt > 0 && !WSS) load_wsc(actc, kt, wsc);
      wait_vmcnt<(NST - 2) * T::NV>();
      __syncthreads();
      if (kt == 0 || WSS) load_wsc(actc, kt, wsc);
      step(actc, kt, kt % NST, kt + NST - 1, (kt + NST - 1) % NST, wsc);
    }
  };
#pragma unroll
  for (int s = 0; s < NST - 1; ++s) issue(s, s);
  const int act = __builtin_amdgcn_readfirstlane(min(T::TM, max(0, (rows - wm * T::WM + 31) / 32)));
  static_assert(T::TM == 1 || T::TM == 2 || T::TM == 4, "row groups per wave");
  if (act == T::TM) {
    kloop(std::integral_constant<int, T::TM>{});
  } else if (act == 0) {
    kloop(std::integral_constant<int, 0>{});
  } else if constexpr (T::TM >= 2) {
    if (act == 1) {
      kloop(std::integral_constant<int, 1>{});
    } else if constexpr (T::TM == 4) {
      if (act == 2)
        kloop(std::integral_constant<int, 2>{});
      else
        kloop(std::integral_constant<int, 3>{});
    }
  }
  wait_vmcnt<0>();

  // ---- epilogue ---------------------------------------------------------------
  if constexpr (!UP) {
    if (S == 1 && p.out_bf16) {
      store_bf16_regs<T::TM, T::TN, T::WM, T::WN>(
          acc, rsrc((uint16_t *)p.out + (size_t)row0 * N, (uint32_t)rows * (uint32_t)N * 2u), N,
          rows, n0, wm, wn);
    } else {
      float *dst = S > 1 ? p.part + (size_t)split * p.R * N : (float *)p.out;
      store_f32_tile<T::TM, T::TN, T::WM, T::WN>(acc, dst, N, row0, rows, n0, wm, wn, lane);
    }
  } else if constexpr (!A8) {
    __syncthreads();  // every wave is done reading the stages
    store_swiglu_bf16_tile<T::TM, T::TN, T::WM, T::WN, BM, NR, T::NT>(
        acc, smem, (uint16_t *)p.out, N, row0, rows, n0, wm, wn, lane, tid);
  } else {
    // MXFP8 hidden staged through LDS: codes [BM][128 + 16 pad], then one
    // 4-B word of scales per row (the tile's 128 columns are 4 blocks).
    constexpr int OC = NR, PITCH = OC + 16;
    static_assert(OC == 128, "four scale blocks per row and tile");
    __syncthreads();  // every wave is done reading the stages
    uint8_t *so = smem;
    uint8_t *sso = smem + BM * PITCH;
#pragma unroll
    for (int tm = 0; tm < T::TM; ++tm) {
      const int r = wm * T::WM + tm * 32 + lr;
#pragma unroll
      for (int j = 0; j < T::TN / 2; ++j) {
        float v[16];
        float amax = 0.f;
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          v[i] = silu(acc[tm][j][i]) * acc[tm][j + T::TN / 2][i];
          amax = fmaxf(amax, fabsf(v[i]));
        }
        // the other 16 columns of the block are in lane l ^ 32
        amax = fmaxf(amax, __shfl_xor(amax, 32, 64));
        const uint32_t code = mx8_scale_code(amax);
        const float inv = mx8_inv_scale(code);
        const int c0 = wn * (T::WN / 2) + j * 32;
#pragma unroll
        for (int g = 0; g < 4; ++g)
          *(uint32_t *)(so + r * PITCH + c0 + g * 8 + lg * 4) = mx8_pack4(v + 4 * g, inv);
        if (lg == 0) sso[r * 4 + c0 / 32] = (uint8_t)code;
      }
    }
    __syncthreads();
    uint8_t *oq = (uint8_t *)p.out;
    const int spo = (N / 32 + 3) / 4 * 4;
    constexpr int CH = OC / 16;
    for (int idx = tid; idx < BM * CH; idx += T::NT) {
      const int r = idx / CH, ch = idx % CH;
      const int col = n0 + ch * 16;
      if (r < rows && col < N)
        *(u32x4 *)(oq + (size_t)(row0 + r) * N + col) = *(const u32x4 *)(so + r * PITCH + ch * 16);
    }
    // n0 / 32 is a multiple of 4 and at most spo - 4: the word is in the row
    for (int r = tid; r < rows; r += T::NT)
      *(uint32_t *)(p.out_s + (size_t)(row0 + r) * spo + n0 / 32) = *(const uint32_t *)(sso + r * 4);
  }
}

template <bool UP, bool GATHER, int BM, int NST, int BK_, bool A8>
__global__ __launch_bounds__(kNT, 1) void mxw_gemm_kernel(MxwParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ TileSlot s_t;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int S = UP ? 1 : (p.splits > 1 ? p.splits : 1);
  if (wave == 0) map_block<BM>(p.offsets, p.E, p.n_tiles, S, lane, &s_t);
  __syncthreads();
  if (s_t.e < 0) return;
  mxw_tile<UP, GATHER, BM, NST, BK_, A8>(p, s_t, smem, tid, lane, wave);
}

// W4A16 with two tile shapes in one launch: a pile of at most 64 rows takes
// one 64-row tile with 256-deep steps (128-byte pieces of the weight rows,
// which stream about a quarter faster), a larger pile 128-row tiles with
// 128-deep steps (half the weight re-reads per row of the 64-row shape).
// The down pass runs its tiles longest first (measured 0.5-1.3% off the Zipf
// layer's step; the up pass, 0.6% slower that way, keeps the plain order).
constexpr int kMixedSmallRows = 64;
// Row tiles per group in the tile order of both passes (map_block_fn RG;
// in the down pass's longest-first order, of its full row tiles).
constexpr int kMixedRowGroup = 4;
template <bool UP, bool GATHER>
__global__ __launch_bounds__(kNT, 1) void mxw16_mixed_kernel(MxwParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ TileSlot s_t;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0)
    map_block_fn<!UP>(p.offsets, p.E, p.n_tiles, 1, lane, &s_t,
                      [](int m) { return m <= kMixedSmallRows ? kMixedSmallRows : 128; },
                      std::integral_constant<bool, false>{}, 0, kMixedRowGroup);
  __syncthreads();
  if (s_t.e < 0) return;
  if (s_t.bm == kMixedSmallRows)
    mxw_tile<UP, GATHER, kMixedSmallRows, 2, 256, false>(p, s_t, smem, tid, lane, wave);
  else
    mxw_tile<UP, GATHER, 128, 2, 128, false>(p, s_t, smem, tid, lane, wave);
}

// W4A16 with two four-wave workgroups per CU, each with its own step
// barrier, so that one workgroup's barrier and LDS waits overlap the other's
// MFMAs.  To fit two workgroups in the LDS, a pile of more than 64 rows takes
// 128-row tiles with 64-deep steps (32-byte pieces of the weight rows), a
// pile of at most 64 rows a 64-row tile with 128-deep steps whose weight
// scales travel with each step (64-byte pieces, which stream from HBM
// faster than 32-byte ones).  Tile list and order as mxw16_mixed_kernel.
constexpr int kPairNW = 4;
template <bool UP, bool GATHER>
__global__ __launch_bounds__(kPairNW * 64, 2) void mxw16_pair_kernel(MxwParams p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ TileSlot s_t;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (wave == 0)
    map_block_fn<!UP>(p.offsets, p.E, p.n_tiles, 1, lane, &s_t,
                      [](int m) { return m <= kMixedSmallRows ? kMixedSmallRows : 128; },
                      std::integral_constant<bool, false>{}, 0, kMixedRowGroup);
  __syncthreads();
  if (s_t.e < 0) return;
  if (s_t.bm == kMixedSmallRows)
    mxw_tile<UP, GATHER, kMixedSmallRows, 2, 128, false, kPairNW, true>(p, s_t, smem, tid, lane,
                                                                       wave);
  else
    mxw_tile<UP, GATHER, 128, 2, 64, false, kPairNW>(p, s_t, smem, tid, lane, wave);
}

// LDS of a launch: the stages and the tile's weight scales.
template <bool UP, int BM, int NST, int BK, bool A8, bool WSS = false>
constexpr int lds_bytes(int K) {
  using T = T8<BM, NST, BK, A8, kNW, WSS>;
  return NST * T::STAGE + (WSS ? 0 : (UP ? 2 : 1) * ws_region(UP ? T::BNB / 2 : T::BNB, K));
}
constexpr int kLdsMax = 160 * 1024 - 256;  // minus the static tile slot

template <bool UP, bool GATHER, int BM, int NST, int BK, bool A8>
hipError_t launch_one(const MxwParams &p, int blocks, hipStream_t st) {
  using T = T8<BM, NST, BK, A8>;
  constexpr int NR = UP ? T::BNB / 2 : T::BNB;
  const int lds = lds_bytes<UP, BM, NST, BK, A8>(p.K);
  if (lds > kLdsMax) return hipErrorInvalidValue;
  static_assert(BM * (NR * (A8 ? 1 : 2) + 16) + BM * 4 <= NST * T::STAGE,
                "epilogue staging fits the stages");
  auto kern = mxw_gemm_kernel<UP, GATHER, BM, NST, BK, A8>;
  // Dynamic LDS above 64 KB must be allowed once per device (at the largest
  // size any call asks for).
  static std::atomic<uint64_t> attr_done{0};
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done.load(std::memory_order_acquire) & bit)) {
    err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kLdsMax);
    if (err != hipSuccess) return err;
    attr_done.fetch_or(bit, std::memory_order_release);
  }
  kern<<<blocks, kNT, lds, st>>>(p);
  return hipGetLastError();
}

// MXFP8 encoding, one lane per 32-block (lanes past a row's last block
// write its zero padding scales).
template <bool BF16>
__global__ __launch_bounds__(256) void quantize_mx8_kernel(const void *x, int rows, int cols,
                                                           uint8_t *q, uint8_t *qs) {
  const int nb = cols / 32, sp = (nb + 3) / 4 * 4;
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= (long long)rows * sp) return;
  const int row = (int)(gid / sp), blk = (int)(gid % sp);
  if (blk >= nb) {
    qs[(size_t)row * sp + blk] = 0;
    return;
  }
  float v[32];
  const size_t at = (size_t)row * cols + (size_t)blk * 32;
  if constexpr (BF16) {
    const u32x4 *src = (const u32x4 *)((const uint16_t *)x + at);
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const u32x4 w = src[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[c * 8 + 2 * i] = __uint_as_float(w[i] << 16);
        v[c * 8 + 2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
      }
    }
  } else {
    const f32x4 *src = (const f32x4 *)((const float *)x + at);
#pragma unroll
    for (int c = 0; c < 8; ++c) {
      const f32x4 w = src[c];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[c * 4 + i] = w[i];
    }
  }
  float amax = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) amax = fmaxf(amax, fabsf(v[i]));
  const uint32_t code = mx8_scale_code(amax);
  const float inv = mx8_inv_scale(code);
  uint32_t o[8];
#pragma unroll
  for (int g = 0; g < 8; ++g) o[g] = mx8_pack4(v + 4 * g, inv);
  u32x4 *dst = (u32x4 *)(q + at);
  dst[0] = u32x4{o[0], o[1], o[2], o[3]};
  dst[1] = u32x4{o[4], o[5], o[6], o[7]};
  qs[(size_t)row * sp + blk] = (uint8_t)code;
}

}  // namespace

bool mxw_fits(bool up, bool a8, int bm, int bk, int K) {
  int lds = kLdsMax + 1;
#define MOE_MXW_LDS(A8_, M, B) \
  if (a8 == A8_ && bm == M && bk == B) \
    lds = up ? lds_bytes<true, M, 2, B, A8_>(K) : lds_bytes<false, M, 2, B, A8_>(K);
  MOE_MXW_LDS(true, 256, 128)
  MOE_MXW_LDS(true, 128, 256)
  MOE_MXW_LDS(false, 128, 128)
  MOE_MXW_LDS(false, 64, 256)
#undef MOE_MXW_LDS
  return lds <= kLdsMax;
}

hipError_t launch_mxw_gemm(const MxwParams &p, bool up, bool gather, bool a8, int bm, int bk,
                           hipStream_t st) {
  const int m_tiles = (p.R + bm - 1) / bm + (p.E < p.R ? p.E : p.R);
  const int blocks = m_tiles * p.n_tiles * (up ? 1 : (p.splits > 1 ? p.splits : 1));
  if (p.K > kW4A8MaxK || p.K % 32 || !mxw_fits(up, a8, bm, bk, p.K)) return hipErrorInvalidValue;
#define MOE_MXW(U, G, A8_, M, B)                                  \
  if (up == U && gather == G && a8 == A8_ && bm == M && bk == B) \
    return launch_one<U, G, M, 2, B, A8_>(p, blocks, st);
  MOE_MXW(true, true, true, 256, 128)
  MOE_MXW(true, false, true, 256, 128)
  MOE_MXW(false, false, true, 256, 128)
  MOE_MXW(true, true, true, 128, 256)
  MOE_MXW(true, false, true, 128, 256)
  MOE_MXW(false, false, true, 128, 256)
  MOE_MXW(true, true, false, 128, 128)
  MOE_MXW(true, false, false, 128, 128)
  MOE_MXW(false, false, false, 128, 128)
  MOE_MXW(true, true, false, 64, 256)
  MOE_MXW(true, false, false, 64, 256)
  MOE_MXW(false, false, false, 64, 256)
#undef MOE_MXW
  return hipErrorInvalidValue;
}

bool mxw16_mixed_fits(bool up, int K) {
  return mxw_fits(up, false, kMixedSmallRows, 256, K) && mxw_fits(up, false, 128, 128, K);
}

hipError_t launch_mxw16_mixed(const MxwParams &p, bool up, bool gather, hipStream_t st) {
  if (p.K > kW4A8MaxK || p.K % 32 || !mxw16_mixed_fits(up, p.K)) return hipErrorInvalidValue;
  // Row tiles: a pile of m <= 64 rows has one, a larger one ceil(m / 128) <
  // m / 128 + 1, so at most (non-empty piles) + R / 128 in all; blocks past
  // the tile count exit after the map.
  const int m_tiles = (p.R + 127) / 128 + (p.E < p.R ? p.E : p.R);
  // The down pass runs longest first (map_block_fn): 16 spare blocks.
  const int blocks = m_tiles * p.n_tiles + (up ? 0 : 16);
  const int lds = up ? std::max(lds_bytes<true, kMixedSmallRows, 2, 256, false>(p.K),
                                lds_bytes<true, 128, 2, 128, false>(p.K))
                     : std::max(lds_bytes<false, kMixedSmallRows, 2, 256, false>(p.K),
                                lds_bytes<false, 128, 2, 128, false>(p.K));
  auto kern = up ? (gather ? mxw16_mixed_kernel<true, true> : mxw16_mixed_kernel<true, false>)
                 : mxw16_mixed_kernel<false, false>;
  if (!up && gather) return hipErrorInvalidValue;
  static std::atomic<uint64_t> attr_done[3];
  const int which = up ? (gather ? 0 : 1) : 2;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done[which].load(std::memory_order_acquire) & bit)) {
    err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kLdsMax);
    if (err != hipSuccess) return err;
    attr_done[which].fetch_or(bit, std::memory_order_release);
  }
  kern<<<blocks, kNT, lds, st>>>(p);
  return hipGetLastError();
}

// Two workgroups per CU: each at most half of the CU's LDS, less the static
// tile slot.
constexpr int kPairLdsMax = 80 * 1024 - 256;
bool mxw16_pair_fits(bool up, int K) {
  if (K > kW4A8MaxK || K % 32) return false;
  const int lds = up ? std::max(lds_bytes<true, kMixedSmallRows, 2, 128, false, true>(K),
                                lds_bytes<true, 128, 2, 64, false>(K))
                     : std::max(lds_bytes<false, kMixedSmallRows, 2, 128, false, true>(K),
                                lds_bytes<false, 128, 2, 64, false>(K));
  return lds <= kPairLdsMax;
}

hipError_t launch_mxw16_pair(const MxwParams &p, bool up, bool gather, hipStream_t st) {
  if (!mxw16_pair_fits(up, p.K)) return hipErrorInvalidValue;
  if (!up && gather) return hipErrorInvalidValue;
  const int m_tiles = (p.R + 127) / 128 + (p.E < p.R ? p.E : p.R);
  const int blocks = m_tiles * p.n_tiles + (up ? 0 : 16);  // down: longest first, 16 spare
  const int lds = up ? std::max(lds_bytes<true, kMixedSmallRows, 2, 128, false, true>(p.K),
                                lds_bytes<true, 128, 2, 64, false>(p.K))
                     : std::max(lds_bytes<false, kMixedSmallRows, 2, 128, false, true>(p.K),
                                lds_bytes<false, 128, 2, 64, false>(p.K));
  auto kern = up ? (gather ? mxw16_pair_kernel<true, true> : mxw16_pair_kernel<true, false>)
                 : mxw16_pair_kernel<false, false>;
  static std::atomic<uint64_t> attr_done[3];
  const int which = up ? (gather ? 0 : 1) : 2;
  int dev = 0;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  const uint64_t bit = 1ull << (dev & 63);
  if (!(attr_done[which].load(std::memory_order_acquire) & bit)) {
    err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                              kPairLdsMax);
    if (err != hipSuccess) return err;
    attr_done[which].fetch_or(bit, std::memory_order_release);
  }
  kern<<<blocks, kPairNW * 64, lds, st>>>(p);
  return hipGetLastError();
}

hipError_t launch_quantize_mx8(const void *x, bool is_bf16, int rows, int cols, uint8_t *q,
                               uint8_t *q_s, hipStream_t st) {
  if (rows <= 0) return hipSuccess;
  const long long lanes = (long long)rows * mx8_scale_pitch(cols);
  if ((lanes + 255) / 256 > 0x7fffffffll) return hipErrorInvalidValue;
  const int blocks = (int)((lanes + 255) / 256);
  if (is_bf16)
    quantize_mx8_kernel<true><<<blocks, 256, 0, st>>>(x, rows, cols, q, q_s);
  else
    quantize_mx8_kernel<false><<<blocks, 256, 0, st>>>(x, rows, cols, q, q_s);
  return hipGetLastError();
}

}  // namespace moe
