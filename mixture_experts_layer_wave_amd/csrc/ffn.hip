// Grouped expert FFN: for each expert e, the rows offsets[e]..offsets[e+1]
// of the pile matrix go through expert e's SiLU-gated FFN.
//
// "How Mixture of Experts Scales Model Parameters", section "Dense models:
// every parameter in the FFN does work for every token" (up-projection W1 to
// d_ff, activation, down-projection W2 back to d) and section "The forward
// pass: dispatch, then combine" (each expert runs its FFN on its own pile;
// an empty pile costs nothing).  The gated form silu(x W1) * (x W3) is the
// SwiGLU expert body of the configured layers.
//
//   up:   H[r]  = silu(A[r] . W1_e^T) * (A[r] . W3_e^T)      [R][d_ff]
//   down: Yp[r] = H[r] . W2_e^T                                [R][d]
//
// bf16 / MXFP4 weights run on MFMA (v_mfma_f32_32x32x16_bf16, fp32
// accumulate).  MXFP4 tiles are dequantised to bf16 as they are written to
// LDS (v_cvt_scalef32_pk_bf16_fp4: E2M1 x 2^(s-127) is exact in bf16), so
// the MFMA loop is shared.  float32 weights take a plain FMA path.
//
// W4A8 mode (MXFP4 weights with act_quant): the expert input and the hidden
// are MXFP8 and both projections run on the scaled MFMA with the weights in
// their stored form (gemm_mxw.hip).  The minseoc03.com feed's review of the
// vLLM paper (section "What's Next") notes that quantised weights are
// usually widened before the arithmetic and that the widening eats the
// gain; here neither operand is widened.
#include <cmath>

#include "common.h"
#include "gemm_big.h"
#include "gemm_mxw.h"
#include "kernels.h"

// W4A16 tile of the GEMM with MXFP4 codes in LDS (rows x K step).
#ifndef MOE_MXW16_BM
#define MOE_MXW16_BM 128
#endif
#ifndef MOE_MXW16_BK
#define MOE_MXW16_BK 128
#endif

namespace moe {
namespace {

// ---------------------------------------------------------------------------
// Expert of pile row r: the largest e with offsets[e] <= r.
__device__ __forceinline__ int expert_of_row(const int32_t *__restrict__ off, int E, int r) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// float32 path: one thread per output element, FMAs in K order.
__global__ __launch_bounds__(256) void ffn_up_f32_kernel(const float *__restrict__ a,
                                                         const int32_t *__restrict__ perm,
                                                         const int32_t *__restrict__ off, int E,
                                                         int R, int d, int f,
                                                         const float *__restrict__ w1,
                                                         const float *__restrict__ w3,
                                                         const int32_t *__restrict__ slot,
                                                         int n_slots, float *__restrict__ h) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)R * f) return;
  const int r = (int)(i / f), c = (int)(i % f);
  if (r >= off[E]) return;
  const int e = phys_slot(slot, n_slots, expert_of_row(off, E, r));
  const float *ar = a + (size_t)(perm ? perm[r] : r) * d;
  const float *g1 = w1 + ((size_t)e * f + c) * d;
  const float *g3 = w3 + ((size_t)e * f + c) * d;
  float g = 0.f, u = 0.f;
  for (int k = 0; k < d; ++k) {
    g = fmaf(ar[k], g1[k], g);
    u = fmaf(ar[k], g3[k], u);
  }
  h[i] = g / (1.0f + expf(-g)) * u;
}

__global__ __launch_bounds__(256) void ffn_down_f32_kernel(const float *__restrict__ h,
                                                           const int32_t *__restrict__ off, int E,
                                                           int R, int d, int f,
                                                           const float *__restrict__ w2,
                                                           const int32_t *__restrict__ slot,
                                                           int n_slots, float *__restrict__ yp) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)R * d) return;
  const int r = (int)(i / d), c = (int)(i % d);
  if (r >= off[E]) return;
  const int e = phys_slot(slot, n_slots, expert_of_row(off, E, r));
  const float *hr = h + (size_t)r * f;
  const float *wr = w2 + ((size_t)e * d + c) * f;
  float acc = 0.f;
  for (int k = 0; k < f; ++k) acc = fmaf(hr[k], wr[k], acc);
  yp[i] = acc;
}

}  // namespace

namespace {

// The large-tile kernel addresses its operands with 32-bit buffer offsets
// (the host rejects larger shapes before anything is launched).
bool big_ok(const FfnArgs &a, size_t a_bytes, int N, int K) {
  const size_t lim = (size_t)1 << 31;
  if (a.w_dtype != 1 && a.w_dtype != 2) return false;
  if (a_bytes >= lim || (size_t)N * K * 2 >= lim) return false;
  // a tile's f32 output rows are addressed from the tile's first row
  if ((size_t)512 * N * 4 >= lim) return false;
  return K % 8 == 0;
}

// Block-tile choice for the large-tile kernel.  Pile sizes live on the
// device, so the host estimates the row tiles: R rows over min(E, R) piles,
// each pile ~ Normal(mean, binomial variance) for uniform routing, and the
// expected ceil(m / bm) of a pile is sum_j P(m > j bm).  A candidate's cost
// is the number of rounds of blocks over the 256 CUs times the K steps of a
// block times the bytes one block loads per step (the kernel is bound by
// loading its tiles; a round lasts as long as its slowest block), plus a
// fixed cost per round (launch to first step, epilogue) and, when K is
// split, the traffic of the partial sums.  Cost units: one step of a
// 256 x 256 tile (64 KB) is 512 units, about 1.6 us.
struct TileChoice {
  int bm, bnb, splits;
  int bk = 0;  // W4A8: the K step (128 or 256)
};

double expected_row_tiles(const FfnArgs &a, int bm) {
  const int piles = a.E < a.R ? a.E : a.R;
  const double avg = (double)a.R / piles;
  const double sd = sqrt(avg * (1.0 - 1.0 / a.E));
  double t = 0.0;
  for (int j = 0; j * (double)bm < a.R; ++j) {
    const double edge = j * (double)bm + 0.5;  // P(m > j bm) for integer m
    t += sd > 0 ? 0.5 * erfc((edge - avg) / (sd * sqrt(2.0))) : (avg > j * (double)bm ? 1.0 : 0.0);
  }
  return piles * t;
}

// Whether the unsplit bf16 down pass with block tile bm x bnb takes the
// tail split (TailPlan below): it runs longest first over more than two
// rounds of blocks, and the piles' last row tiles, split in two along K,
// fill at most the 256 CUs.
bool tail_split_fits(const FfnArgs &a, int bm, int bnb) {
  if (a.w_dtype != 1 || a.act_quant || a.R == 0 || a.k == 1 || !a.split_ok || a.d % 4) return false;
  if (!big_ok(a, (size_t)a.R * a.d_ff * 2, a.d, a.d_ff)) return false;
  const long long piles = a.E < a.R ? a.E : a.R;
  const long long n_tiles = (a.d + bnb - 1) / bnb;
  const long long blocks = ((a.R + bm - 1) / bm + piles) * n_tiles;
  return blocks > 2 * 256 && piles * n_tiles * 2 <= 256 && (a.d_ff + 63) / 64 >= 4;
}

TileChoice choose_tile(const FfnArgs &a, bool up, const TileChoice *cand, int n_cand,
                       bool w4a8 = false) {
  const int N = up ? a.d_ff : a.d, K = up ? a.d : a.d_ff;
  constexpr double kUnitsPerRound = 1500.0;   // ~5 us of per-block fixed cost
  constexpr double kUnitsPerByte = 312.0 / 6.0e6;  // partial sums at ~6 TB/s
  TileChoice best = cand[0];
  double best_cost = -1;
  for (int i = 0; i < n_cand; ++i) {
    // W4A8 steps are bk deep: bm x bk B of E4M3 rows, 256 x bk/2 B of E2M1
    // codes (read 1.24 times slower in the 64-byte pieces of a 128-deep
    // step) and 2 KB of scales.
    const int kstep = w4a8 ? cand[i].bk : 64;
    if (w4a8 && !mxw_fits(up, true, cand[i].bm, cand[i].bk, K)) continue;
    const long long nk = (K + kstep - 1) / kstep;
    const int S = cand[i].splits < 1 ? 1 : cand[i].splits;
    if (S > 1 && (up || !a.split_ok || nk < 2 * S)) continue;
    if (S > 1 && (double)S * a.R * N * 4 >= 2147483647.0) continue;
    const int cols = up ? cand[i].bnb / 2 : cand[i].bnb;
    // (a fraction of a tile below 0.02 is the normal tail, not a tile)
    const double mt = ceil(expected_row_tiles(a, cand[i].bm) - 0.02);
    const long long nt = (N + cols - 1) / cols;
    const long long rounds = ((long long)mt * nt * S + 255) / 256;
    const double step_units =
        w4a8 ? (cand[i].bm * kstep + 128.0 * kstep * (kstep == 128 ? 1.24 : 1.0) + 2048.0) / 128.0
             : (double)(cand[i].bm + cand[i].bnb);
    double cost = (double)rounds * ((nk + S - 1) / S) * step_units + rounds * kUnitsPerRound;
    if (S > 1) cost += (2.0 * S - 1.0) * a.R * (double)N * 4.0 * kUnitsPerByte;
    if (!up && !w4a8 && S == 1 && tail_split_fits(a, cand[i].bm, cand[i].bnb)) {
      // The piles' last row tiles run as twice as many half-K blocks after
      // the rounds of the other tiles; their two f32 planes are written and
      // added once.
      const double piles = a.E < a.R ? a.E : a.R;
      const long long full = ((long long)((mt - piles) * nt) + 255) / 256;
      const long long tail = ((long long)(piles * nt * 2) + 255) / 256;
      cost = ((double)full * nk + (double)tail * ((nk + 1) / 2)) * step_units +
             (double)(full + tail) * kUnitsPerRound +
             3.0 * piles * cand[i].bm * (double)N * 4.0 * kUnitsPerByte;
    }
    if (best_cost < 0 || cost < best_cost) {
      best = cand[i];
      best_cost = cost;
    }
  }
  return best;
}

// The down pass's block tile and K split (a function of the shape alone, so
// the workspace sizing through down_split_factor and the launch agree).
TileChoice down_tile(const FfnArgs &a) {
  static const TileChoice cand_bf16[] = {{256, 256, 1}, {320, 256, 1}, {256, 128, 1}, {128, 128, 1},
                                         {256, 256, 2}, {256, 256, 3}, {256, 256, 4}, {320, 256, 2},
                                         {320, 256, 3}, {320, 256, 4}};
  static const TileChoice cand_mx[] = {{256, 256, 1}, {256, 128, 1}, {128, 128, 1},
                                       {256, 256, 2}, {256, 256, 3}, {256, 256, 4}};
  // W4A8: 128-row tiles with 256-deep steps where their LDS fits (they read
  // 128-byte pieces of the weight rows; measured 15% faster than 256 x 128
  // on the Zipf-skewed layer), else 256-row tiles with 128-deep steps.
  static const TileChoice cand_w4a8_deep[] = {{128, 256, 1, 256}, {128, 256, 2, 256},
                                              {128, 256, 3, 256}};
  static const TileChoice cand_w4a8[] = {{256, 256, 1, 128}, {256, 256, 2, 128},
                                         {256, 256, 3, 128}, {256, 256, 4, 128}};
  if (a.act_quant)
    return mxw_fits(false, true, 128, 256, a.d_ff) ? choose_tile(a, false, cand_w4a8_deep, 3, true)
                                              : choose_tile(a, false, cand_w4a8, 4, true);
  return a.w_dtype == 2 ? choose_tile(a, false, cand_mx, 6) : choose_tile(a, false, cand_bf16, 10);
}

// Operands of the GEMM with MXFP4 codes in LDS: W4A8 takes MXFP8 matrices
// (a of perm ? n : R rows, h of R rows), W4A16 bf16 rows.
MxwParams mxw_params(const FfnArgs &a, bool up) {
  MxwParams p{};
  p.offsets = a.offsets;
  p.slot = a.slot;
  p.n_slots = a.n_slots;
  p.E = a.E;
  p.R = a.R;
  const size_t rows = up ? (size_t)(a.perm ? a.n : a.R) : (size_t)a.R;
  const int K = up ? a.d : a.d_ff;
  const uint8_t *m = (const uint8_t *)(up ? a.a : a.h);
  p.a = m;
  if (a.act_quant) {
    p.as = m + mx8_scale_offset(rows, K);
    p.a_bytes = (uint32_t)(rows * K);
    p.as_bytes = (uint32_t)(rows * mx8_scale_pitch(K));
  } else {
    p.a_bytes = (uint32_t)(rows * K * 2);
  }
  p.K = K;
  if (up) {
    p.perm = a.perm;
    p.N = a.d_ff;
    p.b0 = (const uint8_t *)a.w1;
    p.b1 = (const uint8_t *)a.w3;
    p.s0 = a.s1;
    p.s1 = a.s3;
    p.out = a.h;
    if (a.act_quant) p.out_s = (uint8_t *)a.h + mx8_scale_offset(a.R, a.d_ff);
  } else {
    p.N = a.d;
    p.b0 = (const uint8_t *)a.w2;
    p.s0 = a.s2;
    p.out = a.y_perm;
  }
  return p;
}

// W4A16 tiles: 128 rows with 128-deep steps, or 64 rows with 256-deep steps
// (128-byte pieces of the weight rows).
TileChoice mxw16_tile(const FfnArgs &a, bool up) {
  const int K = up ? a.d : a.d_ff;
  // (the launcher takes K up to kW4A8MaxK, whatever the LDS would hold)
  if (K <= kW4A8MaxK && K % 32 == 0 && mxw_fits(up, false, MOE_MXW16_BM, MOE_MXW16_BK, K))
    return TileChoice{MOE_MXW16_BM, 256, 1, MOE_MXW16_BK};
  return TileChoice{0, 0, 0, 0};
}

// W4A16 up projection on two four-wave workgroups per CU (mxw16_pair_kernel):
// the 128-expert Zipf layer 2.5% faster than with the eight-wave kernel (the
// up pass alone ~14%); its down pass was slower that way and keeps the
// eight-wave kernel.
constexpr bool kMxw16Pair = true;

hipError_t launch_mxw_up(const FfnArgs &a, hipStream_t st) {
  MxwParams p = mxw_params(a, true);
  p.n_tiles = (a.d_ff + 127) / 128;
  if (!a.act_quant && kMxw16Pair && mxw16_pair_fits(true, a.d))
    return launch_mxw16_pair(p, true, a.perm != nullptr, st);
  if (!a.act_quant && mxw16_mixed_fits(true, a.d))
    return launch_mxw16_mixed(p, true, a.perm != nullptr, st);
  TileChoice t;
  if (a.act_quant)
    t = mxw_fits(true, true, 128, 256, a.d) ? TileChoice{128, 256, 1, 256}
                                            : TileChoice{256, 256, 1, 128};
  else
    t = mxw16_tile(a, true);
  return launch_mxw_gemm(p, true, a.perm != nullptr, a.act_quant, t.bm, t.bk, st);
}

hipError_t launch_mxw_down(const FfnArgs &a, hipStream_t st, bool *fused, bool *yp_bf16) {
  MxwParams p = mxw_params(a, false);
  p.n_tiles = (a.d + 255) / 256;
  // bf16 pile outputs where the caller takes them (unsplit passes only)
  const bool piles16 = a.yp_bf16_ok && a.d % 8 == 0;
  if (!a.act_quant && mxw16_mixed_fits(false, a.d_ff)) {
    p.out_bf16 = piles16 ? 1 : 0;
    hipError_t err = launch_mxw16_mixed(p, false, false, st);
    if (err == hipSuccess && yp_bf16) *yp_bf16 = piles16;
    return err;
  }
  const TileChoice t = a.act_quant ? down_tile(a) : mxw16_tile(a, false);
  if (t.splits > 1 && a.split_part && down_split_factor(a) > 1) {
    p.splits = t.splits;
    p.ksplit = ((a.d_ff + t.bk * t.splits - 1) / (t.bk * t.splits)) * t.bk;
    p.part = a.split_part;
    hipError_t err = launch_mxw_gemm(p, false, false, a.act_quant, t.bm, t.bk, st);
    if (err != hipSuccess) return err;
    if (a.comb_y) {
      if (fused) *fused = true;
      return launch_splitk_combine(a.split_part, t.splits, a.R, a.comb_inv, a.comb_w, a.n, a.k,
                                   a.d, a.comb_y, a.comb_bf16, st);
    }
    return launch_splitk_sum(a.split_part, t.splits, a.R, a.d, a.y_perm, st);
  }
  p.out_bf16 = piles16 ? 1 : 0;
  hipError_t err = launch_mxw_gemm(p, false, false, a.act_quant, t.bm, t.bk, st);
  if (err == hipSuccess && yp_bf16) *yp_bf16 = piles16;
  return err;
}

// Prefill of bf16 rows on MXFP4 weights: the GEMM with the codes in LDS
// when its tile fits at this shape.
bool use_mxw16(const FfnArgs &a, bool up) {
  return a.w_dtype == 2 && !a.act_quant && mxw16_tile(a, up).bm > 0 &&
         (size_t)(a.perm ? a.n : a.R) * a.d * 2 < ((size_t)1 << 31) &&
         (size_t)a.R * a.d_ff * 2 < ((size_t)1 << 31);
}

BigGemmParams big_params(const FfnArgs &a, bool up) {
  BigGemmParams p{};
  p.offsets = a.offsets;
  p.slot = a.slot;
  p.n_slots = a.n_slots;
  p.E = a.E;
  p.R = a.R;
  if (up) {
    p.a = (const uint16_t *)a.a;
    p.a_bytes = (uint32_t)((size_t)(a.perm ? a.n : a.R) * a.d * 2);
    p.perm = a.perm;
    p.N = a.d_ff;
    p.K = a.d;
    p.b0 = a.w1;
    p.b1 = a.w3;
    p.s0 = a.s1;
    p.s1 = a.s3;
    p.out = a.h;
  } else {
    p.a = (const uint16_t *)a.h;
    p.a_bytes = (uint32_t)((size_t)a.R * a.d_ff * 2);
    p.N = a.d;
    p.K = a.d_ff;
    p.b0 = a.w2;
    p.s0 = a.s2;
    p.out = a.y_perm;
  }
  return p;
}

}  // namespace

// Small batches of MXFP4 experts are bound by reading the weights: they take
// the weight-streaming kernel instead of the large-tile GEMM (kDecodeMaxRows
// routed rows at most).

bool use_decode(const FfnArgs &a) {
  return a.w_dtype == 2 && a.R <= kDecodeMaxRows && decode_ffn_fits(a.d, a.d_ff, a.E);
}

// Tail split of the bf16 down pass: when the pass runs longest first (more
// than two rounds of blocks) and the last row tiles of the piles fill at
// most half of the 256 CUs, each of those tiles is computed by two blocks
// over the two halves of K, so the last round has about twice the blocks,
// each half as long (one expert per token keeps its fused combine instead).
struct TailPlan {
  int splits, bm, bnb;
};

TailPlan down_tail_plan(const FfnArgs &a) {
  TailPlan t{1, 0, 0};
  if (a.w_dtype != 1 || a.act_quant || a.R == 0 || a.k == 1 || !a.split_ok || a.d % 4) return t;
  if (!big_ok(a, (size_t)a.R * a.d_ff * 2, a.d, a.d_ff)) return t;
  const TileChoice c = down_tile(a);
  if (c.splits > 1 || !tail_split_fits(a, c.bm, c.bnb)) return t;
  t.splits = 2;
  t.bm = c.bm;
  t.bnb = c.bnb;
  return t;
}

size_t down_tail_bytes(const FfnArgs &a) {
  const TailPlan t = down_tail_plan(a);
  return t.splits > 1 ? (size_t)t.splits * a.E * t.bm * a.d * 4 : 0;
}

int down_split_factor(const FfnArgs &a) {
  if (a.act_quant) return a.split_ok && a.R > 0 && !use_decode(a) ? down_tile(a).splits : 1;
  if (!a.split_ok || a.R == 0 || use_decode(a) || a.d % 4 ||
      !big_ok(a, (size_t)a.R * a.d_ff * 2, a.d, a.d_ff))
    return 1;
  return down_tile(a).splits;
}

hipError_t launch_expert_up(const FfnArgs &a, hipStream_t st) {
  if (a.R == 0) return hipSuccess;
  if (use_decode(a)) return launch_decode_up(a, st);
  if (a.act_quant || use_mxw16(a, true)) return launch_mxw_up(a, st);
  if (a.w_dtype == 0) {
    const long long tot = (long long)a.R * a.d_ff;
    ffn_up_f32_kernel<<<(unsigned)((tot + 255) / 256), 256, 0, st>>>(
        (const float *)a.a, a.perm, a.offsets, a.E, a.R, a.d, a.d_ff, (const float *)a.w1,
        (const float *)a.w3, a.slot, a.n_slots, (float *)a.h);
    return hipGetLastError();
  }
  const size_t a_bytes = (size_t)(a.perm ? a.n : a.R) * a.d * 2;
  if (big_ok(a, a_bytes, a.d_ff, a.d)) {
    static const TileChoice cand[2] = {{256, 256, 1}, {320, 256, 1}};
    const TileChoice t = choose_tile(a, true, cand, a.w_dtype == 2 ? 1 : 2);
    BigGemmParams p = big_params(a, true);
    p.n_tiles = (a.d_ff + t.bnb / 2 - 1) / (t.bnb / 2);

    return launch_big_gemm(p, true, a.w_dtype == 2, a.perm != nullptr, false, t.bm, t.bnb, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_expert_down(const FfnArgs &a, hipStream_t st, bool *fused, bool *yp_bf16) {
  if (fused) *fused = false;
  if (yp_bf16) *yp_bf16 = false;
  if (a.R == 0) return hipSuccess;
  if (use_decode(a)) return launch_decode_down(a, st);
  if (a.act_quant || use_mxw16(a, false)) return launch_mxw_down(a, st, fused, yp_bf16);
  if (a.w_dtype == 0) {
    const long long tot = (long long)a.R * a.d;
    ffn_down_f32_kernel<<<(unsigned)((tot + 255) / 256), 256, 0, st>>>(
        (const float *)a.h, a.offsets, a.E, a.R, a.d, a.d_ff, (const float *)a.w2, a.slot,
        a.n_slots, a.y_perm);
    return hipGetLastError();
  }
  if (big_ok(a, (size_t)a.R * a.d_ff * 2, a.d, a.d_ff)) {
    const TileChoice t = down_tile(a);
    const int bm = t.bm, bnb = t.bnb;
    BigGemmParams p = big_params(a, false);
    p.n_tiles = (a.d + bnb - 1) / bnb;
    if (t.splits > 1 && a.split_part && down_split_factor(a) > 1) {
      p.splits = t.splits;
      p.ksplit = ((a.d_ff + 64 * t.splits - 1) / (64 * t.splits)) * 64;
      p.part = a.split_part;
      hipError_t err = launch_big_gemm(p, false, a.w_dtype == 2, false, false, bm, bnb, st);
      if (err != hipSuccess) return err;
      if (a.comb_y) {
        if (fused) *fused = true;
        return launch_splitk_combine(a.split_part, t.splits, a.R, a.comb_inv, a.comb_w, a.n, a.k,
                                     a.d, a.comb_y, a.comb_bf16, st);
      }
      return launch_splitk_sum(a.split_part, t.splits, a.R, a.d, a.y_perm, st);
    }
    const bool fuse = a.fuse_y != nullptr && a.k == 1;
    const TailPlan tp = down_tail_plan(a);
    const bool tail = tp.splits > 1 && a.tail_part && !fuse;
    // bf16 pile outputs where the caller takes them (with a tail split only
    // when the combine follows here: the tail sums are f32)
    const bool piles16 =
        a.yp_bf16_ok && a.w_dtype == 1 && !fuse && (!tail || a.comb_y) && a.d % 8 == 0;
    p.out_bf16 = piles16 ? 1 : 0;
    if (tail) {
      p.tail_splits = tp.splits;
      p.tail_ksplit = ((a.d_ff + 64 * tp.splits - 1) / (64 * tp.splits)) * 64;
      p.tail_part = a.tail_part;
      p.tail_plane = (size_t)a.E * bm * a.d;
      hipError_t err = launch_big_gemm(p, false, false, false, false, bm, bnb, st);
      if (err != hipSuccess) return err;
      if (a.comb_y) {
        if (fused) *fused = true;
        return launch_combine_tail(a.y_perm, piles16, a.tail_part, tp.splits, p.tail_plane,
                                   a.offsets, a.E, bm, a.comb_inv, a.comb_w, a.n, a.k, a.d,
                                   a.comb_y, a.comb_bf16, st);
      }
      return launch_tail_sum(a.tail_part, tp.splits, p.tail_plane, a.offsets, a.E, bm, a.d,
                             a.y_perm, st);
    }
    if (fuse) {
      p.out = a.fuse_y;
      p.perm_out = a.fuse_perm;
      p.comb_w = a.fuse_w;
      p.fuse_rows = a.n;
    }
    hipError_t err = launch_big_gemm(p, false, a.w_dtype == 2, false, fuse, bm, bnb, st);
    if (err == hipSuccess && fused) *fused = fuse;
    if (err == hipSuccess && yp_bf16) *yp_bf16 = piles16;
    return err;
  }
  return hipErrorInvalidValue;
}

hipError_t launch_grouped_ffn(const FfnArgs &a, hipStream_t st, bool *fused, bool *yp_bf16) {
  hipError_t err = launch_expert_up(a, st);
  if (err != hipSuccess) return err;
  return launch_expert_down(a, st, fused, yp_bf16);
}

}  // namespace moe
