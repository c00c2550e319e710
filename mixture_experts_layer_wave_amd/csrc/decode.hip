// Small-batch (decode) path of the MXFP4 expert FFN.
//
// "How Mixture of Experts Scales Model Parameters", section "The forward
// pass: dispatch, then combine": each expert runs its FFN on its own pile.
// With a handful of tokens per expert the work is bound by reading the
// experts' weights, which the lesson "Inference Optimization: The Bandwidth
// Wall, PagedAttention, and FlashAttention" (section on decode) states as
// time >= weight bytes / HBM bandwidth.  MXFP4 storage (the minseoc03.com
// note "What is MXFP4?": 4-bit values, one scale per 32) is read once.
//
// Tile = the weight rows feeding one 16-column MFMA output: 16 rows of W2
// (down), or 8 rows of W1 next to the same 8 rows of W3 (up, so that the
// SwiGLU pair meets in one accumulator).  Work item = (pile, group of 16
// pile rows, tile).  The items of all non-empty experts form one list, cut
// into contiguous ranges, one per workgroup (sized below); two persistent
// workgroups share a CU.  Each streams its tiles through a ring of S LDS
// stages: every byte of a tile (codes and E8M0 scales, contiguous in
// memory) is copied by direct global-to-LDS loads S-1 tiles ahead of the
// tile being multiplied, so a workgroup's compute overlaps its own copies
// and the CU keeps about 100 KB of reads in flight.  Activations of a pile group
// stay in registers for all of its tiles.
//
// The multiply runs on v_mfma_f32_16x16x32_bf16 with pile rows as M (zero-
// padded to 16) and the tile's 16 weight rows as N.  Each lane converts a
// whole 32-element block (16 B of codes + its scale) with
// v_cvt_scalef32_pk_bf16_fp4 and feeds it to 4 MFMAs: for MFMA q of 128-deep
// K step s, lane group g supplies K indices 32 (4 s + g) + 8 q + i, and the
// activations are read in the same order (any fixed K order is valid when
// both operands agree).  The four waves split K; partial sums meet in LDS
// in a fixed order (deterministic).
//
// W4A8 mode (A8): the pile rows are MXFP8 and the multiply runs on
// v_mfma_scale_f32_16x16x128_f8f6f4 with the weight codes as they sit in
// LDS (no conversion).  Operand layout on gfx950: the FP4 operand's lane
// group g holds K [32 g, 32 g + 32) of the 128-deep step (the 16 code bytes
// of block 4 s + g, as above) and gives that block's scale; the FP8
// operand's lane group g holds K [16 g, 16 g + 16) in bytes 0-15 and
// K [64 + 16 g, 80 + 16 g) in bytes 16-31 and gives the scale of block g.
// The up epilogue encodes the hidden as MXFP8: a workgroup's work range is
// cut at multiples of four tiles (the 32 columns of one scale block), wave 0
// keeps the SwiGLU values of the four tiles, then takes each row's block
// maximum across its lanes and writes codes and scale.
#include <atomic>

#include "common.h"
#include "gemm_mxw.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {
namespace {

constexpr int kWaves = 4;      // waves per workgroup, splitting K
constexpr int kCopyWaves = kWaves - 1;  // waves 1.. issue the copies; wave 0 stores
constexpr int kMaxSteps = 8;   // 128-deep K steps per wave: K <= 32 * 4 * 4 * 8 = 4096
constexpr int kBlocksPerCu = 2;  // persistent workgroups per CU (an even grid)
// Share of the work list a CU's second workgroup takes against its first
// (13/16, exact in binary), when each workgroup has at least kShareMinItems
// items (below that the share only makes the ranges lumpier).
constexpr double kSecondShare = 0.8125;
constexpr int kShareMinItems = 4;
constexpr int kMaxStages = 2;    // LDS ring depth per workgroup (2 measured faster than 3)
// Few routed rows: a workgroup has about as many tiles as stages, and a
// third stage (where LDS allows) puts them all in flight at once.
constexpr int kFewRows = 16;
constexpr int kFewRowsStages = 3;
constexpr int kCuLds = 160 * 1024;
constexpr int kRouteMaxR = 64;   // routed rows (n k) of the folded routing
constexpr int kRouteMaxE = 128;  // experts of the folded routing (two per lane)
constexpr int kRoutePer = 2;     // expert slots per lane: topk_per(E) for E <= 128

typedef __attribute__((address_space(3))) void lds_void;

// 128-deep K steps each wave needs for K.
int decode_steps(int K) {
  const int per_wave = (K / 32 + kWaves - 1) / kWaves;  // 32-element blocks
  return (per_wave + 3) / 4;
}

// Rows of each matrix in one tile: 8 of W1 and 8 of W3 (up), 16 of W2 (down).
__host__ __device__ constexpr int tile_rows(bool up) { return up ? 8 : 16; }

// LDS plan of one workgroup.  A stage holds one tile as four regions (two
// for down): the codes of each matrix's rows, then the scales of each
// matrix's rows; each region is copied in 1 KB pieces that never cross a
// region boundary (the last piece of a region is partial).
struct StagePlan {
  int stage_bytes;  // codes + scales of one tile (a multiple of 16)
  int copies;       // 1 KB copies per tile, all waves
  int table_bytes;  // per-expert pile offsets, group prefix and weight slot
  int stages;       // LDS ring depth
  int lds_bytes;    // total per workgroup
};

constexpr int kRedBytes = kWaves * 64 * 16;  // one f32x4 per lane per wave
static_assert(kRedBytes >= (4 * kRouteMaxR + kRouteMaxE) * 4, "folded routing tables fit in red");

StagePlan stage_plan(int K, bool up, int E, int max_stages = kMaxStages) {
  StagePlan s{};
  const int mats = up ? 2 : 1;
  const int code_bytes = tile_rows(up) * (K / 2), scale_bytes = tile_rows(up) * (K / 32);
  s.stage_bytes = mats * (code_bytes + scale_bytes);
  s.copies = mats * ((code_bytes + 1023) / 1024 + (scale_bytes + 1023) / 1024);
  s.table_bytes = ((3 * (E + 1) * 4 + kRouteMaxR * 4) + 15) & ~15;
  const int avail = kCuLds / kBlocksPerCu - kRedBytes - s.table_bytes;
  s.stages = avail > 0 ? avail / s.stage_bytes : 0;
  if (s.stages > max_stages) s.stages = max_stages;
  // Copies a wave may leave in flight: (stages - 1) tiles, < 64.
  const int per_wave = (s.copies + kCopyWaves - 1) / kCopyWaves;
  while (s.stages > 1 && (s.stages - 1) * per_wave > 63) --s.stages;
  s.lds_bytes = s.stages * s.stage_bytes + kRedBytes + s.table_bytes;
  return s;
}

struct DecodeParams {
  const uint16_t *a;       // up: x [n][K] (through perm) or x_perm [R][K]; down: h [R][K]
  const int32_t *perm;     // pile row -> row of a, or NULL for contiguous rows
  const int32_t *offsets;  // [E+1]
  int E, N, K;             // one expert matrix is N x K (N % 16 == 0; K % 64 == 0 up, % 32 down)
  const uint8_t *w0, *w1;  // codes [E][N][K/2] (w1 = W3 for up)
  const uint8_t *s0, *s1;  // scales [E][N][K/32]
  const int32_t *slot;     // [E] logical -> physical weight slot, or NULL
  int n_slots;
  void *out;               // up: bf16 h [R][N] (A8: MXFP8 codes); down: f32 y_perm [R][N]
  const uint8_t *as;       // A8: E8M0 scales of a's rows, pitch sp
  int sp;
  uint8_t *out_s;          // A8 up: scales of the hidden, pitch mx8_scale_pitch(N)
  StagePlan plan;
  // Routing folded into the up kernel (small batches, route_part set): every
  // workgroup takes the top-k of the route_n tokens from the router's S
  // partial logit planes route_part[s][n][E] and builds the piles itself,
  // with the functions of the separate top-k and dispatch kernels (so the
  // results are the same); workgroup 0 writes idx, w, counts, offsets, perm
  // and inv for the later kernels.  offsets and perm above are not read.
  const float *route_part;
  int route_S, route_n, route_k, route_renorm;
  int32_t *r_idx, *r_counts, *r_offsets, *r_perm, *r_inv;
  float *r_w;
};

// Direct copy of 16 B per lane from global memory (wave-uniform base plus
// the lane's 32-bit offset) to LDS bytes lds + 16 * lane
// (global_load_lds_dwordx4, non-temporal).  It is written as inline
// assembly so that the compiler does not order later LDS accesses of the
// other stages behind it (it would wait for every copy in flight before any
// LDS access): completion is awaited explicitly with vm_wait before the
// barrier that publishes a stage.  M0 is a reserved register: the compiler
// sets it right before each instruction of its own that reads it and does
// not honour it in a clobber list, so the asm cannot declare the write.  The
// generated gfx950 code has no other M0 reader (no movrel, LDS-addtid, GWS
// or sendmsg instruction); tests/test_isa_cpu.py checks that every M0
// reference of this file's device code sits inside this asm block.
__device__ __forceinline__ void copy16_to_lds(const uint8_t *base, uint32_t voff, uint32_t lds) {
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1 nt"
               :
               : "v"(voff), "s"(base), "s"(lds)
               : "memory");
}

template <int N>
__device__ __forceinline__ void vm_wait() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// Wait until at most n (wave-uniform, 0..63) vector memory operations of
// this wave are outstanding.
template <int N = 0>
__device__ __forceinline__ void vm_wait_dyn(int n) {
  if constexpr (N >= 63) {
    vm_wait<63>();
  } else {
    if (n <= N) {
      vm_wait<N>();
      return;
    }
    vm_wait_dyn<N + 1>(n);
  }
}

typedef int v8i __attribute__((ext_vector_type(8)));

// The work list's table, by one wave: s_gpre[e] = 16-row groups of the
// piles before expert e (a pile of m rows has ceil(m / 16)), s_gpre[E] the
// total.  Lane l sums a run of consecutive experts; a wave scan gives each
// run its base.
__device__ __forceinline__ void group_prefix_wave(const int *s_off, int *s_gpre, int E) {
  const int lane = threadIdx.x & 63;
  const int per = (E + 63) >> 6;
  const int lo = min(E, lane * per), hi = min(E, lo + per);
  int run = 0;
  for (int e = lo; e < hi; ++e) run += (s_off[e + 1] - s_off[e] + 15) >> 4;
  const int incl = wave_incl_scan(run);
  int base = incl - run;
  for (int e = lo; e < hi; ++e) {
    s_gpre[e] = base;
    base += (s_off[e + 1] - s_off[e] + 15) >> 4;
  }
  if (lane == 63) s_gpre[E] = incl;
}

// KS = 128-deep K steps per wave (decode_steps(K)); A8: MXFP8 pile rows.
template <bool UP, int KS, bool A8>
__global__ __launch_bounds__(256) void mx_decode_kernel(DecodeParams p) {
  constexpr int NMAT = UP ? 2 : 1;
  constexpr int ROWS = tile_rows(UP);  // rows of each matrix per tile
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const StagePlan &P = p.plan;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N, E = p.E;
  const int KB = K / 32;                 // 32-element blocks per row
  const int rowb = K / 2;                // code bytes per row
  const int code_bytes = ROWS * rowb;    // per matrix
  const int scale_bytes = ROWS * KB;     // per matrix
  const int T = N / ROWS;                // tiles per expert
  const int S = P.stages;
  float *red = (float *)(smem + S * P.stage_bytes);  // [4 waves][64][4]
  int *s_off = (int *)((uint8_t *)red + kRedBytes);         // [E+1] pile offsets
  int *s_gpre = s_off + (E + 1);                            // [E+1] groups before expert e
  int *s_slot = s_gpre + (E + 1);                           // [E] physical weight slot
  int *s_perm = s_slot + (E + 1);                           // [kRouteMaxR] folded routing

  // ---- routing (folded) or the piles from dispatch ---------------------------
  // Either way the LDS tables end up holding the pile offsets s_off, the
  // 16-row groups before each expert s_gpre (the work list below) and the
  // weight slots s_slot.  The slot table is read once here: a copying wave
  // that loaded it from global memory per tile would wait for all of its
  // copies in flight too (one in-order counter).
  const int32_t *perm = p.perm;
  if (p.route_part) {
    // Tables in `red` (free until the first tile): chosen ids, weights and
    // pile rows of the (token, slot) pairs, and the pile sizes.
    const int n = p.route_n, k = p.route_k, R = n * k;
    int *s_idx = (int *)red;
    int *s_idx_sink = s_idx + kRouteMaxR;
    float *s_w = (float *)(s_idx_sink + kRouteMaxR);
    int *s_inv = (int *)(s_w + kRouteMaxR);
    int *s_cnt = s_inv + kRouteMaxR;
    const bool publish = blockIdx.x == 0;
    const int G = topk_group(E);
    for (int t0 = 0; t0 < n; t0 += kWaves * 64 / G)  // every lane takes part
      topk_token_t<kRoutePer>(p.route_part, p.route_S, (size_t)n * E, t0 + tid / G, n, E, k,
                              p.route_renorm, publish ? p.r_idx : s_idx_sink,
                              publish ? p.r_w : s_w, nullptr, s_idx);
    __syncthreads();
    if (wave == 0) {
      if (R <= kDispTinyR) {
        dispatch_wave_small<kRoutePer>(s_idx, R, k, E, s_cnt, s_off, s_perm, s_inv, s_gpre);
      } else {
        int nbits = 0;
        while ((1 << nbits) < E) ++nbits;
        dispatch_wave(s_idx, R, k, E, nbits, s_cnt, s_off, s_perm, s_inv);
        group_prefix_wave(s_off, s_gpre, E);
      }
    }
    for (int e = tid; e < E; e += kWaves * 64) s_slot[e] = phys_slot(p.slot, p.n_slots, e);
    __syncthreads();
    if (publish) {
      for (int e = tid; e <= E; e += kWaves * 64) {
        p.r_offsets[e] = s_off[e];
        if (e < E) p.r_counts[e] = s_cnt[e];
      }
      for (int q = tid; q < R; q += kWaves * 64) {
        p.r_perm[q] = s_perm[q];
        p.r_inv[q] = s_inv[q];
      }
    }
    perm = s_perm;
  } else {
    for (int e = tid; e <= E; e += kWaves * 64) s_off[e] = p.offsets[e];
    for (int e = tid; e < E; e += kWaves * 64) s_slot[e] = phys_slot(p.slot, p.n_slots, e);
    __syncthreads();
    if (wave == 0) group_prefix_wave(s_off, s_gpre, E);
    __syncthreads();
  }
  const int W = s_gpre[E] * T;  // work items
  const int G = gridDim.x;
  // A8 up: ranges in whole quads of tiles (T % 4 == 0, so quads never
  // straddle a group).  The dispatcher places blocks [0, G/2) first, one per
  // CU, then [G/2, G) as each CU's second workgroup, whose waves are younger
  // and issue after the first's: with equal ranges the second workgroups
  // finished 13-15% later (per-block timelines at 8 and 64 tokens), leaving
  // each CU half used at the end.  With several items per workgroup they get
  // kSecondShare of a first workgroup's share.  The bounds are floor(W c(b) /
  // c(G)) in double precision with the cumulative share c(b) a multiple of
  // 1/16: exact products, one correctly rounded division, the same
  // expression for a block's end and the next block's start, so the ranges
  // tile [0, W).
  // Fewer items (one to a few per workgroup): q each and one more for the
  // first W mod G blocks, which puts the extra items on first workgroups
  // whenever there are at most G/2 of them (n = 1 layer 0.4-0.7 us faster
  // than spreading them evenly).
  constexpr int QT = (UP && A8) ? 4 : 1;
  int w_lo, w_hi;
  if (W / QT >= kShareMinItems * G) {
    const int H = G / 2;
    auto cum = [&](int b) {
      return b <= H ? (double)b : (double)H + (double)(b - H) * kSecondShare;
    };
    const double c_all = cum(G);
    w_lo = QT * (int)floor((double)(W / QT) * cum(blockIdx.x) / c_all);
    w_hi = QT * (int)floor((double)(W / QT) * cum(blockIdx.x + 1) / c_all);
  } else {
    const int q = (W / QT) / G, rem = (W / QT) % G, b = blockIdx.x;
    w_lo = QT * (b * q + min(b, rem));
    w_hi = QT * ((b + 1) * q + min(b + 1, rem));
  }
  const int n_my = w_hi - w_lo;
  if (n_my <= 0) return;

  // Expert of group index gidx < s_gpre[E]: the e with s_gpre[e] <= gidx <
  // s_gpre[e + 1], by a forward walk from an earlier answer (gidx only grows).
  auto expert_of = [&](int gidx, int from) {
    int e = from;
    while (s_gpre[e + 1] <= gidx) ++e;
    return e;
  };
  // The first item's expert: the number of experts e with s_gpre[e] <= g0,
  // less one (s_gpre does not decrease, so they are a prefix of [0, E), and
  // the last of them has a group, since s_gpre[e + 1] > g0); ballots over
  // chunks of 64 experts, in every wave.
  int e_first;
  {
    const int g0 = w_lo / T;
    int c = 0;
    for (int e0 = 0; e0 < E; e0 += 64)
      c += __popcll(__ballot(e0 + lane < E && s_gpre[e0 + lane] <= g0));
    e_first = c - 1;
  }

  // ---- copy of one tile into stage st -------------------------------------
  // Stage layout: codes of matrix 0 [ROWS][K/2], (up) codes of matrix 1,
  // scales of matrix 0 [ROWS][K/32], (up) scales of matrix 1; each region is
  // contiguous in memory.  Copy q of a tile (regions in that order, 1 KB
  // pieces) belongs to wave 1 + q % 3; lane l moves bytes 16 l of the piece.
  // Wave 0 issues no copies: it writes the outputs, and its stores would
  // otherwise sit in the same in-order counter as its copies and make its
  // wait for a tile's copies also wait for later copies.
  const uint32_t lds_base = (uint32_t)(size_t)(lds_void *)smem;
  const uint32_t voff = lane * 16;
  const int code_pieces = (code_bytes + 1023) >> 10, scale_pieces = (scale_bytes + 1023) >> 10;
  auto issue_region = [&](const uint8_t *src, int bytes, int pieces, uint32_t lds, int q0) {
    if (wave == 0) return;
    for (int j = ((wave - 1 - q0) % kCopyWaves + kCopyWaves) % kCopyWaves; j < pieces;
         j += kCopyWaves) {
      const uint32_t at = (uint32_t)j << 10;
      if (at + voff < (uint32_t)bytes)
        copy16_to_lds(src + at, voff, __builtin_amdgcn_readfirstlane(lds + at));
    }
  };
  auto issue_tile = [&](int e, int tile, int st) {
    const size_t wrow = (size_t)s_slot[e] * N + (size_t)tile * ROWS;
    const uint32_t dst = lds_base + st * P.stage_bytes;
    issue_region(p.w0 + wrow * rowb, code_bytes, code_pieces, dst, 0);
    if constexpr (UP) issue_region(p.w1 + wrow * rowb, code_bytes, code_pieces, dst + code_bytes,
                                   code_pieces);
    issue_region(p.s0 + wrow * KB, scale_bytes, scale_pieces, dst + NMAT * code_bytes,
                 NMAT * code_pieces);
    if constexpr (UP)
      issue_region(p.s1 + wrow * KB, scale_bytes, scale_pieces,
                   dst + NMAT * code_bytes + scale_bytes, NMAT * code_pieces + scale_pieces);
  };
  // Copies this wave issues per tile.
  int my_copies = 0;
  if (wave > 0)
    for (int q = wave - 1; q < P.copies; q += kCopyWaves) ++my_copies;

  // Prologue: the first S tiles in flight.
  {
    int e = e_first;
    for (int j = 0; j < S && j < n_my; ++j) {
      const int w = w_lo + j;
      e = expert_of(w / T, e);
      issue_tile(e, w % T, j);
    }
  }

  // Lane (r, g): B column r is row r of W2 (down), or row r & 7 of W1 (r < 8)
  // or W3 (r >= 8) (up); A row r is pile row t0 + r.
  const int r = lane & 15, g = lane >> 4;
  const int bmat = UP ? (r >> 3) : 0, brow = UP ? (r & 7) : r;
  const int kb_lo = (KB * wave) / kWaves, kb_hi = (KB * (wave + 1)) / kWaves;
  const u32x4 z4 = {0u, 0u, 0u, 0u};
  u32x4 act[A8 ? 1 : KS][4];
  u32x4 act8[A8 ? KS : 1][2];    // A8: the two 16-B halves of each step
  uint32_t asc[A8 ? KS : 1];     // A8: the row's scale of block 4 s + g
  float hq[(UP && A8) ? 4 : 1][4];  // A8 up (wave 0): SwiGLU values of a quad
  int cur_group = -1, e_cur = e_first, row0 = 0, m = 0, t0 = 0;

  for (int i = 0; i < n_my; ++i) {
    const int w = w_lo + i, gidx = w / T, tile = w % T, st = i % S;
    // A copying wave's copies of tile i have landed once at most the copies
    // of the tiles issued after it are outstanding (they complete in order).
    // The first item always opens a group.  When the prologue put all of
    // the workgroup's tiles in flight, its activation loads go out right
    // behind those copies and the one wait below covers both (one trip to
    // memory instead of two); with more tiles, waiting for all of the
    // prologue's copies before tile 0 measured slower.
    if (wave > 0 && (i > 0 || n_my > S)) vm_wait_dyn(min(S - 1, n_my - 1 - i) * my_copies);
    if (gidx != cur_group) {
      // ---- activations of the new group (rows t0..t0+15 of the pile) ----
      // Pile rows are gathered from the token matrix when perm is given
      // (the fused forward), else read in place (x_perm, or h for down).
      e_cur = expert_of(gidx, e_cur);
      cur_group = gidx;
      row0 = s_off[e_cur];
      m = s_off[e_cur + 1] - row0;
      t0 = (gidx - s_gpre[e_cur]) * 16;
      const int t = t0 + r;
      const bool tv = t < m;
      const int arow = tv ? (perm ? perm[row0 + t] : row0 + t) : 0;
      if constexpr (A8) {
        const uint8_t *ap = (const uint8_t *)p.a + (size_t)arow * K;
        const uint8_t *sp = p.as + (size_t)arow * p.sp;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int wb = kb_lo + 4 * s;  // first block of the step
          const int blo = wb + (g >> 1), bhi = wb + 2 + (g >> 1);
          act8[s][0] = (tv && blo < kb_hi) ? *(const u32x4 *)(ap + wb * 32 + 16 * g) : z4;
          act8[s][1] = (tv && bhi < kb_hi) ? *(const u32x4 *)(ap + wb * 32 + 64 + 16 * g) : z4;
          asc[s] = (tv && wb + g < kb_hi) ? (uint32_t)sp[wb + g] : 127u;
        }
      } else {
        const uint16_t *ap = p.a + (size_t)arow * K;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const int b = kb_lo + 4 * s + g;
          const bool ok = tv && b < kb_hi;
#pragma unroll
          for (int q = 0; q < 4; ++q) act[s][q] = ok ? *(const u32x4 *)(ap + b * 32 + q * 8) : z4;
        }
      }
      vm_wait<0>();
    }
    lds_barrier();  // every wave's copies of tile i have landed

    // ---- MFMA over this wave's K range (two independent chains) ---------
    const uint8_t *lw = smem + st * P.stage_bytes + bmat * code_bytes;  // this lane's codes
    const uint8_t *ls = smem + st * P.stage_bytes + NMAT * code_bytes + bmat * scale_bytes;
    f32x4 acc2[2] = {f32x4{0.f, 0.f, 0.f, 0.f}, f32x4{0.f, 0.f, 0.f, 0.f}};
    // All of the step's LDS reads first (codes and scale of each block), so
    // that their latencies overlap, then the conversions and MFMAs.
    u32x4 codes[KS];
    uint32_t sbyte[KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int b = kb_lo + 4 * s + g;
      const bool bv = b < kb_hi;
      codes[s] = bv ? *(const u32x4 *)(lw + brow * rowb + b * 16) : z4;
      // a block past this wave's range has zero codes; its scale byte is
      // replaced by 1.0 so that no NaN can enter
      sbyte[s] = bv ? (uint32_t)ls[brow * KB + b] : 127u;
    }
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      if constexpr (A8) {
        const v8i av = {(int)act8[s][0].x, (int)act8[s][0].y, (int)act8[s][0].z, (int)act8[s][0].w,
                        (int)act8[s][1].x, (int)act8[s][1].y, (int)act8[s][1].z, (int)act8[s][1].w};
        const v8i bw = {(int)codes[s].x, (int)codes[s].y, (int)codes[s].z, (int)codes[s].w, 0, 0, 0, 0};
        acc2[s & 1] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(av, bw, acc2[s & 1], 0, 4, 0,
                                                                       (int)asc[s], 0, (int)sbyte[s]);
        continue;
      }
      const float sc = e8m0_to_f32(sbyte[s]);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint32_t wv = codes[s][q];
        const bf16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 0);
        const bf16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 1);
        const bf16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 2);
        const bf16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 3);
        const u32x4 bw = {__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1),
                          __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3)};
        acc2[q & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, act[s][q]), __builtin_bit_cast(bf16x8, bw), acc2[q & 1], 0,
            0, 0);
      }
    }
    *(f32x4 *)(red + (wave * 64 + lane) * 4) = acc2[0] + acc2[1];
    lds_barrier();  // stage st is free; all partial sums are in LDS

    // ---- wave 0: fixed-order sum (w0 + w1) + (w2 + w3), epilogue ---------
    // Nothing in the loop waits for its stores.
    if (wave == 0) {
      auto column_sum = [&](int l) {
        return (*(const f32x4 *)(red + (0 * 64 + l) * 4) + *(const f32x4 *)(red + (1 * 64 + l) * 4)) +
               (*(const f32x4 *)(red + (2 * 64 + l) * 4) + *(const f32x4 *)(red + (3 * 64 + l) * 4));
      };
      const f32x4 v = column_sum(lane);
      // Up: columns 0-7 are W1 rows (gate), 8-15 the same W3 rows (up); the
      // partner column c + 8 is summed from the LDS partials of lane l + 8.
      const f32x4 u = UP ? column_sum(lane ^ 8) : v;
      // 16x16 output: lane l holds pile rows t0 + (l / 16) * 4 + i, column l % 16.
      if constexpr (UP && A8) {
        // MXFP8 hidden: columns quad * 32 + sub * 8 + r (r < 8) of each row;
        // the block maximum is taken over the four tiles here and over the
        // eight lanes r = 0..7 of the row's lane group.
        const int sub = tile & 3;
#pragma unroll
        for (int ii = 0; ii < 4; ++ii) hq[sub][ii] = silu(v[ii]) * u[ii];
        if (sub == 3) {
          const int quad = tile >> 2, spo = mx8_scale_pitch_dev(N);
#pragma unroll
          for (int ii = 0; ii < 4; ++ii) {
            float am = fmaxf(fmaxf(fabsf(hq[0][ii]), fabsf(hq[1][ii])),
                             fmaxf(fabsf(hq[2][ii]), fabsf(hq[3][ii])));
            am = fmaxf(am, __shfl_xor(am, 1, 64));
            am = fmaxf(am, __shfl_xor(am, 2, 64));
            am = fmaxf(am, __shfl_xor(am, 4, 64));
            const uint32_t code = mx8_scale_code(am);
            const float vv[4] = {hq[0][ii], hq[1][ii], hq[2][ii], hq[3][ii]};
            const uint32_t pk = mx8_pack4(vv, mx8_inv_scale(code));
            const int tt = t0 + (lane >> 4) * 4 + ii;
            if (tt < m && r < 8) {
              uint8_t *o = (uint8_t *)p.out + (size_t)(row0 + tt) * N + quad * 32 + r;
#pragma unroll
              for (int q = 0; q < 4; ++q) o[8 * q] = (uint8_t)(pk >> (8 * q));
              if (r == 0) {
                uint8_t *os = p.out_s + (size_t)(row0 + tt) * spo;
                os[quad] = (uint8_t)code;
                if (quad == N / 32 - 1)  // the row's padding scale bytes are 0
                  for (int b = N / 32; b < spo; ++b) os[b] = 0;
              }
            }
          }
        }
      } else {
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int tt = t0 + (lane >> 4) * 4 + ii;
        if constexpr (UP) {
          if (tt < m && r < 8)
            ((uint16_t *)p.out)[(size_t)(row0 + tt) * N + tile * ROWS + r] =
                (uint16_t)f32_to_bf16_bits(silu(v[ii]) * u[ii]);
        } else {
          if (tt < m) ((float *)p.out)[(size_t)(row0 + tt) * N + tile * ROWS + r] = v[ii];
        }
      }
      }
    }
    if (i + S < n_my) {
      const int wn = w_lo + i + S;
      issue_tile(expert_of(wn / T, e_cur), wn % T, st);
    }
  }
}


template <bool UP, int KS, bool A8>
hipError_t launch_decode_ks(const DecodeParams &p, hipStream_t st) {
  auto kern = mx_decode_kernel<UP, KS, A8>;
  const int lds = p.plan.lds_bytes;
  if (lds > 64 * 1024) {
    // The LDS limit is raised once per device (a per-device kernel attribute).
    static std::atomic<uint64_t> attr_done{0};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(attr_done.load(std::memory_order_acquire) & bit)) {
      err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                kCuLds);
      if (err != hipSuccess) return err;
      attr_done.fetch_or(bit, std::memory_order_release);
    }
  }
  kern<<<kBlocksPerCu * cu_count(), kWaves * 64, lds, st>>>(p);
  return hipGetLastError();
}

// R = routed rows (an upper bound on the pile rows).
template <bool UP, bool A8>
hipError_t launch_decode(DecodeParams p, int R, hipStream_t st) {
  p.plan = stage_plan(p.K, UP, p.E, R <= kFewRows ? kFewRowsStages : kMaxStages);
  if (p.plan.stages < 1) return hipErrorInvalidValue;
  switch (decode_steps(p.K)) {
    case 1: return launch_decode_ks<UP, 1, A8>(p, st);
    case 2: return launch_decode_ks<UP, 2, A8>(p, st);
    case 3: return launch_decode_ks<UP, 3, A8>(p, st);
    case 4: return launch_decode_ks<UP, 4, A8>(p, st);
    case 5: return launch_decode_ks<UP, 5, A8>(p, st);
    case 6: return launch_decode_ks<UP, 6, A8>(p, st);
    case 7: return launch_decode_ks<UP, 7, A8>(p, st);
    case 8: return launch_decode_ks<UP, 8, A8>(p, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int cu_count() {
  static std::atomic<int> cached{0};
  int c = cached.load(std::memory_order_relaxed);
  if (c > 0) return c;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || c <= 0)
    c = 256;
  cached.store(c, std::memory_order_relaxed);
  return c;
}

// Regions are copied in 16 B pieces: the up tile's 8 rows of scales need
// d % 64 == 0; the down tile has 16 rows, so d_ff % 32 == 0 suffices.
bool decode_ffn_fits(int d, int d_ff, int E) {
  return d % 64 == 0 && d_ff % 32 == 0 && decode_steps(d) <= kMaxSteps &&
         decode_steps(d_ff) <= kMaxSteps && stage_plan(d, true, E).stages >= 1 &&
         stage_plan(d_ff, false, E).stages >= 1;
}

bool decode_route_fold_ok(const FfnArgs &a) {
  return a.w_dtype == 2 && a.R <= kDecodeMaxRows && decode_ffn_fits(a.d, a.d_ff, a.E) &&
         a.E <= kRouteMaxE && a.R <= kRouteMaxR && topk_per(a.E) == kRoutePer &&
         a.n * topk_group(a.E) <= kWaves * 64 && a.perm != nullptr;
}

hipError_t launch_decode_up(const FfnArgs &a, hipStream_t st) {
  DecodeParams p{};
  p.a = (const uint16_t *)a.a;
  p.perm = a.perm;
  p.offsets = a.offsets;
  p.E = a.E;
  p.N = a.d_ff;
  p.K = a.d;
  p.w0 = (const uint8_t *)a.w1;
  p.w1 = (const uint8_t *)a.w3;
  p.s0 = a.s1;
  p.s1 = a.s3;
  p.slot = a.slot;
  p.n_slots = a.n_slots;
  p.out = a.h;
  if (a.route_part) {
    if (!decode_route_fold_ok(a)) return hipErrorInvalidValue;
    p.route_part = a.route_part;
    p.route_S = a.route_S;
    p.route_n = a.n;
    p.route_k = a.k;
    p.route_renorm = a.route_renorm;
    p.r_idx = a.r_idx;
    p.r_w = a.r_w;
    p.r_counts = a.r_counts;
    p.r_offsets = a.r_offsets;
    p.r_perm = a.r_perm;
    p.r_inv = a.r_inv;
  }
  if (a.act_quant) {
    const size_t rows = (size_t)(a.perm ? a.n : a.R);
    p.as = (const uint8_t *)a.a + mx8_scale_offset(rows, a.d);
    p.sp = mx8_scale_pitch(a.d);
    p.out_s = (uint8_t *)a.h + mx8_scale_offset(a.R, a.d_ff);
    return launch_decode<true, true>(p, a.R, st);
  }
  return launch_decode<true, false>(p, a.R, st);
}

hipError_t launch_decode_down(const FfnArgs &a, hipStream_t st) {
  DecodeParams p{};
  p.a = (const uint16_t *)a.h;
  p.perm = nullptr;
  p.offsets = a.offsets;
  p.E = a.E;
  p.N = a.d;
  p.K = a.d_ff;
  p.w0 = (const uint8_t *)a.w2;
  p.s0 = a.s2;
  p.slot = a.slot;
  p.n_slots = a.n_slots;
  p.out = a.y_perm;
  if (a.act_quant) {
    p.as = (const uint8_t *)a.h + mx8_scale_offset(a.R, a.d_ff);
    p.sp = mx8_scale_pitch(a.d_ff);
    return launch_decode<false, true>(p, a.R, st);
  }
  return launch_decode<false, false>(p, a.R, st);
}

}  // namespace moe
