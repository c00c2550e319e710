// Internal launch helpers of libmoe_mi355x (host side).  Each returns the
// hipError_t of its launches; argument validation happens in moe_api.cpp.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// ---- router ---------------------------------------------------------------
// Number of K splits the router logits use for this shape (>= 1; a function
// of d alone).  Split s writes part[s][n][E]; the top-k pass sums the splits
// in order.
int router_splits(int n, int E, int d);
// part[s][n][E] = x[n][d] . wg[E][d] over split s's K range (+ bias[E] in
// split 0); x, wg are bf16 (is_bf16) or f32 (f32 always uses one split).
// Large batches get the splits summed in order inside the launch: then one
// plane, part[0] = p0 + p1 + ..., with the bits the top-k pass would form.
hipError_t launch_router_logits(const void *x, const void *wg, const float *bias, float *part,
                                int n, int d, int E, bool is_bf16, int splits, hipStream_t st);
// Planes launch_router_logits writes for these arguments (1 or splits).
int router_planes(int n, int E, int d, bool is_bf16, int splits);
// idx/w[n][k] from the summed logits: softmax over E, top-k, optional
// renorm; logits[n][E] (may be NULL) receives the summed logits.
hipError_t launch_router_topk(const float *part, int splits, int n, int E, int k, bool renorm,
                              int32_t *idx, float *w, float *logits, hipStream_t st);

// ---- dispatch -------------------------------------------------------------
// Up to kDispSmallR pairs one wave builds the piles (dispatch_wave); above
// kDispChunkMinR pairs, given scratch of dispatch_scratch_bytes(n, k, E)
// (per-chunk counts), one workgroup per chunk of 1024 pairs in two passes;
// else one 1024-thread workgroup (dispatch_block).  All give the same piles.
constexpr int kDispSmallR = 256;
constexpr int kDispChunkMinR = 1024;
size_t dispatch_scratch_bytes(int n, int k, int E);
// Top-k and dispatch in one kernel for small batches (n k <= kDispSmallR
// and one pass of top-k over 256 threads): the same idx, w and piles as
// launch_router_topk followed by launch_dispatch.
bool route_small_ok(int n, int k, int E);
hipError_t launch_route_small(const float *part, int splits, int n, int E, int k, bool renorm,
                              int32_t *idx, float *w, int32_t *counts, int32_t *offsets,
                              int32_t *perm, int32_t *inv, hipStream_t st);
hipError_t launch_dispatch(const int32_t *idx, int n, int k, int E, int32_t *counts,
                           int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *scratch,
                           hipStream_t st);
// Router statistics (stats.hip): P [E], f [E], loss [1]; norm is [n]
// scratch for the per-token softmax normalisers.
hipError_t launch_router_stats(const float *logits, const int32_t *idx, int n, int E, int k,
                               float alpha, float *P, float *f, float *loss, float2 *norm,
                               hipStream_t st);

// active[j] = j-th expert with counts > 0 (ascending), -1 after; *n_active.
hipError_t launch_active_experts(const int32_t *counts, int E, int32_t *active,
                                 int32_t *n_active, hipStream_t st);
// x_perm[r] = x[perm[r]] for r < R, rows of row_bytes bytes (multiple of 4);
// rows with perm[r] outside [0, n) are zeros.
hipError_t launch_gather_rows(const void *x, const int32_t *perm, void *x_perm, int R, int n,
                              int row_bytes, hipStream_t st);

// ---- grouped FFN ----------------------------------------------------------
struct FfnArgs {
  const void *a;          // activations: x (gathered through perm) or x_perm
  const int32_t *perm;    // row -> token, or NULL for contiguous rows
  const int32_t *offsets; // [E+1]
  int E, R, d, d_ff;
  int w_dtype;            // 0 f32, 1 bf16, 2 mxfp4
  const void *w1, *w3, *w2;
  const uint8_t *s1, *s3, *s2;
  const int32_t *slot;    // [E] logical -> physical expert slot, or NULL
  int n_slots;            // physical slots when slot is given
  void *h;                // [R][d_ff] hidden (bf16, or f32 for f32 weights)
  float *y_perm;          // [R][d] f32 (or bf16, see yp_bf16_ok)
  // The caller takes bf16 pile outputs (each the f32 result rounded once)
  // when the down pass can write them (the prefill GEMMs without a K
  // split); launch_expert_down reports whether it did.
  bool yp_bf16_ok;
  int n, k;               // tokens and experts per token
  // Optional combine fused into the down-projection (used when k == 1):
  // y[perm[r]] = w[perm[r]] * (h[r] W2^T), bf16 [n][d].
  void *fuse_y;
  const int32_t *fuse_perm;
  const float *fuse_w;
  // Optional split-K workspace of the down pass: partial planes
  // (down_split_factor(a) x R x d f32).  When K is split the down pass also
  // adds the planes: into y_perm, or, given comb_y, straight into the layer
  // output y[t] = sum_j comb_w[t][j] * (sum of planes)[comb_inv[t][j]].
  bool split_ok;         // the caller provides split_part
  float *split_part;
  void *comb_y;
  const int32_t *comb_inv;
  const float *comb_w;
  bool comb_bf16;
  // Tail split of the down pass (down_tail_bytes > 0): workspace for the
  // partial sums of each pile's last row tile.
  float *tail_part;
  // W4A8 mode (MXFP4 weights only): a and h are MXFP8 matrices (E4M3 codes,
  // then E8M0 scales; layout in gemm_mxw.h) of (perm ? n : R) and R rows,
  // and both projections run on the scaled MFMA.
  bool act_quant;
  // Routing folded into the decode up kernel (decode_route_fold_ok): the
  // router's route_S partial logit planes [S][n][E]; the up kernel then
  // writes r_idx, r_w [n][k], r_counts [E], r_offsets [E+1], r_perm [R],
  // r_inv [n][k] (perm and offsets above must point at r_perm / r_offsets
  // for the down pass and the combine).
  const float *route_part;
  int route_S, route_renorm;
  int32_t *r_idx, *r_counts, *r_offsets, *r_perm, *r_inv;
  float *r_w;
};
// K splits the down pass takes for these arguments (1 = none); with
// split_ok set it tells the workspace layout how many partial planes
// (splits x R x d f32) to reserve.
int down_split_factor(const FfnArgs &a);
// Workspace bytes of the down pass's tail split for these arguments (0 when
// the down pass does not split its tail).
size_t down_tail_bytes(const FfnArgs &a);
hipError_t launch_expert_up(const FfnArgs &a, hipStream_t st);    // A -> h
// h -> y_perm, or straight into fuse_y; *fused (may be NULL) tells which,
// and *yp_bf16 (may be NULL) whether y_perm holds bf16 pile outputs.
hipError_t launch_expert_down(const FfnArgs &a, hipStream_t st, bool *fused = nullptr,
                              bool *yp_bf16 = nullptr);
hipError_t launch_grouped_ffn(const FfnArgs &a, hipStream_t st, bool *fused = nullptr,
                              bool *yp_bf16 = nullptr);

// Compute units of the current device (read once and cached).
int cu_count();

// Small-batch MXFP4 path (decode.hip): persistent workgroups stream 16-row
// weight tiles through an LDS ring.  decode_ffn_fits tells whether the
// shape is supported.
bool decode_ffn_fits(int d, int d_ff, int E);
// The decode up kernel can take the top-k and dispatch of this batch itself
// (MXFP4 weights on the decode path, E <= 128, n k <= 64, one pass of
// top-k over the workgroup, rows gathered through perm).
bool decode_route_fold_ok(const FfnArgs &a);
constexpr int kDecodeMaxRows = 1024;  // routed rows the decode path takes
hipError_t launch_decode_up(const FfnArgs &a, hipStream_t st);
hipError_t launch_decode_down(const FfnArgs &a, hipStream_t st);

// ---- combine --------------------------------------------------------------
// Split-K: y = combine of (sum of the S planes part[s][R][d]); or y_perm =
// that sum.  d % 4 == 0.
hipError_t launch_splitk_combine(const float *part, int S, int R, const int32_t *inv,
                                 const float *w, int n, int k, int d, void *y, bool out_bf16,
                                 hipStream_t st);
hipError_t launch_splitk_sum(const float *part, int S, int R, int d, float *yp, hipStream_t st);
// y_perm: [R][d] f32, or bf16 with in_bf16 (then d % 8 == 0).
hipError_t launch_combine(const void *y_perm, bool in_bf16, const int32_t *inv, const float *w,
                          int n, int k, int d, void *y, bool out_bf16, hipStream_t st);
// The same combine when the last row tile of each pile (bm-row tiles from
// offsets[e]) holds S f32 partial planes tail[s][e * bm + row][d] instead of
// y_perm rows: those rows are the planes' sum in split order.  d % 4 == 0
// (d % 8 == 0 with in_bf16).
hipError_t launch_combine_tail(const void *y_perm, bool in_bf16, const float *tail, int S,
                               size_t plane, const int32_t *offsets, int E, int bm,
                               const int32_t *inv, const float *w, int n, int k, int d, void *y,
                               bool out_bf16, hipStream_t st);
// y_perm rows of the last row tiles = the sum of their S tail planes.
hipError_t launch_tail_sum(const float *tail, int S, size_t plane, const int32_t *offsets, int E,
                           int bm, int d, float *y_perm, hipStream_t st);
// dst[i] = bf16(src[i]) (round to nearest even) for i < count; both 16-byte
// aligned.
hipError_t launch_f32_to_bf16(const float *src, uint16_t *dst, size_t count, hipStream_t st);

}  // namespace moe
