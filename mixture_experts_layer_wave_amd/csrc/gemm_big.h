// Large-tile grouped expert GEMM (gemm_big.hip): host launch interface.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

struct BigGemmParams {
  const uint16_t *a;        // bf16 activation rows (x gathered through perm, or contiguous)
  uint32_t a_bytes;         // bytes of the whole activation buffer (< 2^31)
  const int32_t *perm;      // up: pile row -> row of a (NULL = contiguous)
  const int32_t *offsets;   // [E+1] pile boundaries (device)
  int E, R, N, K, n_tiles;  // R = rows of the pile matrix; N, K of one expert matrix
  const void *b0, *b1;      // [E][N][K] bf16 or [E][N][K/2] MXFP4; b1 (W3) for up only
  const uint8_t *s0, *s1;   // MXFP4 E8M0 scales [E][N][K/32]
  const int32_t *slot;      // [E] logical -> physical weight slot, or NULL
  int n_slots;
  void *out;                // up: bf16 [R][N]; down: f32 [R][N]; fused: bf16 y [n][N]
  const int32_t *perm_out;  // fused combine: pile row -> token
  const float *comb_w;      // fused combine: token -> weight (one expert per token)
  int fuse_rows;            // fused combine: rows of y (tokens)
  int out_bf16;             // down, neither fused nor split: pile outputs as bf16
                            // (the f32 result rounded once) in out
  // Split K (down only): each block tile is computed by `splits` blocks over
  // consecutive K ranges of ksplit (a multiple of 64); block s writes its
  // partial sums to part[s][R][N] f32 (out and the fused combine unused),
  // and a later kernel adds the planes in split order.
  int splits, ksplit;
  float *part;
  // Tail split (unsplit down GEMMs run longest first): the last row tile of
  // each pile is computed by tail_splits blocks over K ranges of tail_ksplit
  // (a multiple of 64); split s writes its rows of the tile to tail_part +
  // s * tail_plane, at row e * bm + (row - the tile's first row), [.][N] f32.
  // The pile outputs of those rows are the sum of the planes in split order
  // (the combine or launch_tail_sum adds them).
  int tail_splits, tail_ksplit;
  float *tail_part;
  size_t tail_plane;
};

// up: H = silu(A W1^T) * (A W3^T); down: Yp = H W2^T (or the fused combine).
// bm x bnb is the block tile (256x256 or 320x256 for up; 320x256, 256x256,
// 256x128 or 128x128 for down).  Returns hipErrorInvalidValue for a
// combination not built.
hipError_t launch_big_gemm(const BigGemmParams &p, bool up, bool mx, bool gather, bool fuse,
                           int bm, int bnb, hipStream_t st);


}  // namespace moe
