// Grouped expert GEMM with MXFP4 weights kept as codes in LDS
// (gemm_mxw.hip): host launch interface.  Two activation modes: MXFP8 rows
// on the scaled MFMA (W4A8), or bf16 rows with the codes converted to bf16
// as MFMA fragments are read (W4A16).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

// MXFP8 matrix in memory (rows x cols, cols % 32 == 0): E4M3 codes
// [rows][cols], then, from a 256-B aligned offset, E8M0 scales [rows][sp]
// with sp = cols / 32 rounded up to a multiple of 4 (the padding bytes are
// 0, the smallest scale).
inline int mx8_scale_pitch(int cols) { return (cols / 32 + 3) / 4 * 4; }
inline size_t mx8_scale_offset(size_t rows, int cols) {
  return (rows * (size_t)cols + 255) / 256 * 256;
}
inline size_t mx8_bytes(size_t rows, int cols) {
  return mx8_scale_offset(rows, cols) + rows * (size_t)mx8_scale_pitch(cols);
}

struct MxwParams {
  const uint8_t *a;         // token rows (gathered through perm) or pile rows: E4M3 codes
                            // (W4A8) or bf16 (W4A16)
  const uint8_t *as;        // W4A8: their E8M0 scales, pitch mx8_scale_pitch(K)
  uint32_t a_bytes, as_bytes;  // bytes of the code and scale parts (< 2^31)
  const int32_t *perm;      // up: pile row -> row of a (NULL = contiguous)
  const int32_t *offsets;   // [E+1] pile boundaries (device)
  int E, R, N, K, n_tiles;  // R = rows of the pile matrix; N, K of one expert matrix
  const uint8_t *b0, *b1;   // MXFP4 codes [E][N][K/2]; b1 (W3) for up only
  const uint8_t *s0, *s1;   // their E8M0 scales [E][N][K/32]
  const int32_t *slot;      // [E] logical -> physical weight slot, or NULL
  int n_slots;
  // up: the hidden, W4A8 as MXFP8 (codes [R][N] at out, scales
  // [R][pitch(N)] at out_s), W4A16 as bf16 [R][N]; down: f32 [R][N] at out.
  void *out;
  uint8_t *out_s;
  // Split K (down only), as in the bf16 GEMM: block s of a tile covers K
  // range [s ksplit, (s+1) ksplit) and writes part[s][R][N].
  int splits, ksplit;
  float *part;
  int out_bf16;  // down without a K split: pile outputs as bf16 [R][N] (the
                 // f32 result rounded once) instead of f32
};

// Largest K the kernel takes (the whole K range of a tile's weight scales
// is kept in LDS).
constexpr int kW4A8MaxK = 7168;

// up: H = silu(A W1^T) * (A W3^T) (W4A8: encoded as MXFP8); down: Yp =
// H W2^T.  Block tile bm x 256 with a K step of bk, two LDS stages:
// W4A8 (bm, bk) = (256, 128) or (128, 256); W4A16 (128, 128) or (64, 256).
// mxw_fits tells whether the tile's LDS fits at this K.  Returns
// hipErrorInvalidValue for a combination not built or too large.
bool mxw_fits(bool up, bool a8, int bm, int bk, int K);
// W4A16 with two tile shapes in one launch: piles of at most 64 rows take a
// 64-row tile with 256-deep steps, larger piles 128-row tiles with 128-deep
// steps (no K split).
bool mxw16_mixed_fits(bool up, int K);
hipError_t launch_mxw16_mixed(const MxwParams &p, bool up, bool gather, hipStream_t st);
// The same tile list on two four-wave workgroups per CU with 64-deep steps
// (64-row tiles with three stages, 128-row tiles with two).
bool mxw16_pair_fits(bool up, int K);
hipError_t launch_mxw16_pair(const MxwParams &p, bool up, bool gather, hipStream_t st);
hipError_t launch_mxw_gemm(const MxwParams &p, bool up, bool gather, bool a8, int bm, int bk,
                           hipStream_t st);

// MXFP8 encoding of rows x cols bf16 (is_bf16) or f32 values into an
// MXFP8 matrix (codes at q, scales at q_s).
hipError_t launch_quantize_mx8(const void *x, bool is_bf16, int rows, int cols, uint8_t *q,
                               uint8_t *q_s, hipStream_t st);

}  // namespace moe
