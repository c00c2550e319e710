// Combine: put the weighted expert outputs back in token order.
//
// "How Mixture of Experts Scales Model Parameters", section "The forward
// pass: dispatch, then combine" (every output row is multiplied by the
// probability its token was routed with, then rows return to the tokens'
// original order) and section "Top-K: several experts, added up by weight"
// (the K weighted outputs are added).
//
// y[t] = sum_{j<k} w[t][j] * y_perm[inv[t][j]], in slot order, in float32.
// (After a split-K down pass, y_perm[r] is itself the sum of the partial
// planes in split order.)
// A gather-reduce: each output element is written once, with no atomics,
// so the result does not depend on scheduling.  A pair whose pile row is
// outside [0, n k) (its expert id was outside [0, E) at dispatch) adds
// nothing.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

// Each thread owns 4 consecutive columns of one token row (d % 4 == 0).
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_vec4_kernel(const float *__restrict__ yp,
                                                           const int32_t *__restrict__ inv,
                                                           const float *__restrict__ w, int n,
                                                           int k, int d, void *__restrict__ y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (t >= n || c >= d) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const unsigned R = (unsigned)n * (unsigned)k;
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const int r = inv[(size_t)t * k + j];
    if ((unsigned)r >= R) continue;
    const f32x4 v = *(const f32x4 *)(yp + (size_t)r * d + c);
    acc[0] = fmaf(wj, v[0], acc[0]);
    acc[1] = fmaf(wj, v[1], acc[1]);
    acc[2] = fmaf(wj, v[2], acc[2]);
    acc[3] = fmaf(wj, v[3], acc[3]);
  }
  if constexpr (OUT_BF16) {
    u32x2 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *(u32x2 *)((uint16_t *)y + (size_t)t * d + c) = o;
  } else {
    *(f32x4 *)((float *)y + (size_t)t * d + c) = acc;
  }
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_scalar_kernel(const float *__restrict__ yp,
                                                             const int32_t *__restrict__ inv,
                                                             const float *__restrict__ w, int n,
                                                             int k, int d, void *__restrict__ y) {
  const int t = blockIdx.y;
  const int c = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= n || c >= d) return;
  const unsigned R = (unsigned)n * (unsigned)k;
  float acc = 0.f;
  for (int j = 0; j < k; ++j) {
    const int r = inv[(size_t)t * k + j];
    if ((unsigned)r < R) acc = fmaf(w[(size_t)t * k + j], yp[(size_t)r * d + c], acc);
  }
  if constexpr (OUT_BF16)
    ((uint16_t *)y)[(size_t)t * d + c] = (uint16_t)f32_to_bf16_bits(acc);
  else
    ((float *)y)[(size_t)t * d + c] = acc;
}

// Split-K down pass: the pile output is the sum of S partial planes
// part[s][R][d] (added in split order), then combined like y_perm above.
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void splitk_combine_kernel(const float *__restrict__ part, int S,
                                                             size_t plane,
                                                             const int32_t *__restrict__ inv,
                                                             const float *__restrict__ w, int n,
                                                             int k, int d, void *__restrict__ y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (t >= n || c >= d) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const unsigned R = (unsigned)n * (unsigned)k;
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const int r = inv[(size_t)t * k + j];
    if ((unsigned)r >= R) continue;
    const float *src = part + (size_t)r * d + c;
    f32x4 v = *(const f32x4 *)src;
    for (int sp = 1; sp < S; ++sp) v += *(const f32x4 *)(src + sp * plane);
    acc[0] = fmaf(wj, v[0], acc[0]);
    acc[1] = fmaf(wj, v[1], acc[1]);
    acc[2] = fmaf(wj, v[2], acc[2]);
    acc[3] = fmaf(wj, v[3], acc[3]);
  }
  if constexpr (OUT_BF16) {
    u32x2 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *(u32x2 *)((uint16_t *)y + (size_t)t * d + c) = o;
  } else {
    *(f32x4 *)((float *)y + (size_t)t * d + c) = acc;
  }
}

// y_perm = the sum of the S partial planes, in split order (4 floats a thread).
__global__ __launch_bounds__(256) void splitk_sum_kernel(const float *__restrict__ part, int S,
                                                         size_t plane, size_t total4,
                                                         float *__restrict__ yp) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= total4) return;
  f32x4 v = *(const f32x4 *)(part + i * 4);
  for (int sp = 1; sp < S; ++sp) v += *(const f32x4 *)(part + sp * plane + i * 4);
  *(f32x4 *)(yp + i * 4) = v;
}

// Pile e's last row tile starts at offsets[e] + (ceil(m / bm) - 1) bm.
__device__ __forceinline__ int expert_of(const int32_t *__restrict__ off, int E, int r) {
  int lo = 0, hi = E;
  while (hi - lo > 1) {
    const int mid = (lo + hi) >> 1;
    if (off[mid] <= r) lo = mid; else hi = mid;
  }
  return lo;
}
__device__ __forceinline__ int tail_begin(const int32_t *__restrict__ off, int e, int bm) {
  const int m = off[e + 1] - off[e];
  return off[e] + ((m + bm - 1) / bm - 1) * bm;
}

// Four columns of pile row r: from y_perm, or, in a last row tile, the sum
// of its S partial planes in split order.
__device__ __forceinline__ f32x4 pile_row4(const float *__restrict__ yp,
                                           const float *__restrict__ tail, int S, size_t plane,
                                           const int32_t *__restrict__ off, int E, int bm, int r,
                                           int d, int c) {
  const int e = expert_of(off, E, r);
  const int tb = tail_begin(off, e, bm);
  if (r < tb) return *(const f32x4 *)(yp + (size_t)r * d + c);
  const float *q = tail + ((size_t)e * bm + (r - tb)) * d + c;
  f32x4 v = *(const f32x4 *)q;
  for (int sp = 1; sp < S; ++sp) v += *(const f32x4 *)(q + sp * plane);
  return v;
}

template <bool OUT_BF16>
__global__ __launch_bounds__(256) void combine_tail_kernel(
    const float *__restrict__ yp, const float *__restrict__ tail, int S, size_t plane,
    const int32_t *__restrict__ off, int E, int bm, const int32_t *__restrict__ inv,
    const float *__restrict__ w, int n, int k, int d, void *__restrict__ y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (t >= n || c >= d) return;
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  const unsigned R = (unsigned)n * (unsigned)k;
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const int r = inv[(size_t)t * k + j];
    if ((unsigned)r >= R) continue;
    const f32x4 v = pile_row4(yp, tail, S, plane, off, E, bm, r, d, c);
    acc[0] = fmaf(wj, v[0], acc[0]);
    acc[1] = fmaf(wj, v[1], acc[1]);
    acc[2] = fmaf(wj, v[2], acc[2]);
    acc[3] = fmaf(wj, v[3], acc[3]);
  }
  if constexpr (OUT_BF16) {
    u32x2 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3])};
    *(u32x2 *)((uint16_t *)y + (size_t)t * d + c) = o;
  } else {
    *(f32x4 *)((float *)y + (size_t)t * d + c) = acc;
  }
}

// The combine of bf16 pile outputs (each the f32 pile output rounded once),
// eight columns a thread (d % 8 == 0); with TAIL the rows of each pile's
// last row tile (bm-row tiles from offsets[e]) are instead the sum of their
// S f32 partial planes tail[s][e * bm + row][d], in split order.
template <bool OUT_BF16, bool TAIL>
__global__ __launch_bounds__(256) void combine_bf16in_kernel(
    const uint16_t *__restrict__ yp, const float *__restrict__ tail, int S, size_t plane,
    const int32_t *__restrict__ off, int E, int bm, const int32_t *__restrict__ inv,
    const float *__restrict__ w, int n, int k, int d, void *__restrict__ y) {
  const int t = blockIdx.y;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (t >= n || c >= d) return;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  const unsigned R = (unsigned)n * (unsigned)k;
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const int r = inv[(size_t)t * k + j];
    if ((unsigned)r >= R) continue;
    float v[8];
    bool planes = false;
    if constexpr (TAIL) {
      const int e = expert_of(off, E, r);
      const int tb = tail_begin(off, e, bm);
      if (r >= tb) {
        const float *q = tail + ((size_t)e * bm + (r - tb)) * d + c;
        f32x4 lo = *(const f32x4 *)q, hi = *(const f32x4 *)(q + 4);
        for (int sp = 1; sp < S; ++sp) {
          lo += *(const f32x4 *)(q + sp * plane);
          hi += *(const f32x4 *)(q + sp * plane + 4);
        }
        for (int i = 0; i < 4; ++i) {
          v[i] = lo[i];
          v[i + 4] = hi[i];
        }
        planes = true;
      }
    }
    if (!planes) {
      const u32x4 raw = *(const u32x4 *)(yp + (size_t)r * d + c);
      for (int i = 0; i < 4; ++i) {
        v[2 * i] = bf16_bits_to_f32(raw[i] & 0xffffu);
        v[2 * i + 1] = bf16_bits_to_f32(raw[i] >> 16);
      }
    }
    for (int i = 0; i < 8; ++i) acc[i] = fmaf(wj, v[i], acc[i]);
  }
  if constexpr (OUT_BF16) {
    const u32x4 o = {pack_bf16x2(acc[0], acc[1]), pack_bf16x2(acc[2], acc[3]),
                     pack_bf16x2(acc[4], acc[5]), pack_bf16x2(acc[6], acc[7])};
    *(u32x4 *)((uint16_t *)y + (size_t)t * d + c) = o;
  } else {
    float *o = (float *)y + (size_t)t * d + c;
    *(f32x4 *)o = f32x4{acc[0], acc[1], acc[2], acc[3]};
    *(f32x4 *)(o + 4) = f32x4{acc[4], acc[5], acc[6], acc[7]};
  }
}

template <bool TAIL>
hipError_t launch_bf16in(const uint16_t *yp, const float *tail, int S, size_t plane,
                         const int32_t *off, int E, int bm, const int32_t *inv, const float *w,
                         int n, int k, int d, void *y, bool out_bf16, hipStream_t st) {
  if (d % 8) return hipErrorInvalidValue;
  dim3 grid((d / 8 + 255) / 256, n);
  if (out_bf16)
    combine_bf16in_kernel<true, TAIL><<<grid, 256, 0, st>>>(yp, tail, S, plane, off, E, bm, inv, w,
                                                            n, k, d, y);
  else
    combine_bf16in_kernel<false, TAIL><<<grid, 256, 0, st>>>(yp, tail, S, plane, off, E, bm, inv,
                                                             w, n, k, d, y);
  return hipGetLastError();
}

// Block row (e, i): row i of pile e's last row tile, if the pile has it.
__global__ __launch_bounds__(256) void tail_sum_kernel(const float *__restrict__ tail, int S,
                                                       size_t plane,
                                                       const int32_t *__restrict__ off, int bm,
                                                       int d, float *__restrict__ yp) {
  const int e = blockIdx.y / bm, i = blockIdx.y % bm;
  const int c = (blockIdx.x * blockDim.x + threadIdx.x) * 4;
  const int tb = tail_begin(off, e, bm);
  if (off[e + 1] == off[e] || tb + i >= off[e + 1] || c >= d) return;
  const float *q = tail + ((size_t)e * bm + i) * d + c;
  f32x4 v = *(const f32x4 *)q;
  for (int sp = 1; sp < S; ++sp) v += *(const f32x4 *)(q + sp * plane);
  *(f32x4 *)(yp + (size_t)(tb + i) * d + c) = v;
}

// bf16 copy of an f32 array: 8 values a thread in the body, then the tail.
__global__ __launch_bounds__(256) void f32_to_bf16_kernel(const float *__restrict__ src,
                                                          uint16_t *__restrict__ dst,
                                                          size_t count) {
  const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 8;
  if (i + 8 <= count) {
    const f32x4 a = *(const f32x4 *)(src + i), b = *(const f32x4 *)(src + i + 4);
    const u32x4 o = {pack_bf16x2(a[0], a[1]), pack_bf16x2(a[2], a[3]), pack_bf16x2(b[0], b[1]),
                     pack_bf16x2(b[2], b[3])};
    *(u32x4 *)(dst + i) = o;
  } else {
    for (size_t j = i; j < count; ++j) dst[j] = (uint16_t)f32_to_bf16_bits(src[j]);
  }
}

}  // namespace

hipError_t launch_f32_to_bf16(const float *src, uint16_t *dst, size_t count, hipStream_t st) {
  if (count == 0) return hipSuccess;
  const size_t threads = (count + 7) / 8;
  f32_to_bf16_kernel<<<(unsigned)((threads + 255) / 256), 256, 0, st>>>(src, dst, count);
  return hipGetLastError();
}

hipError_t launch_splitk_combine(const float *part, int S, int R, const int32_t *inv,
                                 const float *w, int n, int k, int d, void *y, bool out_bf16,
                                 hipStream_t st) {
  dim3 grid((d / 4 + 255) / 256, n);
  const size_t plane = (size_t)R * d;
  if (out_bf16)
    splitk_combine_kernel<true><<<grid, 256, 0, st>>>(part, S, plane, inv, w, n, k, d, y);
  else
    splitk_combine_kernel<false><<<grid, 256, 0, st>>>(part, S, plane, inv, w, n, k, d, y);
  return hipGetLastError();
}

hipError_t launch_splitk_sum(const float *part, int S, int R, int d, float *yp, hipStream_t st) {
  const size_t total4 = (size_t)R * d / 4;
  splitk_sum_kernel<<<(unsigned)((total4 + 255) / 256), 256, 0, st>>>(part, S, (size_t)R * d,
                                                                       total4, yp);
  return hipGetLastError();
}

hipError_t launch_combine_tail(const void *y_perm, bool in_bf16, const float *tail, int S,
                               size_t plane, const int32_t *offsets, int E, int bm,
                               const int32_t *inv, const float *w, int n, int k, int d, void *y,
                               bool out_bf16, hipStream_t st) {
  if (in_bf16)
    return launch_bf16in<true>((const uint16_t *)y_perm, tail, S, plane, offsets, E, bm, inv, w, n,
                               k, d, y, out_bf16, st);
  if (d % 4) return hipErrorInvalidValue;
  dim3 grid((d / 4 + 255) / 256, n);
  if (out_bf16)
    combine_tail_kernel<true><<<grid, 256, 0, st>>>((const float *)y_perm, tail, S, plane, offsets,
                                                    E, bm, inv, w, n, k, d, y);
  else
    combine_tail_kernel<false><<<grid, 256, 0, st>>>((const float *)y_perm, tail, S, plane, offsets,
                                                     E, bm, inv, w, n, k, d, y);
  return hipGetLastError();
}

hipError_t launch_tail_sum(const float *tail, int S, size_t plane, const int32_t *offsets, int E,
                           int bm, int d, float *y_perm, hipStream_t st) {
  if (d % 4) return hipErrorInvalidValue;
  dim3 grid((d / 4 + 255) / 256, (unsigned)E * bm);
  tail_sum_kernel<<<grid, 256, 0, st>>>(tail, S, plane, offsets, bm, d, y_perm);
  return hipGetLastError();
}

hipError_t launch_combine(const void *y_perm, bool in_bf16, const int32_t *inv, const float *w,
                          int n, int k, int d, void *y, bool out_bf16, hipStream_t st) {
  if (in_bf16)
    return launch_bf16in<false>((const uint16_t *)y_perm, nullptr, 0, 0, nullptr, 0, 0, inv, w, n,
                                k, d, y, out_bf16, st);
  const float *yp = (const float *)y_perm;
  if (d % 4 == 0) {
    dim3 grid((d / 4 + 255) / 256, n);
    if (out_bf16)
      combine_vec4_kernel<true><<<grid, 256, 0, st>>>(yp, inv, w, n, k, d, y);
    else
      combine_vec4_kernel<false><<<grid, 256, 0, st>>>(yp, inv, w, n, k, d, y);
  } else {
    dim3 grid((d + 255) / 256, n);
    if (out_bf16)
      combine_scalar_kernel<true><<<grid, 256, 0, st>>>(yp, inv, w, n, k, d, y);
    else
      combine_scalar_kernel<false><<<grid, 256, 0, st>>>(yp, inv, w, n, k, d, y);
  }
  return hipGetLastError();
}

}  // namespace moe
