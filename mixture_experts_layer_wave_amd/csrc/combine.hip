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
// so the result does not depend on scheduling.
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
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const f32x4 v = *(const f32x4 *)(yp + (size_t)inv[(size_t)t * k + j] * d + c);
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
  float acc = 0.f;
  for (int j = 0; j < k; ++j)
    acc = fmaf(w[(size_t)t * k + j], yp[(size_t)inv[(size_t)t * k + j] * d + c], acc);
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
  for (int j = 0; j < k; ++j) {
    const float wj = w[(size_t)t * k + j];
    const float *src = part + (size_t)inv[(size_t)t * k + j] * d + c;
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

}  // namespace

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

hipError_t launch_combine(const float *y_perm, const int32_t *inv, const float *w, int n, int k,
                          int d, void *y, bool out_bf16, hipStream_t st) {
  if (d % 4 == 0) {
    dim3 grid((d / 4 + 255) / 256, n);
    if (out_bf16)
      combine_vec4_kernel<true><<<grid, 256, 0, st>>>(y_perm, inv, w, n, k, d, y);
    else
      combine_vec4_kernel<false><<<grid, 256, 0, st>>>(y_perm, inv, w, n, k, d, y);
  } else {
    dim3 grid((d + 255) / 256, n);
    if (out_bf16)
      combine_scalar_kernel<true><<<grid, 256, 0, st>>>(y_perm, inv, w, n, k, d, y);
    else
      combine_scalar_kernel<false><<<grid, 256, 0, st>>>(y_perm, inv, w, n, k, d, y);
  }
  return hipGetLastError();
}

}  // namespace moe
