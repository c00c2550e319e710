// Dispatch: regroup (token, slot) pairs into per-expert piles.
//
// "How Mixture of Experts Scales Model Parameters", section "The forward
// pass: dispatch, then combine": tokens sent to the same expert are pulled
// out, in their original order, into that expert's input matrix; a pile can
// be empty, and pile sizes depend on the data only.
//
// One workgroup of 1024 threads does the whole job deterministically (see
// dispatch_block in route_dev.h).
#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {
namespace {

__global__ __launch_bounds__(1024) void dispatch_kernel(const int32_t *__restrict__ idx, int R,
                                                        int k, int E, int nbits,
                                                        int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ perm,
                                                        int32_t *__restrict__ inv) {
  extern __shared__ int smem[];
  dispatch_block<16>(idx, R, k, E, nbits, counts, offsets, perm, inv, smem);
}

// Small batches: top-k of every token (one group of lanes per token, see
// topk_token_t) and the dispatch in one workgroup, saving a launch on the
// decode path.  n <= kRouteSmallN, so n * k <= 2048 pairs: two register
// chunks.
template <int PER>
__global__ __launch_bounds__(1024) void route_dispatch_kernel(
    const float *__restrict__ part, int S, int n, int E, int k, int renorm, int nbits,
    int32_t *__restrict__ idx, float *__restrict__ w, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv) {
  extern __shared__ int smem[];
  int *s_idx = smem + dispatch_lds_ints(E);  // [n * k] chosen experts
  const int G = topk_group(E);
  for (int t0 = 0; t0 < n; t0 += kDispThreads / G)  // uniform trip count
    topk_token_t<PER>(part, S, (size_t)n * E, t0 + threadIdx.x / G, n, E, k, renorm, idx, w,
                      nullptr, s_idx);
  lds_barrier();
  dispatch_block<2>(s_idx, n * k, k, E, nbits, counts, offsets, perm, inv, smem);
}

__global__ __launch_bounds__(256) void gather_rows_kernel(const uint32_t *__restrict__ x,
                                                          const int32_t *__restrict__ perm,
                                                          uint32_t *__restrict__ xp, int R,
                                                          int words) {
  const int r = blockIdx.x;
  if (r >= R) return;
  const uint32_t *src = x + (size_t)perm[r] * words;
  uint32_t *dst = xp + (size_t)r * words;
  if ((words & 3) == 0) {
    const u32x4 *s4 = (const u32x4 *)src;
    u32x4 *d4 = (u32x4 *)dst;
    for (int i = threadIdx.x; i < words / 4; i += blockDim.x) d4[i] = s4[i];
  } else {
    for (int i = threadIdx.x; i < words; i += blockDim.x) dst[i] = src[i];
  }
}

}  // namespace

static int id_bits(int E) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  return nbits;
}

template <typename K>
static hipError_t allow_lds(K kern, size_t lds) {
  if (lds <= 64 * 1024) return hipSuccess;
  return hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                             (int)lds);
}

hipError_t launch_dispatch(const int32_t *idx, int n, int k, int E, int32_t *counts,
                           int32_t *offsets, int32_t *perm, int32_t *inv, hipStream_t st) {
  const size_t lds = sizeof(int) * (size_t)dispatch_lds_ints(E);
  hipError_t err = allow_lds(dispatch_kernel, lds);
  if (err != hipSuccess) return err;
  dispatch_kernel<<<1, kDispThreads, lds, st>>>(idx, n * k, k, E, id_bits(E), counts, offsets,
                                                perm, inv);
  return hipGetLastError();
}

template <int PER>
static hipError_t route_dispatch_per(const float *part, int splits, int n, int E, int k,
                                     bool renorm, int32_t *idx, float *w, int32_t *counts,
                                     int32_t *offsets, int32_t *perm, int32_t *inv,
                                     hipStream_t st) {
  const size_t lds = sizeof(int) * ((size_t)dispatch_lds_ints(E) + (size_t)n * k);
  hipError_t err = allow_lds(route_dispatch_kernel<PER>, lds);
  if (err != hipSuccess) return err;
  route_dispatch_kernel<PER><<<1, kDispThreads, lds, st>>>(part, splits, n, E, k, renorm ? 1 : 0,
                                                           id_bits(E), idx, w, counts, offsets,
                                                           perm, inv);
  return hipGetLastError();
}

hipError_t launch_route_dispatch(const float *part, int splits, int n, int E, int k, bool renorm,
                                 int32_t *idx, float *w, int32_t *counts, int32_t *offsets,
                                 int32_t *perm, int32_t *inv, hipStream_t st) {
  if (n > kRouteSmallN || n * k > 2 * kDispThreads) return hipErrorInvalidValue;
  switch (topk_per(E)) {
    case 2: return route_dispatch_per<2>(part, splits, n, E, k, renorm, idx, w, counts, offsets, perm, inv, st);
    case 4: return route_dispatch_per<4>(part, splits, n, E, k, renorm, idx, w, counts, offsets, perm, inv, st);
    default:
      return route_dispatch_per<MOE_MAX_E / MOE_WAVE>(part, splits, n, E, k, renorm, idx, w,
                                                       counts, offsets, perm, inv, st);
  }
}

hipError_t launch_gather_rows(const void *x, const int32_t *perm, void *x_perm, int R,
                              int row_bytes, hipStream_t st) {
  if (R == 0) return hipSuccess;
  gather_rows_kernel<<<R, 256, 0, st>>>((const uint32_t *)x, perm, (uint32_t *)x_perm, R,
                                        row_bytes / 4);
  return hipGetLastError();
}

}  // namespace moe
