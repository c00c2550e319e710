// Dispatch: regroup (token, slot) pairs into per-expert piles.
//
// "How Mixture of Experts Scales Model Parameters", section "The forward
// pass: dispatch, then combine": tokens sent to the same expert are pulled
// out, in their original order, into that expert's input matrix; a pile can
// be empty, and pile sizes depend on the data only.
//
// One workgroup does the whole job deterministically: one wave for up to 256
// pairs (dispatch_wave in route_dev.h), else 1024 threads (dispatch_block).
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

// Small batches (n * k <= 256 pairs): one wave builds the piles in LDS
// (dispatch_wave), then the workgroup writes them out.
__global__ __launch_bounds__(256) void dispatch_small_kernel(const int32_t *__restrict__ idx,
                                                             int R, int k, int E, int nbits,
                                                             int32_t *__restrict__ counts,
                                                             int32_t *__restrict__ offsets,
                                                             int32_t *__restrict__ perm,
                                                             int32_t *__restrict__ inv) {
  extern __shared__ int smem[];
  int *s_cnt = smem, *s_off = s_cnt + E, *s_perm = s_off + E + 1, *s_inv = s_perm + R;
  if (threadIdx.x < MOE_WAVE) dispatch_wave(idx, R, k, E, nbits, s_cnt, s_off, s_perm, s_inv);
  __syncthreads();
  for (int e = threadIdx.x; e <= E; e += blockDim.x) {
    if (e < E) counts[e] = s_cnt[e];
    offsets[e] = s_off[e];
  }
  for (int r = threadIdx.x; r < R; r += blockDim.x) {
    perm[r] = s_perm[r];
    inv[r] = s_inv[r];
  }
}

// Compaction of the experts with a non-empty pile, in expert order: per
// chunk of 64 experts a ballot gives each active expert its rank.
__global__ __launch_bounds__(64) void active_experts_kernel(const int32_t *__restrict__ counts,
                                                            int E, int32_t *__restrict__ active,
                                                            int32_t *__restrict__ n_active) {
  const int lane = threadIdx.x;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int base = 0;
  for (int e0 = 0; e0 < E; e0 += MOE_WAVE) {
    const int e = e0 + lane;
    const bool on = e < E && counts[e] > 0;
    const uint64_t bits = __ballot(on);
    if (on) active[base + __popcll(bits & lt_mask)] = e;
    base += __popcll(bits);
  }
  for (int j = base + lane; j < E; j += MOE_WAVE) active[j] = -1;
  if (lane == 0) *n_active = base;
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
  if (n * k <= kDispSmallR) {
    const size_t lds_s = sizeof(int) * (2 * (size_t)E + 1 + 2 * (size_t)n * k);
    hipError_t err = allow_lds(dispatch_small_kernel, lds_s);
    if (err != hipSuccess) return err;
    dispatch_small_kernel<<<1, 256, lds_s, st>>>(idx, n * k, k, E, id_bits(E), counts, offsets,
                                                 perm, inv);
    return hipGetLastError();
  }
  const size_t lds = sizeof(int) * (size_t)dispatch_lds_ints(E);
  hipError_t err = allow_lds(dispatch_kernel, lds);
  if (err != hipSuccess) return err;
  dispatch_kernel<<<1, kDispThreads, lds, st>>>(idx, n * k, k, E, id_bits(E), counts, offsets,
                                                perm, inv);
  return hipGetLastError();
}

hipError_t launch_active_experts(const int32_t *counts, int E, int32_t *active,
                                 int32_t *n_active, hipStream_t st) {
  active_experts_kernel<<<1, MOE_WAVE, 0, st>>>(counts, E, active, n_active);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *x, const int32_t *perm, void *x_perm, int R,
                              int row_bytes, hipStream_t st) {
  if (R == 0) return hipSuccess;
  gather_rows_kernel<<<R, 256, 0, st>>>((const uint32_t *)x, perm, (uint32_t *)x_perm, R,
                                        row_bytes / 4);
  return hipGetLastError();
}

}  // namespace moe
