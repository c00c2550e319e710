// Dispatch: regroup (token, slot) pairs into per-expert piles.
//
// "How Mixture of Experts Scales Model Parameters", section "The forward
// pass: dispatch, then combine": tokens sent to the same expert are pulled
// out, in their original order, into that expert's input matrix; a pile can
// be empty, and pile sizes depend on the data only.
//
// One workgroup of 1024 threads does the whole job deterministically:
//   1. histogram of expert ids in LDS (integer atomics: order-independent),
//   2. exclusive scan -> offsets,
//   3. stable placement in chunks of 1024 pairs, in (token, slot) order.  A
//      lane's rank among same-expert lanes of its wave comes from ballots on
//      the bits of the expert id; ranks across the 16 waves of the chunk come
//      from a per-wave count table; a per-expert cursor carries the count of
//      earlier chunks.  No atomics decide positions, so the result is the
//      unique stable grouping.
#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kDispThreads = 1024;
constexpr int kDispWaves = kDispThreads / MOE_WAVE;

__global__ __launch_bounds__(1024) void dispatch_kernel(const int32_t *__restrict__ idx, int R,
                                                        int k, int E, int nbits,
                                                        int32_t *__restrict__ counts,
                                                        int32_t *__restrict__ offsets,
                                                        int32_t *__restrict__ perm,
                                                        int32_t *__restrict__ inv) {
  extern __shared__ int smem[];
  int *s_cnt = smem;               // [E]   histogram
  int *s_cur = s_cnt + E;          // [E]   placement cursor (starts at offsets)
  int *s_wc = s_cur + E;           // [16][E] per-wave counts of the current chunk
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;

  for (int e = tid; e < E; e += kDispThreads) s_cnt[e] = 0;
  for (int i = tid; i < kDispWaves * E; i += kDispThreads) s_wc[i] = 0;
  __syncthreads();
  for (int r = tid; r < R; r += kDispThreads) {
    const int e = idx[r];
    if (e >= 0 && e < E) atomicAdd(&s_cnt[e], 1);
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < E; base += MOE_WAVE) {
      const int e = base + lane;
      const int c = e < E ? s_cnt[e] : 0;
      int incl = c;
#pragma unroll
      for (int o = 1; o < MOE_WAVE; o <<= 1) {
        const int v = __shfl_up(incl, o, 64);
        if (lane >= o) incl += v;
      }
      if (e < E) {
        s_cur[e] = carry + incl - c;
        counts[e] = c;
        offsets[e] = carry + incl - c;
      }
      carry += __shfl(incl, MOE_WAVE - 1, 64);
    }
    if (lane == 0) offsets[E] = carry;
  }
  __syncthreads();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < R; c0 += kDispThreads) {
    const int r = c0 + tid;
    int e = r < R ? idx[r] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & lt_mask);
    if (valid && rank == 0) s_wc[wave * E + e] = __popcll(same);
    __syncthreads();
    if (valid) {
      int base = s_cur[e];
      for (int w = 0; w < wave; ++w) base += s_wc[w * E + e];
      const int pos = base + rank;
      perm[pos] = r / k;
      inv[r] = pos;
    }
    __syncthreads();
    for (int ee = tid; ee < E; ee += kDispThreads) {
      int add = 0;
      for (int w = 0; w < kDispWaves; ++w) {
        add += s_wc[w * E + ee];
        s_wc[w * E + ee] = 0;
      }
      s_cur[ee] += add;
    }
    __syncthreads();
  }
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

hipError_t launch_dispatch(const int32_t *idx, int n, int k, int E, int32_t *counts,
                           int32_t *offsets, int32_t *perm, int32_t *inv, hipStream_t st) {
  int nbits = 0;
  while ((1 << nbits) < E) ++nbits;
  const size_t lds = sizeof(int) * (size_t)E * (2 + kDispWaves);
  if (lds > 64 * 1024) {
    hipError_t err = hipFuncSetAttribute((const void *)dispatch_kernel,
                                         hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (err != hipSuccess) return err;
  }
  dispatch_kernel<<<1, kDispThreads, lds, st>>>(idx, n * k, k, E, nbits, counts, offsets, perm,
                                                inv);
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
