// Dispatch: regroup (token, slot) pairs into per-expert piles.
//
// "How Mixture of Experts Scales Model Parameters", section "The forward
// pass: dispatch, then combine": tokens sent to the same expert are pulled
// out, in their original order, into that expert's input matrix; a pile can
// be empty, and pile sizes depend on the data only.
//
// Deterministic in all three forms: one wave for up to 256 pairs
// (dispatch_wave in route_dev.h, or dispatch_wave_small for a few pairs
// of at most 128 experts); one 1024-thread workgroup (dispatch_block)
// when no scratch is given; otherwise two passes over chunks of 1024 pairs,
// one workgroup per chunk: (1) each chunk's per-expert counts and each
// pair's stable rank among its chunk's pairs of the same expert, (2) every
// workgroup adds up the counts of the chunks before its own and moves its
// pairs to offsets[e] + (pairs of e in earlier chunks) + rank.
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

// Pass 1 of the chunked dispatch: chunk b = pairs [1024 b, 1024 b + 1024).
// A lane's rank among same-expert lanes of its wave comes from ballots on
// the bits of the expert id; the 16 waves' counts, scanned per expert, give
// each pair its rank in the chunk (parked in inv) and the chunk's counts
// (hist[b][E]).
__global__ __launch_bounds__(kDispThreads) void dispatch_chunk_rank_kernel(
    const int32_t *__restrict__ idx, int R, int E, int nbits, int32_t *__restrict__ hist,
    int32_t *__restrict__ inv) {
  extern __shared__ int smem[];
  int *s_wc = smem;                    // [16][E] per-wave counts
  int *s_base = s_wc + kDispWaves * E;  // [16][E] first rank of (wave, expert)
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int r = blockIdx.x * kDispThreads + tid;
  for (int i = tid; i < kDispWaves * E; i += kDispThreads) s_wc[i] = 0;
  const int e = r < R ? idx[r] : -1;
  const bool valid = e >= 0 && e < E;
  __syncthreads();
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  uint64_t same = __ballot(valid);
  for (int b = 0; b < nbits; ++b) {
    const bool bit = valid && ((e >> b) & 1);
    const uint64_t bal = __ballot(bit);
    same &= bit ? bal : ~bal;
  }
  const int rank = __popcll(same & lt_mask);
  if (valid && rank == 0) s_wc[wave * E + e] = __popcll(same);
  __syncthreads();
  for (int ee = tid; ee < E; ee += kDispThreads) {
    int run = 0;
#pragma unroll
    for (int wv = 0; wv < kDispWaves; ++wv) {
      s_base[wv * E + ee] = run;
      run += s_wc[wv * E + ee];
    }
    hist[(size_t)blockIdx.x * E + ee] = run;
  }
  __syncthreads();
  if (valid) inv[r] = s_base[wave * E + e] + rank;
}

// Pass 2: every workgroup sums the chunk counts (all chunks for the pile
// sizes, the chunks before its own for its base), scans the sizes into
// offsets, and moves its chunk's pairs.  Workgroup 0 writes counts and
// offsets.
__global__ __launch_bounds__(kDispThreads) void dispatch_chunk_move_kernel(
    const int32_t *__restrict__ idx, int R, int k, int E, const int32_t *__restrict__ hist,
    int32_t *__restrict__ counts, int32_t *__restrict__ offsets, int32_t *__restrict__ perm,
    int32_t *__restrict__ inv) {
  extern __shared__ int smem[];
  int *s_tot = smem;       // [E] pile sizes
  int *s_base = s_tot + E;  // [E] first pile row of this chunk's pairs of e
  __shared__ int s_used;    // rows in all piles together
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int b = blockIdx.x, nb = gridDim.x;
  for (int e = tid; e < E; e += kDispThreads) {
    int tot = 0, pre = 0;
    for (int c = 0; c < nb; ++c) {
      const int h = hist[(size_t)c * E + e];
      pre += c < b ? h : 0;
      tot += h;
    }
    s_tot[e] = tot;
    s_base[e] = pre;
  }
  __syncthreads();
  if (wave == 0) {
    int carry = 0;
    for (int e0 = 0; e0 < E; e0 += MOE_WAVE) {
      const int e = e0 + lane;
      const int c = e < E ? s_tot[e] : 0;
      const int incl = wave_incl_scan(c);
      if (e < E) {
        const int off = carry + incl - c;
        s_base[e] += off;
        if (b == 0) {
          counts[e] = c;
          offsets[e] = off;
        }
      }
      carry += __builtin_amdgcn_readlane(incl, MOE_WAVE - 1);
    }
    if (b == 0 && lane == 0) offsets[E] = carry;
    if (lane == 0) s_used = carry;
  }
  __syncthreads();
  const int r = b * kDispThreads + tid;
  if (r < R) {
    const int e = idx[r];
    if (e >= 0 && e < E) {
      const int pos = s_base[e] + inv[r];
      perm[pos] = r / k;
      inv[r] = pos;
    } else {
      inv[r] = -1;  // id outside [0, E): the pair is in no pile
    }
  }
  // Pile rows past the last pile (one per skipped pair) hold -1; every
  // workgroup clears the part of that tail inside its own chunk.
  if (r < R && r >= s_used) perm[r] = -1;
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
  if (threadIdx.x < MOE_WAVE) {
    if (R <= kDispTinyR && E <= 2 * MOE_WAVE)
      dispatch_wave_small<2>(idx, R, k, E, s_cnt, s_off, s_perm, s_inv, nullptr);
    else
      dispatch_wave(idx, R, k, E, nbits, s_cnt, s_off, s_perm, s_inv);
  }
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

// Top-k and dispatch of a small batch in one workgroup (route_small_ok: one
// pass of top-k over the 256 threads): the top-k rounds of the router's
// top-k pass (topk_token_t) also leave each token's experts in LDS, where
// one wave then builds the piles as dispatch_small_kernel does.  Same idx, w
// and piles as the two kernels, one launch fewer on the decode path (n = 1:
// 41.6 -> 41.0 us per layer).  With two passes (n = 8 at 128 experts) it
// was 3% slower than the two kernels.
template <int PER>
__global__ __launch_bounds__(256) void route_small_kernel(
    const float *__restrict__ part, int S, int n, int E, int k, int renorm, int nbits,
    int32_t *__restrict__ idx, float *__restrict__ w, int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ perm, int32_t *__restrict__ inv) {
  extern __shared__ int smem[];
  const int R = n * k;
  int *s_idx = smem, *s_cnt = s_idx + R, *s_off = s_cnt + E, *s_perm = s_off + E + 1,
      *s_inv = s_perm + R;
  const int G = topk_group(E);
  for (int t0 = 0; t0 < n; t0 += 256 / G)  // every lane takes part (group reductions)
    topk_token_t<PER>(part, S, (size_t)n * E, t0 + (int)threadIdx.x / G, n, E, k, renorm, idx, w,
                      nullptr, s_idx);
  __syncthreads();
  if (threadIdx.x < MOE_WAVE) {
    if (R <= kDispTinyR && E <= 2 * MOE_WAVE)
      dispatch_wave_small<2>(s_idx, R, k, E, s_cnt, s_off, s_perm, s_inv, nullptr);
    else
      dispatch_wave(s_idx, R, k, E, nbits, s_cnt, s_off, s_perm, s_inv);
  }
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

// x_perm[r] = x[perm[r]]; a row whose perm entry is outside [0, n) (a pile
// row past the last pile) is written as zeros.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint32_t *__restrict__ x,
                                                          const int32_t *__restrict__ perm,
                                                          uint32_t *__restrict__ xp, int R,
                                                          int n, int words) {
  const int r = blockIdx.x;
  if (r >= R) return;
  const int t = perm[r];
  uint32_t *dst = xp + (size_t)r * words;
  if (t < 0 || t >= n) {
    for (int i = threadIdx.x; i < words; i += blockDim.x) dst[i] = 0u;
    return;
  }
  const uint32_t *src = x + (size_t)t * words;
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

size_t dispatch_scratch_bytes(int n, int k, int E) {
  const long long R = (long long)n * k;
  if (R <= kDispChunkMinR) return 0;
  return (size_t)((R + kDispThreads - 1) / kDispThreads) * E * sizeof(int32_t);
}

hipError_t launch_dispatch(const int32_t *idx, int n, int k, int E, int32_t *counts,
                           int32_t *offsets, int32_t *perm, int32_t *inv, int32_t *scratch,
                           hipStream_t st) {
  const int R = n * k;
  if (scratch && R > kDispChunkMinR) {
    const int nb = (R + kDispThreads - 1) / kDispThreads;
    const size_t lds1 = sizeof(int) * 2 * (size_t)kDispWaves * E;
    hipError_t err = allow_lds(dispatch_chunk_rank_kernel, lds1);
    if (err != hipSuccess) return err;
    dispatch_chunk_rank_kernel<<<nb, kDispThreads, lds1, st>>>(idx, R, E, id_bits(E), scratch, inv);
    err = hipGetLastError();
    if (err != hipSuccess) return err;
    dispatch_chunk_move_kernel<<<nb, kDispThreads, sizeof(int) * 2 * (size_t)E, st>>>(
        idx, R, k, E, scratch, counts, offsets, perm, inv);
    return hipGetLastError();
  }
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

bool route_small_ok(int n, int k, int E) {
  return n * k <= kDispSmallR && n * topk_group(E) <= 256;
}

hipError_t launch_route_small(const float *part, int splits, int n, int E, int k, bool renorm,
                              int32_t *idx, float *w, int32_t *counts, int32_t *offsets,
                              int32_t *perm, int32_t *inv, hipStream_t st) {
  if (!route_small_ok(n, k, E)) return hipErrorInvalidValue;
  const size_t lds = sizeof(int) * (2 * (size_t)E + 1 + 3 * (size_t)n * k);
  const int rn = renorm ? 1 : 0;
  hipError_t err = hipSuccess;
  switch (topk_per(E)) {
    case 2:
      err = allow_lds(route_small_kernel<2>, lds);
      if (err == hipSuccess)
        route_small_kernel<2><<<1, 256, lds, st>>>(part, splits, n, E, k, rn, id_bits(E), idx, w,
                                                   counts, offsets, perm, inv);
      break;
    case 4:
      err = allow_lds(route_small_kernel<4>, lds);
      if (err == hipSuccess)
        route_small_kernel<4><<<1, 256, lds, st>>>(part, splits, n, E, k, rn, id_bits(E), idx, w,
                                                   counts, offsets, perm, inv);
      break;
    default:
      err = allow_lds(route_small_kernel<MOE_MAX_E / MOE_WAVE>, lds);
      if (err == hipSuccess)
        route_small_kernel<MOE_MAX_E / MOE_WAVE><<<1, 256, lds, st>>>(
            part, splits, n, E, k, rn, id_bits(E), idx, w, counts, offsets, perm, inv);
  }
  if (err != hipSuccess) return err;
  return hipGetLastError();
}

hipError_t launch_active_experts(const int32_t *counts, int E, int32_t *active,
                                 int32_t *n_active, hipStream_t st) {
  active_experts_kernel<<<1, MOE_WAVE, 0, st>>>(counts, E, active, n_active);
  return hipGetLastError();
}

hipError_t launch_gather_rows(const void *x, const int32_t *perm, void *x_perm, int R, int n,
                              int row_bytes, hipStream_t st) {
  if (R == 0) return hipSuccess;
  gather_rows_kernel<<<R, 256, 0, st>>>((const uint32_t *)x, perm, (uint32_t *)x_perm, R, n,
                                        row_bytes / 4);
  return hipGetLastError();
}

}  // namespace moe
