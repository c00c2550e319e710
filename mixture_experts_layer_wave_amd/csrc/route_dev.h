// Device-side building blocks shared by the router and dispatch kernels.
//
//   topk_token:   softmax over E logits, top-k selection and combine weights
//                 for one token, executed by one wave ("How Mixture of Experts
//                 Scales Model Parameters", sections "Routing: a router scores
//                 the experts, and the top one runs" and "Top-K: several
//                 experts, added up by weight"; the softmax subtracts the row
//                 maximum first, "Why FlashAttention is So Fast", section "A
//                 fused kernel, and an overflow problem").
//   dispatch_block: stable regrouping of (token, slot) pairs into per-expert
//                 piles by one 1024-thread workgroup (section "The forward
//                 pass: dispatch, then combine").
#pragma once

#include <type_traits>

#include "common.h"

namespace moe {


// Lane-group width for E experts: the next power of two >= E, at most 64.
__host__ __device__ constexpr int topk_group(int E) {
  int g = 1;
  while (g < E && g < MOE_WAVE) g <<= 1;
  return g;
}

// Reductions over aligned groups of G lanes (G a power of two <= 64), with
// the result in every lane of the group.  Within a 16-lane row the steps are
// DPP lane permutations (lane pairs 1 and 2 apart, then the 8- and 16-lane
// mirrors), which cost a few cycles where a cross-lane shuffle through the
// LDS crossbar costs a memory round trip; rows are then combined with
// readlane.  The combination order is fixed, so results are deterministic.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
  return __builtin_amdgcn_update_dpp(v, v, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __builtin_bit_cast(float, dpp_i<CTRL>(__builtin_bit_cast(int, v)));
}
constexpr int kDppXor1 = 0xB1;        // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;        // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141; // lane i <-> 7 - i within 8
constexpr int kDppMirror = 0x140;     // lane i <-> 15 - i within 16

template <typename T, typename Op>
__device__ __forceinline__ T group_reduce(T v, int G, Op op) {
  auto dpp = [](T x, auto ctrl_tag) {
    constexpr int C = decltype(ctrl_tag)::value;
    if constexpr (sizeof(T) == 4 && __is_same(T, float)) return dpp_f<C>(x);
    else return (T)dpp_i<C>((int)x);
  };
  if (G >= 2) v = op(v, dpp(v, std::integral_constant<int, kDppXor1>{}));
  if (G >= 4) v = op(v, dpp(v, std::integral_constant<int, kDppXor2>{}));
  if (G >= 8) v = op(v, dpp(v, std::integral_constant<int, kDppHalfMirror>{}));
  if (G >= 16) v = op(v, dpp(v, std::integral_constant<int, kDppMirror>{}));
  if (G >= 32) {
    const int lane = threadIdx.x & 63;
    const T r0 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 0));
    const T r1 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 16));
    const T r2 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 32));
    const T r3 = __builtin_bit_cast(T, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 48));
    if (G == 64) v = op(op(r0, r1), op(r2, r3));
    else v = lane < 32 ? op(r0, r1) : op(r2, r3);
  }
  return v;
}
__device__ __forceinline__ float group_max(float v, int G) {
  return group_reduce(v, G, [](float a, float b) { return fmaxf(a, b); });
}
__device__ __forceinline__ float group_sum(float v, int G) {
  return group_reduce(v, G, [](float a, float b) { return a + b; });
}
__device__ __forceinline__ int group_min_i(int v, int G) {
  return group_reduce(v, G, [](int a, int b) { return a < b ? a : b; });
}
// Best (value, lowest index) of the group: the maximum value, then the
// smallest index among the lanes holding it.
__device__ __forceinline__ void group_argmax(float &v, int &i, int G) {
  const float m = group_max(v, G);
  i = group_min_i(v == m ? i : 0x7fffffff, G);
  v = m;
}

// One token per group of G = topk_group(E) lanes (64 / G tokens per wave;
// every lane of the wave must call it, with t >= n marking idle groups).
// The token's logits are the sum, in split order, of S partial rows
// part[s * part_stride + t * E + e] (S = 1: the logits themselves).  Lane
// l of a group owns experts l, l + G, ...; each of the k rounds takes the
// group-wide best (value, lowest index) among experts not yet taken.
// Weights: exp(z - max) over the sum for all E, or over the chosen k when
// renormalising.  If logits_out is given the summed logits are stored too.
// PER = expert slots per lane (a compile-time bound on ceil(E / G)).
template <int PER>
__device__ __forceinline__ void topk_token_t(const float *__restrict__ part, int S,
                                             size_t part_stride, int t, int n, int E, int k,
                                             int renorm, int32_t *__restrict__ idx,
                                             float *__restrict__ w,
                                             float *__restrict__ logits_out, int *lds_idx) {
  constexpr int kTopkPer = PER;
  const int G = topk_group(E);
  const int gl = (threadIdx.x & 63) & (G - 1);  // lane within the group
  const bool live = t < n;
  const float NEG = -__builtin_inff();
  float v[kTopkPer];
  const float *pz = part + (size_t)t * E + gl;
  // Split-major: each split's loads for all expert slots are independent,
  // and every slot accumulates its splits in order (deterministic).  The
  // sum starts from -0, which added to any value gives that value, so the
  // first split needs no load of its own ahead of the batch (one round trip
  // to memory instead of two when the splits fit one batch).
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) v[j] = (live && gl + G * j < E) ? -0.f : NEG;
  constexpr int kBatch = kTopkPer >= 32 ? 1 : 32 / kTopkPer;  // splits loaded per batch
  for (int s0 = 0; s0 < S; s0 += kBatch) {
    float q[kBatch][kTopkPer];
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int j = 0; j < kTopkPer; ++j)
        q[u][j] = (s0 + u < S && live && gl + G * j < E)
                      ? pz[(size_t)(s0 + u) * part_stride + G * j] : 0.f;
#pragma unroll
    for (int u = 0; u < kBatch; ++u)
#pragma unroll
      for (int j = 0; j < kTopkPer; ++j)
        if (s0 + u < S) v[j] += q[u][j];
  }
  if (logits_out) {
#pragma unroll
    for (int j = 0; j < kTopkPer; ++j)
      if (live && gl + G * j < E) logits_out[(size_t)t * E + gl + G * j] = v[j];
  }
  // A NaN logit ranks below every number: it takes part as -inf.  A round
  // whose best value is -inf then picks the lowest untaken expert, so every
  // chosen id lies in [0, E) whatever the logits hold.
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) v[j] = v[j] == v[j] ? v[j] : NEG;
  float m = NEG;
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j) m = fmaxf(m, v[j]);
  m = group_max(m, G);
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < kTopkPer; ++j)
    if (live && gl + G * j < E) sum += expf(v[j] - m);
  sum = group_sum(sum, G);

  // Rounds: the group maximum over experts not yet taken (round 0 reuses the
  // softmax maximum), then the lowest expert index holding it, found with
  // ballots in index order (slot j covers experts j G .. j G + G - 1).
  const int lane = threadIdx.x & 63;
  const int gbase = lane & ~(G - 1);
  const uint64_t gmask = G == 64 ? ~0ull : (((1ull << G) - 1) << gbase);
  uint32_t taken = 0;
  float my_v = NEG;
  int my_i = 0;
  for (int r = 0; r < k; ++r) {
    float mx = m;
    if (r > 0) {
      float bv = NEG;
#pragma unroll
      for (int j = 0; j < kTopkPer; ++j)
        if (gl + G * j < E && !((taken >> j) & 1u)) bv = fmaxf(bv, v[j]);
      mx = group_max(bv, G);
    }
    int bi = 0x7fffffff;
#pragma unroll
    for (int j = 0; j < kTopkPer; ++j) {
      const bool hit = live && gl + G * j < E && !((taken >> j) & 1u) && v[j] == mx;
      const uint64_t bits = __ballot(hit) & gmask;
      if (bi == 0x7fffffff && bits) bi = G * j + (__ffsll((long long)bits) - 1 - gbase);
    }
    if (bi < E && (bi & (G - 1)) == gl) taken |= 1u << (bi / G);
    if (gl == r) {
      my_v = mx;
      my_i = bi;
    }
  }
  // k <= G always (k <= E <= G, or G = 64 >= 32 >= k).
  const float num = gl < k ? expf(my_v - m) : 0.f;
  float den = sum;
  if (renorm) den = group_sum(num, G);
  if (live && gl < k) {
    idx[(size_t)t * k + gl] = my_i;
    w[(size_t)t * k + gl] = num / den;
    if (lds_idx) lds_idx[t * k + gl] = my_i;
  }
}

// Expert slots per lane for E experts: the compile-time bound that
// topk_token_t is instantiated with (2, 4 or 16).
__host__ __device__ constexpr int topk_per(int E) {
  return E <= 2 * MOE_WAVE ? 2 : (E <= 4 * MOE_WAVE ? 4 : MOE_MAX_E / MOE_WAVE);
}

constexpr int kDispThreads = 1024;
constexpr int kDispWaves = kDispThreads / MOE_WAVE;

// Rows in all piles together: offsets[E - 1] + counts[E - 1] from LDS.
__device__ __forceinline__ int s_cur_total(const int *s_off, const int *s_cur, int E) {
  return s_off[E - 1] + s_cur[E - 1];
}

// LDS ints needed by dispatch_block.
__host__ __device__ constexpr int dispatch_lds_ints(int E) { return E * (2 + 2 * kDispWaves); }

// Whole workgroup of kDispThreads, deterministic:
//   1. stable ranks: the pairs are taken in chunks of 1024 in (token, slot)
//      order.  A lane's rank among same-expert lanes of its wave comes from
//      ballots on the bits of the expert id; a per-wave count table, scanned
//      per expert, gives each (wave, expert) its first rank in the chunk, and
//      a per-expert cursor carries the earlier chunks;
//   2. the cursors are now the pile sizes: exclusive scan -> offsets;
//   3. every pair moves to offsets[e] + rank (perm, inv).
// No atomics decide positions, so the result is the unique stable grouping.
// Ids outside [0, E) are skipped: their pairs get inv = -1, and the pile
// rows past the last pile get perm = -1.  The ids and ranks of up to RC chunks
// stay in registers; longer inputs park ranks in inv[] (each thread reads
// back only its own entries).  Barriers order LDS only.  `idx` may point to
// LDS or global memory.
template <int RC>
__device__ __forceinline__ void dispatch_block(const int32_t *__restrict__ idx, int R, int k,
                                               int E, int nbits, int32_t *__restrict__ counts,
                                               int32_t *__restrict__ offsets,
                                               int32_t *__restrict__ perm,
                                               int32_t *__restrict__ inv, int *smem) {
  int *s_cur = smem;                  // [E]     running count per expert
  int *s_off = s_cur + E;             // [E]     offsets
  int *s_wc = s_off + E;              // [16][E] per-wave counts of the current chunk
  int *s_base = s_wc + kDispWaves * E;  // [16][E] first rank of (wave, expert) in the chunk
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const bool in_regs = R <= RC * kDispThreads;

  for (int e = tid; e < E; e += kDispThreads) s_cur[e] = 0;
  for (int i = tid; i < kDispWaves * E; i += kDispThreads) s_wc[i] = 0;
  int ids[RC], rk[RC];
#pragma unroll
  for (int q = 0; q < RC; ++q) {
    const int rq = q * kDispThreads + tid;
    ids[q] = (in_regs && rq < R) ? idx[rq] : -1;
    rk[q] = 0;
  }
  lds_barrier();

  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  for (int c0 = 0; c0 < R; c0 += kDispThreads) {
    const int ci = c0 / kDispThreads;
    const int r = c0 + tid;
    int e = -1;
    if (in_regs) {
#pragma unroll
      for (int q = 0; q < RC; ++q) e = q == ci ? ids[q] : e;
    } else {
      e = r < R ? idx[r] : -1;
    }
    const bool valid = e >= 0 && e < E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & lt_mask);
    if (valid && rank == 0) s_wc[wave * E + e] = __popcll(same);
    lds_barrier();
    // Per expert: exclusive prefix of the 16 wave counts (independent LDS
    // loads), cursor advance, and the counts cleared for the next chunk.
    for (int ee = tid; ee < E; ee += kDispThreads) {
      int cw[kDispWaves];
#pragma unroll
      for (int wv = 0; wv < kDispWaves; ++wv) cw[wv] = s_wc[wv * E + ee];
      int run = s_cur[ee];
#pragma unroll
      for (int wv = 0; wv < kDispWaves; ++wv) {
        s_base[wv * E + ee] = run;
        run += cw[wv];
        s_wc[wv * E + ee] = 0;
      }
      s_cur[ee] = run;
    }
    lds_barrier();
    if (valid) {
      const int pos = s_base[wave * E + e] + rank;  // rank within the expert's pile
      if (in_regs) {
#pragma unroll
        for (int q = 0; q < RC; ++q) rk[q] = q == ci ? pos : rk[q];
      } else {
        inv[r] = pos;
      }
    }
  }
  lds_barrier();

  if (wave == 0) {
    int carry = 0;
    for (int base = 0; base < E; base += MOE_WAVE) {
      const int e = base + lane;
      const int c = e < E ? s_cur[e] : 0;
      const int incl = wave_incl_scan(c);
      if (e < E) s_off[e] = carry + incl - c;
      carry += __builtin_amdgcn_readlane(incl, MOE_WAVE - 1);
    }
    if (lane == 0) offsets[E] = carry;
  }
  lds_barrier();
  for (int e = tid; e < E; e += kDispThreads) {
    counts[e] = s_cur[e];
    offsets[e] = s_off[e];
  }
  if (in_regs) {
#pragma unroll
    for (int q = 0; q < RC; ++q) {
      const int r = q * kDispThreads + tid;
      const int e = ids[q];
      if (r < R && e >= 0 && e < E) {
        const int pos = s_off[e] + rk[q];
        perm[pos] = r / k;
        inv[r] = pos;
      } else if (r < R) {
        inv[r] = -1;
      }
    }
  } else {
    for (int r = tid; r < R; r += kDispThreads) {
      const int e = idx[r];
      if (e >= 0 && e < E) {
        const int pos = s_off[e] + inv[r];
        perm[pos] = r / k;
        inv[r] = pos;
      } else {
        inv[r] = -1;
      }
    }
  }
  // Pile rows past the last pile (pairs with ids outside [0, E)) hold -1.
  const int used = s_cur_total(s_off, s_cur, E);
  for (int r = used + tid; r < R; r += kDispThreads) perm[r] = -1;
}

// Stable piles of R <= 4 * 64 (token, slot) pairs built by one wave in LDS
// (the small-batch dispatch).  Pairs are taken in (token, slot) order in
// chunks of 64; a lane's rank among same-expert lanes of its chunk comes
// from ballots on the bits of the expert id, and a per-expert cursor s_cnt
// carries the earlier chunks.  Outputs: s_cnt [E] pile sizes, s_off [E+1]
// pile offsets, s_perm [R] token of each pile row, s_inv [R] pile row of
// each pair.  The LDS accesses of one wave complete in order, so a chunk's
// cursor reads see the previous chunk's updates.  Ids outside [0, E) are
// skipped: their pairs get s_inv = -1, and the pile rows past the last pile
// hold s_perm = -1.
__device__ __forceinline__ void dispatch_wave(const int32_t *__restrict__ idx, int R, int k,
                                              int E, int nbits, int *s_cnt, int *s_off,
                                              int *s_perm, int *s_inv) {
  const int lane = threadIdx.x & 63;
  for (int e = lane; e < E; e += MOE_WAVE) s_cnt[e] = 0;
  const uint64_t lt_mask = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int ids[4], rk[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = c * MOE_WAVE + lane;
    const int e = r < R ? idx[r] : -1;
    const bool valid = e >= 0 && e < E;
    uint64_t same = __ballot(valid);
    for (int b = 0; b < nbits; ++b) {
      const bool bit = valid && ((e >> b) & 1);
      const uint64_t bal = __ballot(bit);
      same &= bit ? bal : ~bal;
    }
    const int rank = __popcll(same & lt_mask);
    const int base = valid ? s_cnt[e] : 0;
    if (valid && rank == 0) s_cnt[e] = base + __popcll(same);
    ids[c] = valid ? e : -1;
    rk[c] = base + rank;
  }
  int carry = 0;
  for (int b0 = 0; b0 < E; b0 += MOE_WAVE) {
    const int e = b0 + lane;
    const int cnt = e < E ? s_cnt[e] : 0;
    const int incl = wave_incl_scan(cnt);
    if (e < E) s_off[e] = carry + incl - cnt;
    carry += __builtin_amdgcn_readlane(incl, MOE_WAVE - 1);
  }
  if (lane == 0) s_off[E] = carry;
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int r = c * MOE_WAVE + lane;
    if (ids[c] >= 0) {
      const int pos = s_off[ids[c]] + rk[c];
      s_perm[pos] = r / k;
      s_inv[r] = pos;
    } else if (r < R) {
      s_inv[r] = -1;
    }
  }
  for (int r = carry + lane; r < R; r += MOE_WAVE) s_perm[r] = -1;
}

// The same piles for R <= kDispTinyR pairs and E <= 64 * PE experts, by one
// wave with no LDS round trips in between: lane r holds pair r, and the
// pairs are read one at a time across the wave (readlane, a uniform value
// per step).  A pair's rank is the number of earlier pairs with its expert,
// and its pile row is the number of pairs with a smaller expert plus that
// rank, so the grouping is the unique stable one, as dispatch_wave builds
// it.  Lane l also counts, for its experts l + 64 j, the pairs of smaller
// experts (s_off) and of the expert itself (s_cnt).  When s_gpre is given it
// also receives, per expert, the number of 16-row groups of the piles before
// it (a pile of m rows has ceil(m / 16); the pairs of rank 0, 16, 32 ...
// each open one), with the total in s_gpre[E].  Same outputs as
// dispatch_wave otherwise, including the -1 entries for ids outside [0, E).
// Its cost grows with R (two steps per pair), while dispatch_wave's is about
// flat up to 64 pairs: measured faster for 4 pairs, slower for 32.
constexpr int kDispTinyR = 8;

template <int PE>
__device__ __forceinline__ void dispatch_wave_small(const int32_t *__restrict__ idx, int R, int k,
                                                    int E, int *s_cnt, int *s_off, int *s_perm,
                                                    int *s_inv, int *s_gpre) {
  const int lane = threadIdx.x & 63;
  const int my_e = lane < R ? idx[lane] : -1;
  const bool my_valid = my_e >= 0 && my_e < E;
  // pass 1: the lane's own pair (rank, pairs of smaller experts); ids
  // outside [0, E) count nowhere (an invalid er matches no valid my_e, and
  // is not below one only when er >= E, so both tests carry the range)
  int rank = 0, below = 0;
  for (int r = 0; r < R; ++r) {
    const int er = __builtin_amdgcn_readlane(my_e, r);
    const bool vr = er >= 0 && er < E;
    rank += (vr && r < lane && er == my_e) ? 1 : 0;
    below += (vr && er < my_e) ? 1 : 0;
  }
  // pass 2: per expert of the lane, counts and group prefix
  int cnt[PE], less[PE], gless[PE];
#pragma unroll
  for (int j = 0; j < PE; ++j) cnt[j] = less[j] = gless[j] = 0;
  int used = 0, groups = 0;
  for (int r = 0; r < R; ++r) {
    const int er = __builtin_amdgcn_readlane(my_e, r);
    const bool vr = er >= 0 && er < E;
    const bool opens = vr && (__builtin_amdgcn_readlane(rank, r) & 15) == 0;
    used += vr ? 1 : 0;
    groups += opens ? 1 : 0;
#pragma unroll
    for (int j = 0; j < PE; ++j) {
      const int e = lane + MOE_WAVE * j;
      cnt[j] += (vr && er == e) ? 1 : 0;
      less[j] += (vr && er < e) ? 1 : 0;
      gless[j] += (opens && er < e) ? 1 : 0;
    }
  }
#pragma unroll
  for (int j = 0; j < PE; ++j) {
    const int e = lane + MOE_WAVE * j;
    if (e < E) {
      s_cnt[e] = cnt[j];
      s_off[e] = less[j];
      if (s_gpre) s_gpre[e] = gless[j];
    }
  }
  if (lane == 0) {
    s_off[E] = used;
    if (s_gpre) s_gpre[E] = groups;
  }
  if (my_valid) {
    const int pos = below + rank;
    s_perm[pos] = lane / k;
    s_inv[lane] = pos;
  } else if (lane < R) {
    s_inv[lane] = -1;
  }
  if (lane >= used && lane < R) s_perm[lane] = -1;
}

}  // namespace moe
