// Router: logits = x W_g (+ bias), row softmax, top-k and combine weights.
//
// "How Mixture of Experts Scales Model Parameters", section "Routing: a
// router scores the experts, and the top one runs" (a single d x E linear
// layer followed by a softmax per token) and section "Top-K: several
// experts, added up by weight" (keep the K best, renormalise over them).
// The softmax subtracts the row maximum first ("Why FlashAttention is So
// Fast", section "A fused kernel, and an overflow problem").
#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {
namespace {

// bf16 logits on MFMA.  One wave owns TT x ET tiles of 16 tokens x 16
// experts and walks its K split in steps of 32 with
// v_mfma_f32_16x16x32_bf16 (bf16 products are exact in the fp32
// accumulator); the loaded fragments of a step serve every tile of the wave
// (each x fragment ET tiles, each wg fragment TT tiles).  Lane l holds
// tokens/experts (l % 16) and the 8 consecutive K values (l / 16) * 8 of each
// 32-wide step for both operands.  Each tile accumulates in the same order
// whatever TT and ET: 64-deep steps into two chains (first half acc0,
// second half acc1), a 32-deep tail into acc0, then acc0 + acc1 (+ bias).
// Grid: x = groups of 16 TT tokens, y = groups of 4 wave columns of 16 ET
// experts, z = K splits.  Split z writes part[z][n][E] over K range
// [z * kc, (z + 1) * kc); split 0 adds the bias.  The top-k pass sums the
// splits in order.
// The wave tile of K split z (tokens t0.., experts e0..): acc0 + acc1
// (+ bias for z = 0), per lane rows (l / 16) * 4 + i of each token block a
// and column l % 16 of each expert block b.
template <int TT, int ET>
__device__ __forceinline__ void router_split_tile(const uint16_t *__restrict__ x,
                                                  const uint16_t *__restrict__ wg,
                                                  const float *__restrict__ bias, int n, int d,
                                                  int E, int kc, int t0, int e0, int z,
                                                  f32x4 (&res)[TT][ET]) {
  const int lane = threadIdx.x & 63;
  const int kbeg = z * kc, kend = min(d, kbeg + kc);
  const int row = lane & 15, kg = lane >> 4;
  const uint16_t *xr[TT], *wr[ET];
  bool tv[TT], ev[ET];
#pragma unroll
  for (int a = 0; a < TT; ++a) {
    const int t = t0 + 16 * a + row;
    tv[a] = t < n;
    xr[a] = x + (size_t)(tv[a] ? t : 0) * d + kg * 8;
  }
#pragma unroll
  for (int b = 0; b < ET; ++b) {
    const int e = e0 + 16 * b + row;
    ev[b] = e < E;
    wr[b] = wg + (size_t)(ev[b] ? e : 0) * d + kg * 8;
  }
  f32x4 acc0[TT][ET], acc1[TT][ET];
#pragma unroll
  for (int a = 0; a < TT; ++a)
#pragma unroll
    for (int b = 0; b < ET; ++b) acc0[a][b] = acc1[a][b] = f32x4{0.f, 0.f, 0.f, 0.f};
  const u32x4 zero = {0u, 0u, 0u, 0u};
  // 64-deep steps, the next step's fragments loaded while this one's MFMAs
  // run (the addresses of invalid rows are clamped to row 0, so every load
  // is in bounds and is issued; invalid rows are zeroed after the load).
  struct Frag {
    u32x4 a0[TT], a1[TT], b0[ET], b1[ET];
  };
  auto load = [&](int k, Frag &f) {
#pragma unroll
    for (int a = 0; a < TT; ++a) {
      f.a0[a] = *(const u32x4 *)(xr[a] + k);
      f.a1[a] = *(const u32x4 *)(xr[a] + k + 32);
    }
#pragma unroll
    for (int b = 0; b < ET; ++b) {
      f.b0[b] = *(const u32x4 *)(wr[b] + k);
      f.b1[b] = *(const u32x4 *)(wr[b] + k + 32);
    }
#pragma unroll
    for (int a = 0; a < TT; ++a)
      if (!tv[a]) f.a0[a] = f.a1[a] = zero;
#pragma unroll
    for (int b = 0; b < ET; ++b)
      if (!ev[b]) f.b0[b] = f.b1[b] = zero;
  };
  auto mfma = [&](const Frag &f) {
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < ET; ++b) {
        acc0[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, f.a0[a]), __builtin_bit_cast(bf16x8, f.b0[b]), acc0[a][b], 0, 0, 0);
        acc1[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, f.a1[a]), __builtin_bit_cast(bf16x8, f.b1[b]), acc1[a][b], 0, 0, 0);
      }
  };
  const int nfull = (kend - kbeg) / 64;
  if (nfull > 0) {
    Frag p, q;
    load(kbeg, p);
    for (int i = 0; i < nfull; i += 2) {
      if (i + 1 < nfull) load(kbeg + 64 * (i + 1), q);
      mfma(p);
      if (i + 1 < nfull) {
        if (i + 2 < nfull) load(kbeg + 64 * (i + 2), p);
        mfma(q);
      }
    }
  }
  int k0 = kbeg + 64 * nfull;
  for (; k0 < kend; k0 += 32) {
    const bool kv = k0 + kg * 8 < kend;  // d % 8 == 0: a chunk is all in or all out
    u32x4 a0[TT], b0[ET];
#pragma unroll
    for (int a = 0; a < TT; ++a) a0[a] = (tv[a] && kv) ? *(const u32x4 *)(xr[a] + k0) : zero;
#pragma unroll
    for (int b = 0; b < ET; ++b) b0[b] = (ev[b] && kv) ? *(const u32x4 *)(wr[b] + k0) : zero;
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int b = 0; b < ET; ++b)
        acc0[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            __builtin_bit_cast(bf16x8, a0[a]), __builtin_bit_cast(bf16x8, b0[b]), acc0[a][b], 0, 0, 0);
  }
#pragma unroll
  for (int b = 0; b < ET; ++b) {
    const float bb = (bias && z == 0 && ev[b]) ? bias[e0 + 16 * b + row] : 0.f;
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) res[a][b][i] = acc0[a][b][i] + acc1[a][b][i] + bb;
  }
}

template <int TT, int ET>
__global__ __launch_bounds__(256) void router_logits_bf16_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg,
    const float *__restrict__ bias, float *__restrict__ part, int n, int d, int E, int kc) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t0 = blockIdx.x * 16 * TT;
  const int e0 = (blockIdx.y * 4 + wave) * 16 * ET;
  if (e0 >= E) return;  // no barriers in this kernel
  const int row = lane & 15, kg = lane >> 4;
  f32x4 res[TT][ET];
  router_split_tile<TT, ET>(x, wg, bias, n, d, E, kc, t0, e0, blockIdx.z, res);
  // Output layout of a 16x16 tile: lane l holds rows (l / 16) * 4 + i, column l % 16.
  float *out = part + (size_t)blockIdx.z * n * E;
#pragma unroll
  for (int b = 0; b < ET; ++b) {
    const int e = e0 + 16 * b + row;
    if (e >= E) continue;
#pragma unroll
    for (int a = 0; a < TT; ++a)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = t0 + 16 * a + kg * 4 + i;
        if (tt < n) out[(size_t)tt * E + e] = res[a][b][i];
      }
  }
}

// The same logits with the K splits summed inside the launch: one block per
// tile of 16 TT tokens x 16 ET experts, its NW waves computing splits
// NW r + w in round r (each exactly as router_logits_bf16_kernel does); the
// block adds the splits in order, p0 + p1 + ... (the order in which the
// top-k pass sums split planes), and writes one plane, so the logits carry
// the same bits while the partial planes never reach memory.
template <int TT, int ET, int NW>
__global__ __launch_bounds__(NW * 64) void router_logits_sum_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ wg,
    const float *__restrict__ bias, float *__restrict__ logits, int n, int d, int E, int kc,
    int S) {
  constexpr int NT = NW * 64;
  constexpr int TR = 16 * TT, TC = 16 * ET, TILE = TR * TC, PER = (TILE + NT - 1) / NT;
  __shared__ float pl[NW][TILE];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, tid = threadIdx.x;
  const int row = lane & 15, kg = lane >> 4;
  const int t0 = blockIdx.x * TR, e0 = blockIdx.y * TC;
  float tot[PER];
  for (int r = 0; r * NW < S; ++r) {
    const int z = NW * r + wave;
    if (z < S) {
      f32x4 res[TT][ET];
      router_split_tile<TT, ET>(x, wg, bias, n, d, E, kc, t0, e0, z, res);
#pragma unroll
      for (int a = 0; a < TT; ++a)
#pragma unroll
        for (int b = 0; b < ET; ++b)
#pragma unroll
          for (int i = 0; i < 4; ++i) pl[wave][(16 * a + kg * 4 + i) * TC + 16 * b + row] = res[a][b][i];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int q = tid + NT * j;
      if (q < TILE) {
        for (int u = 0; u < NW && NW * r + u < S; ++u) {
          if (r == 0 && u == 0)
            tot[j] = pl[0][q];
          else
            tot[j] += pl[u][q];
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < PER; ++j) {
    const int q = tid + NT * j;
    const int tt = t0 + q / TC, e = e0 + q % TC;
    if (q < TILE && tt < n && e < E) logits[(size_t)tt * E + e] = tot[j];
  }
}

// float32 logits (any dtype pair is handled here when MFMA does not apply):
// one thread per (token, expert), plain fused multiply-adds in K order.
template <typename T>
__global__ __launch_bounds__(256) void router_logits_valu_kernel(
    const T *__restrict__ x, const T *__restrict__ wg, const float *__restrict__ bias,
    float *__restrict__ logits, int n, int d, int E) {
  const long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= (long long)n * E) return;
  const int t = (int)(i / E), e = (int)(i % E);
  const T *xr = x + (size_t)t * d;
  const T *wr = wg + (size_t)e * d;
  float acc = 0.f;
  for (int k = 0; k < d; ++k) {
    float a, b;
    if constexpr (sizeof(T) == 2) {
      a = bf16_bits_to_f32(xr[k]);
      b = bf16_bits_to_f32(wr[k]);
    } else {
      a = xr[k];
      b = wr[k];
    }
    acc = fmaf(a, b, acc);
  }
  logits[i] = acc + (bias ? bias[e] : 0.f);
}

// Softmax + top-k: one token per group of topk_group(E) lanes (see
// topk_token in route_dev.h); a block of 4 waves covers 4 * 64 / G tokens.
template <int PER>
__global__ __launch_bounds__(256) void router_topk_kernel(const float *__restrict__ part, int S,
                                                          int n, int E, int k, int renorm,
                                                          int32_t *__restrict__ idx,
                                                          float *__restrict__ w,
                                                          float *__restrict__ logits) {
  const int G = topk_group(E);
  const int t = (blockIdx.x * 256 + threadIdx.x) / G;
  if ((blockIdx.x * 256 + (threadIdx.x & ~63)) / G >= n) return;  // whole wave idle
  topk_token_t<PER>(part, S, (size_t)n * E, t, n, E, k, renorm, idx, w, logits, nullptr);
}

}  // namespace

// K range of one split: a multiple of 32 (one MFMA K step).
static int split_kc(int d, int splits) { return ((d + splits - 1) / splits + 31) / 32 * 32; }

// The split count depends on d only, so a token's logits are summed in the
// same order whatever the batch it arrives in (outputs are batch-invariant).
int router_splits(int n, int E, int d) {
  (void)n;
  (void)E;
  constexpr int kSplitK = 256;
  const int s = (d + kSplitK - 1) / kSplitK;
  const int kc = split_kc(d, s);
  return (d + kc - 1) / kc;  // splits that the rounded K range actually yields
}

// Large batches get the logits of all K splits summed inside the launch
// (one plane out); small ones (decode) keep one block per split, whose
// planes the top-k pass sums (more blocks for few tokens).
int router_planes(int n, int E, int d, bool is_bf16, int splits) {
  (void)E;
  return (is_bf16 && d % 8 == 0 && n >= 256) ? 1 : splits;
}

hipError_t launch_router_logits(const void *x, const void *wg, const float *bias, float *part,
                                int n, int d, int E, bool is_bf16, int splits, hipStream_t st) {
  if (is_bf16 && d % 8 == 0) {
    const int kc = split_kc(d, splits);
    const int S = (d + kc - 1) / kc;
    const uint16_t *xb = (const uint16_t *)x, *wb = (const uint16_t *)wg;
    if (router_planes(n, E, d, is_bf16, splits) == 1 && S > 1) {
      // eight waves (splits) per round: 64 KB of planes for the wide tile
      if (E > 16) {
        dim3 grid((n + 31) / 32, (E + 63) / 64);
        router_logits_sum_kernel<2, 4, 8><<<grid, 512, 0, st>>>(xb, wb, bias, part, n, d, E, kc, S);
      } else {
        dim3 grid((n + 15) / 16, (E + 15) / 16);
        router_logits_sum_kernel<1, 1, 8><<<grid, 512, 0, st>>>(xb, wb, bias, part, n, d, E, kc, S);
      }
      return hipGetLastError();
    }
    // Wave tiles of 32 tokens x 64 experts for wide routers on large
    // batches (the 128-expert prefill step 10 us faster), else 16 x 16.  A
    // 64 x 16 tile for E <= 16 measured 1% slower on the 8-expert layers.
    if (E > 16 && n >= 256) {
      dim3 grid((n + 31) / 32, (E + 255) / 256, S);
      router_logits_bf16_kernel<2, 4><<<grid, 256, 0, st>>>(xb, wb, bias, part, n, d, E, kc);
    } else {
      dim3 grid((n + 15) / 16, (E + 63) / 64, S);
      router_logits_bf16_kernel<1, 1><<<grid, 256, 0, st>>>(xb, wb, bias, part, n, d, E, kc);
    }
  } else if (is_bf16) {
    const long long tot = (long long)n * E;
    router_logits_valu_kernel<uint16_t><<<(unsigned)((tot + 255) / 256), 256, 0, st>>>(
        (const uint16_t *)x, (const uint16_t *)wg, bias, part, n, d, E);
  } else {
    const long long tot = (long long)n * E;
    router_logits_valu_kernel<float><<<(unsigned)((tot + 255) / 256), 256, 0, st>>>(
        (const float *)x, (const float *)wg, bias, part, n, d, E);
  }
  return hipGetLastError();
}

hipError_t launch_router_topk(const float *part, int splits, int n, int E, int k, bool renorm,
                              int32_t *idx, float *w, float *logits, hipStream_t st) {
  const int per_block = 256 / topk_group(E);
  const int grid = (n + per_block - 1) / per_block;
  const int rn = renorm ? 1 : 0;
  switch (topk_per(E)) {
    case 2:
      router_topk_kernel<2><<<grid, 256, 0, st>>>(part, splits, n, E, k, rn, idx, w, logits);
      break;
    case 4:
      router_topk_kernel<4><<<grid, 256, 0, st>>>(part, splits, n, E, k, rn, idx, w, logits);
      break;
    default:
      router_topk_kernel<MOE_MAX_E / MOE_WAVE><<<grid, 256, 0, st>>>(part, splits, n, E, k, rn,
                                                                      idx, w, logits);
  }
  return hipGetLastError();
}

}  // namespace moe
