// Router statistics and the load-balancing loss.
//
// "How Mixture of Experts Scales Model Parameters", load-balancing section:
// P_i is the router probability of expert i averaged over the batch, f_i the
// fraction of tokens whose highest-scoring expert is i, and the auxiliary
// loss is alpha * E * sum_i f_i P_i (1 when routing is uniform, E * P_1
// when every token goes to one expert).
//
// Three small passes, all in a fixed order (deterministic):
//   1. per token, the softmax normaliser of its logits: max and 1 / sum;
//   2. per expert, sum over tokens of exp(z - max) / sum, and the count of
//      tokens whose first choice it is (one workgroup per 64 experts, tokens
//      strided over its 16 waves, the 16 partial sums added in wave order);
//   3. the loss, a sum over experts in a fixed order.
#include "common.h"
#include "kernels.h"
#include "route_dev.h"

namespace moe {
namespace {

// One group of G = topk_group(E) lanes per token.
__global__ __launch_bounds__(256) void token_norm_kernel(const float *__restrict__ logits, int n,
                                                         int E, float2 *__restrict__ norm) {
  const int G = topk_group(E);
  const int gl = (threadIdx.x & 63) & (G - 1);
  const int t = (blockIdx.x * 256 + threadIdx.x) / G;
  if ((blockIdx.x * 256 + (threadIdx.x & ~63)) / G >= n) return;  // whole wave idle
  const bool live = t < n;
  const float *z = logits + (size_t)(live ? t : 0) * E;
  float m = -__builtin_inff();
  for (int e = gl; e < E; e += G) m = fmaxf(m, live ? z[e] : -__builtin_inff());
  m = group_max(m, G);
  float s = 0.f;
  if (live)
    for (int e = gl; e < E; e += G) s += expf(z[e] - m);
  s = group_sum(s, G);
  if (live && gl == 0) norm[t] = make_float2(m, 1.f / s);
}

constexpr int kStatWaves = 16;

__global__ __launch_bounds__(kStatWaves * 64) void expert_stats_kernel(
    const float *__restrict__ logits, const float2 *__restrict__ norm,
    const int32_t *__restrict__ idx, int n, int E, int k, float *__restrict__ P,
    float *__restrict__ f) {
  __shared__ float s_p[kStatWaves][64];
  __shared__ int s_c[kStatWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int e = blockIdx.x * 64 + lane;
  float acc = 0.f;
  int cnt = 0;
  if (e < E) {
    for (int t = wave; t < n; t += kStatWaves) {
      const float2 nt = norm[t];
      acc += expf(logits[(size_t)t * E + e] - nt.x) * nt.y;
      cnt += idx[(size_t)t * k] == e;
    }
  }
  s_p[wave][lane] = acc;
  s_c[wave][lane] = cnt;
  __syncthreads();
  if (wave == 0 && e < E) {
    float sp = 0.f;
    int sc = 0;
    for (int w = 0; w < kStatWaves; ++w) {
      sp += s_p[w][lane];
      sc += s_c[w][lane];
    }
    P[e] = sp / (float)n;
    f[e] = (float)sc / (float)n;
  }
}

__global__ __launch_bounds__(64) void aux_loss_kernel(const float *__restrict__ P,
                                                      const float *__restrict__ f, int E,
                                                      float alpha, float *__restrict__ loss) {
  const int lane = threadIdx.x;
  float s = 0.f;
  for (int e = lane; e < E; e += 64) s += f[e] * P[e];
  s = group_sum(s, 64);
  if (lane == 0) *loss = alpha * (float)E * s;
}

}  // namespace

hipError_t launch_router_stats(const float *logits, const int32_t *idx, int n, int E, int k,
                               float alpha, float *P, float *f, float *loss, float2 *norm,
                               hipStream_t st) {
  const int per_block = 256 / topk_group(E);
  token_norm_kernel<<<(n + per_block - 1) / per_block, 256, 0, st>>>(logits, n, E, norm);
  expert_stats_kernel<<<(E + 63) / 64, kStatWaves * 64, 0, st>>>(logits, norm, idx, n, E, k, P, f);
  aux_loss_kernel<<<1, 64, 0, st>>>(P, f, E, alpha, loss);
  return hipGetLastError();
}

}  // namespace moe
