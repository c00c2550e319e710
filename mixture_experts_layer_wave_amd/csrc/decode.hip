// Small-batch (decode) path of the MXFP4 expert FFN.
//
// "How Mixture of Experts Scales Model Parameters", section "The forward
// pass: dispatch, then combine": each expert runs its FFN on its own pile.
// With a handful of tokens per expert the work is bound by reading the
// experts' weights, which the lesson "Inference Optimization: The Bandwidth
// Wall, PagedAttention, and FlashAttention" (section on decode) states as
// time >= weight bytes / HBM bandwidth.  MXFP4 storage (the minseoc03.com
// note "What is MXFP4?": 4-bit values, one scale per 32) is read once.
//
// One block owns 16 consecutive weight rows of one non-empty expert (the up
// kernel also the same 16 rows of W3).  At entry it issues every byte of
// its rows -- codes and E8M0 scales, contiguous in memory -- as direct
// global-to-LDS copies, and right behind them the activations of its first
// 16 pile rows into registers, so both are in flight together and a CU
// keeps over 100 KB of HBM reads outstanding (three blocks fit in its LDS).
// Then the waves multiply on v_mfma_f32_16x16x32_bf16 with tokens as M (16
// per group, zero-padded) and the 16 weight rows as N.  Each lane converts a
// whole 32-element block (16 B of codes + its scale) with
// v_cvt_scalef32_pk_bf16_fp4 and feeds it to 4 MFMAs: for MFMA q of a
// 128-deep K step, lane group g supplies K indices 32 (4 s + g) + 8 q + i,
// and the activations are read in the same order (any fixed K order is
// valid when both operands agree).  The four waves split K; each wave does
// both matrices of the up projection on its K range, so one activation
// register file feeds both.  Partial sums meet in LDS in a fixed order
// (deterministic).
#include <atomic>

#include "common.h"
#include "kernels.h"

namespace moe {
namespace {

constexpr int kRows = 16;   // weight rows per block
constexpr int kWaves = 4;   // waves per block, splitting K
constexpr int kMaxSteps = 8;  // 128-deep K steps per wave: K <= 32 * 4 * 4 * 8 = 4096

typedef __attribute__((address_space(3))) void lds_void;

// LDS of one block: per matrix the codes [16][K/2] and the scales [16][K/32]
// of its rows, then 2 KB per matrix for the cross-wave reduction.
size_t decode_lds_bytes(int K, int mats) {
  return (size_t)mats * kRows * (K / 2 + K / 32) + 2 * (size_t)mats * 64 * sizeof(float) * 4;
}

// 128-deep K steps each wave needs for K.
int decode_steps(int K) {
  const int per_wave = (K / 32 + kWaves - 1) / kWaves;  // 32-element blocks
  return (per_wave + 3) / 4;
}

struct DecodeParams {
  const uint16_t *a;       // up: x [n][K] (through perm) or x_perm [R][K]; down: h [R][K]
  const int32_t *perm;     // pile row -> row of a, or NULL for contiguous rows
  const int32_t *offsets;  // [E+1]
  int E, N, K;             // one expert matrix is N x K (N % 16 == 0)
  const uint8_t *w0, *w1;  // codes [E][N][K/2] (w1 = W3 for up)
  const uint8_t *s0, *s1;  // scales [E][N][K/32]
  void *out;               // up: bf16 h [R][N]; down: f32 y_perm [R][N]
};

// Block b works on the (b / tiles)-th non-empty expert, rows 16 (b % tiles).
// KS = 128-deep K steps per wave (decode_steps(K)).
template <bool UP, int KS>
__global__ __launch_bounds__(256) void mx_decode_kernel(DecodeParams p, int tiles) {
  constexpr int NMAT = UP ? 2 : 1;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  __shared__ int s_e;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int K = p.K, N = p.N;
  const int KB = K / 32;                  // 32-element blocks per row
  const int rowb = K / 2;                 // code bytes per row
  const int code_bytes = kRows * rowb;    // per matrix
  const int mat_bytes = code_bytes + kRows * KB;
  const int stage_bytes = NMAT * mat_bytes;
  const int slot = blockIdx.x / tiles, tile = blockIdx.x % tiles;
  const int n0 = tile * kRows;

  // ---- the slot-th non-empty expert ---------------------------------------
  // Wave 0 reads the offsets of up to 256 experts per round with all loads
  // in flight together, then ranks the non-empty ones with ballots.
  if (wave == 0) {
    int found = -1, before = 0;
    for (int base = 0; base < p.E && found < 0; base += 4 * 64) {
      int lo[4], hi[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = base + j * 64 + lane;
        lo[j] = e < p.E ? p.offsets[e] : 0;
        hi[j] = e < p.E ? p.offsets[e + 1] : 0;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int e = base + j * 64 + lane;
        const bool ne = hi[j] > lo[j];
        const uint64_t msk = __ballot(ne);
        const int rank = before + __popcll(msk & ((lane == 0) ? 0ull : (~0ull >> (64 - lane))));
        const uint64_t hm = __ballot(ne && rank == slot);
        if (found < 0 && hm) found = base + j * 64 + __ffsll((long long)hm) - 1;
        before += __popcll(msk);
        (void)e;
      }
    }
    if (lane == 0) s_e = found;
  }
  __syncthreads();
  const int e = s_e;
  if (e < 0) return;
  const int row0 = p.offsets[e], m = p.offsets[e + 1] - row0;

  // ---- issue all weight bytes of the tile ---------------------------------
  // The stage holds, per matrix, the 16 rows' codes then their scales; both
  // are contiguous in memory (N % 16 == 0, so every row exists).  1 KB chunk
  // c goes to wave c % 4; lane l copies stage bytes c * 1024 + 16 l.
  {
    const size_t wrow = (size_t)e * N + n0;
    for (int c = wave; c * 1024 < stage_bytes; c += kWaves) {
      const int o = c * 1024 + lane * 16;
      if (o < stage_bytes) {
        const int mat = (NMAT == 2 && o >= mat_bytes) ? 1 : 0;
        const int r = o - mat * mat_bytes;
        const uint8_t *src = r < code_bytes
                                 ? (mat ? p.w1 : p.w0) + wrow * rowb + r
                                 : (mat ? p.s1 : p.s0) + wrow * KB + (r - code_bytes);
        __builtin_amdgcn_global_load_lds(src, (lds_void *)(smem + c * 1024), 16, 0, 2);
      }
    }
  }

  const int r = lane & 15, g = lane >> 4;
  const int kb_lo = (KB * wave) / kWaves, kb_hi = (KB * (wave + 1)) / kWaves;
  float *red = (float *)(smem + stage_bytes);  // [2 waves][NMAT][64 lanes][4]
  const u32x4 z4 = {0u, 0u, 0u, 0u};

  for (int t0 = 0; t0 < m; t0 += 16) {
    // ---- activations of pile rows t0..t0+15 on this wave's K range ------
    // Pile rows are gathered from the token matrix when perm is given (the
    // fused forward), else read in place (x_perm, or h for down).
    const int t = t0 + r;
    const bool tv = t < m;
    const int arow = tv ? (p.perm ? p.perm[row0 + t] : row0 + t) : 0;
    const uint16_t *ap = p.a + (size_t)arow * K;
    u32x4 act[KS][4];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int b = kb_lo + 4 * s + g;
      const bool ok = tv && b < kb_hi;
#pragma unroll
      for (int q = 0; q < 4; ++q) act[s][q] = ok ? *(const u32x4 *)(ap + b * 32 + q * 8) : z4;
    }
    if (t0 == 0) {
      __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8));  // own copies landed
      __syncthreads();                                        // everyone's
    }

    // ---- MFMA over this wave's K range ----------------------------------
    // Two accumulators per matrix (even and odd MFMAs of a step) keep
    // independent MFMA chains in flight; they are summed in a fixed order.
    f32x4 acc2[NMAT][2];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
#pragma unroll
      for (int q = 0; q < 2; ++q) acc2[mat][q] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const int b = kb_lo + 4 * s + g;
      const bool bv = b < kb_hi;
#pragma unroll
      for (int mat = 0; mat < NMAT; ++mat) {
        const uint8_t *lw = smem + mat * mat_bytes;
        const u32x4 codes = bv ? *(const u32x4 *)(lw + r * rowb + b * 16) : z4;
        const float sc = bv ? e8m0_to_f32(lw[code_bytes + r * KB + b]) : 0.f;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const uint32_t wv = codes[q];
          const bf16x2 q0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 0);
          const bf16x2 q1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 1);
          const bf16x2 q2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 2);
          const bf16x2 q3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(wv, sc, 3);
          const u32x4 bw = {__builtin_bit_cast(uint32_t, q0), __builtin_bit_cast(uint32_t, q1),
                            __builtin_bit_cast(uint32_t, q2), __builtin_bit_cast(uint32_t, q3)};
          acc2[mat][q & 1] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              __builtin_bit_cast(bf16x8, act[s][q]), __builtin_bit_cast(bf16x8, bw),
              acc2[mat][q & 1], 0, 0, 0);
        }
      }
    }
    f32x4 acc[NMAT];
#pragma unroll
    for (int mat = 0; mat < NMAT; ++mat)
      acc[mat] = acc2[mat][0] + acc2[mat][1];

    // ---- fixed-order reduction: (w0 + w2) + (w1 + w3) -------------------
    if (wave >= 2) {
#pragma unroll
      for (int mat = 0; mat < NMAT; ++mat)
        *(f32x4 *)(red + (((wave - 2) * NMAT + mat) * 64 + lane) * 4) = acc[mat];
    }
    lds_barrier();
    if (wave < 2) {
#pragma unroll
      for (int mat = 0; mat < NMAT; ++mat)
        acc[mat] += *(const f32x4 *)(red + ((wave * NMAT + mat) * 64 + lane) * 4);
    }
    lds_barrier();
    if (wave == 1) {
#pragma unroll
      for (int mat = 0; mat < NMAT; ++mat)
        *(f32x4 *)(red + (mat * 64 + lane) * 4) = acc[mat];
    }
    lds_barrier();
    if (wave == 0) {
#pragma unroll
      for (int mat = 0; mat < NMAT; ++mat)
        acc[mat] += *(const f32x4 *)(red + (mat * 64 + lane) * 4);
      // 16x16 output: lane l holds tokens (l / 16) * 4 + i, weight row l % 16.
      const int col = n0 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int tt = t0 + (lane >> 4) * 4 + i;
        if (tt < m) {
          if constexpr (UP) {
            ((uint16_t *)p.out)[(size_t)(row0 + tt) * N + col] =
                (uint16_t)f32_to_bf16_bits(silu(acc[0][i]) * acc[1][i]);
          } else {
            ((float *)p.out)[(size_t)(row0 + tt) * N + col] = acc[0][i];
          }
        }
      }
    }
    if (t0 + 16 < m) lds_barrier();  // the reduction area is reused
  }
}

template <bool UP, int KS>
hipError_t launch_decode_ks(const DecodeParams &p, int grid, size_t lds, hipStream_t st) {
  auto kern = mx_decode_kernel<UP, KS>;
  if (lds > 64 * 1024) {
    // Set once per device (the attribute is per device and kernel).
    static std::atomic<uint64_t> attr_done{0};
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    const uint64_t bit = 1ull << (dev & 63);
    if (!(attr_done.load(std::memory_order_acquire) & bit)) {
      err = hipFuncSetAttribute((const void *)kern, hipFuncAttributeMaxDynamicSharedMemorySize,
                                160 * 1024);
      if (err != hipSuccess) return err;
      attr_done.fetch_or(bit, std::memory_order_release);
    }
  }
  kern<<<grid, kWaves * 64, lds, st>>>(p, (p.N + kRows - 1) / kRows);
  return hipGetLastError();
}

template <bool UP>
hipError_t launch_decode(const DecodeParams &p, int max_active, hipStream_t st) {
  const int tiles = p.N / kRows;
  const size_t lds = decode_lds_bytes(p.K, UP ? 2 : 1);
  if (lds > 160 * 1024) return hipErrorInvalidValue;
  const int grid = max_active * tiles;
  switch (decode_steps(p.K)) {
    case 1: return launch_decode_ks<UP, 1>(p, grid, lds, st);
    case 2: return launch_decode_ks<UP, 2>(p, grid, lds, st);
    case 3: return launch_decode_ks<UP, 3>(p, grid, lds, st);
    case 4: return launch_decode_ks<UP, 4>(p, grid, lds, st);
    case 5: return launch_decode_ks<UP, 5>(p, grid, lds, st);
    case 6: return launch_decode_ks<UP, 6>(p, grid, lds, st);
    case 7: return launch_decode_ks<UP, 7>(p, grid, lds, st);
    case 8: return launch_decode_ks<UP, 8>(p, grid, lds, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool decode_ffn_fits(int d, int d_ff, int E) {
  (void)E;
  return d % 32 == 0 && d_ff % 32 == 0 && decode_steps(d) <= kMaxSteps &&
         decode_steps(d_ff) <= kMaxSteps && decode_lds_bytes(d, 2) <= 160 * 1024 &&
         decode_lds_bytes(d_ff, 1) <= 160 * 1024;
}

hipError_t launch_decode_up(const FfnArgs &a, hipStream_t st) {
  DecodeParams p{};
  p.a = (const uint16_t *)a.a;
  p.perm = a.perm;
  p.offsets = a.offsets;
  p.E = a.E;
  p.N = a.d_ff;
  p.K = a.d;
  p.w0 = (const uint8_t *)a.w1;
  p.w1 = (const uint8_t *)a.w3;
  p.s0 = a.s1;
  p.s1 = a.s3;
  p.out = a.h;
  const int max_active = a.E < a.R ? a.E : a.R;
  return launch_decode<true>(p, max_active, st);
}

hipError_t launch_decode_down(const FfnArgs &a, hipStream_t st) {
  DecodeParams p{};
  p.a = (const uint16_t *)a.h;
  p.perm = nullptr;
  p.offsets = a.offsets;
  p.E = a.E;
  p.N = a.d;
  p.K = a.d_ff;
  p.w0 = (const uint8_t *)a.w2;
  p.s0 = a.s2;
  p.out = a.y_perm;
  const int max_active = a.E < a.R ? a.E : a.R;
  return launch_decode<false>(p, max_active, st);
}

}  // namespace moe
