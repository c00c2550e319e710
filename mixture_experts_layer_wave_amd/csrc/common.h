// Shared device helpers for the gfx950 MoE kernels: vector types, bf16
// rounding, wave64 reductions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

#define MOE_WAVE 64
#define MOE_MAX_E 1024
#define MOE_MAX_K 32

namespace moe {

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) {
  return __uint_as_float(b << 16);
}

// float32 -> bfloat16 bits, round to nearest even (v_cvt_pk_bf16_f32 on
// gfx950); NaN stays NaN.
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2 v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// Wave-wide "best" of (value, index): larger value wins, equal values go to
// the lower index.  Every lane returns the winner.
__device__ __forceinline__ void wave_argmax(float &v, int &i) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    float ov = __shfl_xor(v, o, 64);
    int oi = __shfl_xor(i, o, 64);
    bool take = (ov > v) || (ov == v && oi < i);
    v = take ? ov : v;
    i = take ? oi : i;
  }
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP: four shifted
// adds inside each 16-lane row (lanes without a source add 0), then the
// totals of rows 0 and 2 are broadcast into rows 1 and 3 (row_bcast:15)
// and the total of rows 0-1 into rows 2-3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Workgroup barrier that orders LDS only.  __syncthreads() also waits for
// every outstanding global access of the wave (stores and direct-to-LDS
// copies share one counter), which would drain a copy pipeline; copies into
// LDS are waited for explicitly with s_waitcnt vmcnt before this barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Physical weight slot of logical expert e: slot[e] clamped into
// [0, n_slots), or e itself without a table.
__device__ __forceinline__ int phys_slot(const int32_t *slot, int n_slots, int e) {
  if (!slot) return e;
  const int s = slot[e];
  return s < 0 ? 0 : (s >= n_slots ? n_slots - 1 : s);
}

// silu(g) = g * sigma(g) = g / (1 + e^-g), with the hardware exp2 and
// reciprocal (about 1 ulp each) in place of a correctly rounded division.
// g -> -inf gives e^-g = inf and a reciprocal of 0, so the limit 0 holds.
__device__ __forceinline__ float silu(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(g * -1.44269504088896341f));
}

// E8M0 scale code -> float (2^(s-127)); 0 -> 2^-127 (subnormal), 255 -> NaN.
__device__ __forceinline__ float e8m0_to_f32(uint32_t s) {
  // branch-free: s << 23 is the value for 1..254; s = 0 (2^-127, a float32
  // subnormal) and s = 255 (NaN) both add the top mantissa bit
  const uint32_t edge = ((s + 1u) & 255u) <= 1u;
  return __uint_as_float((s << 23) | (edge << 22));
}

// ---- MXFP8 encoding (OCP MX v1.0: E4M3 elements, one E8M0 scale per 32) --
// E8M0 code of the shared exponent for a block whose largest magnitude is
// amax: floor(log2 amax) - 8 + 127 from the float32 exponent field (0 for
// zero and float32 subnormals, the clamp at the bottom of the range).
__device__ __forceinline__ uint32_t mx8_scale_code(float amax) {
  const int ef = (int)((__float_as_uint(amax) >> 23) & 255u);
  return (uint32_t)max(ef - 8, 0);
}
// Scale bytes per row of an MXFP8 matrix: cols / 32 rounded up to 4.
__host__ __device__ __forceinline__ int mx8_scale_pitch_dev(int cols) {
  return (cols / 32 + 3) / 4 * 4;
}
// 2^-X for scale code c = X + 127 (c <= 247, so 254 - c is a normal exponent).
__device__ __forceinline__ float mx8_inv_scale(uint32_t code) {
  return __uint_as_float((254u - code) << 23);
}

// Four E4M3 codes of v[0..3] * inv (exact: a power of two), packed low to
// high.  v_cvt_pk_fp8_f32 rounds to nearest even but turns magnitudes of
// 464 and above into NaN, so the values are clamped to +-448 first; a value
// in (448, 464) rounds to 448 either way, so this is the saturating
// conversion.
__device__ __forceinline__ uint32_t mx8_pack4(const float *v, float inv) {
  float c[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) c[i] = fminf(fmaxf(v[i] * inv, -448.f), 448.f);
  int w = __builtin_amdgcn_cvt_pk_fp8_f32(c[0], c[1], 0, false);
  w = __builtin_amdgcn_cvt_pk_fp8_f32(c[2], c[3], w, true);
  return (uint32_t)w;
}

}  // namespace moe
