// Host side of the C ABI declared in include/moe.h: argument validation,
// workspace layout and the launch sequence on the caller's stream.  Nothing
// here allocates device memory or synchronises with the host.
#include "moe.h"

#include <hip/hip_runtime.h>

#include <algorithm>

#include "api_internal.h"
#include "gemm_mxw.h"
#include "kernels.h"

namespace {

constexpr size_t kAlign = 256;

size_t align_up(size_t v) { return (v + kAlign - 1) / kAlign * kAlign; }

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

struct WsLayout {
  size_t logits, idx, w, counts, offsets, perm, inv, dscratch, h, yp, part, tail, total;
  int splits;
};

// The FFN arguments that decide kernel shapes (no pointers).
moe::FfnArgs plan_args(const moe_shape *s, int wdt) {
  moe::FfnArgs f{};
  f.E = s->E;
  f.R = s->n * s->k;
  f.d = s->d;
  f.d_ff = s->d_ff;
  f.w_dtype = wdt;
  f.n = s->n;
  f.k = s->k;
  f.split_ok = true;
  return f;
}

int check_shape(const moe_shape *s) {
  if (!s) return MOE_ERR_NULL;
  if (s->n < 1 || s->d < 1 || s->d_ff < 1 || s->E < 1 || s->E > 1024 || s->k < 1 ||
      s->k > s->E || s->k > 32 || s->renorm < -1 || s->renorm > 1)
    return MOE_ERR_SHAPE;
  if ((long long)s->n * s->k >= (1ll << 31)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

bool renorm_of(const moe_shape *s) { return s->renorm < 0 ? s->k > 1 : s->renorm == 1; }

// Activation / weight dtype pairing and the shape rules each needs.
int check_dtypes(const moe_shape *s, int act, int wdt) {
  if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_DTYPE;
  if (wdt == MOE_F32) {
    if (act != MOE_F32) return MOE_ERR_DTYPE;
  } else if (wdt == MOE_BF16 || wdt == MOE_MXFP4) {
    if (act != MOE_BF16) return MOE_ERR_DTYPE;
    if (s->d % 8 || s->d_ff % 8) return MOE_ERR_SHAPE;
    if (wdt == MOE_MXFP4 && (s->d % 32 || s->d_ff % 32)) return MOE_ERR_SHAPE;
    // The MFMA GEMMs address the pile matrices (R x d and R x d_ff bf16) and
    // one expert matrix (d x d_ff) with 32-bit byte offsets.
    const long long R = (long long)s->n * s->k;
    if (R * std::max(s->d, s->d_ff) * 2 >= (1ll << 31) || (long long)s->d * s->d_ff * 2 >= (1ll << 31))
      return MOE_ERR_SHAPE;
  } else {
    return MOE_ERR_DTYPE;
  }
  return MOE_OK;
}

// K splits of the router logits (the bf16 MFMA router only).
int splits_of(const moe_shape *s, int wdt) {
  return (wdt == MOE_F32 || s->d % 8) ? 1 : moe::router_splits(s->n, s->E, s->d);
}

WsLayout layout(const moe_shape *s, int wdt) {
  WsLayout L{};
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align_up(o + bytes);
    return at;
  };
  const size_t n = (size_t)s->n, E = (size_t)s->E, R = n * (size_t)s->k;
  L.logits = take((size_t)splits_of(s, wdt) * n * E * 4);  // per-split partial logits
  L.idx = take(R * 4);
  L.w = take(R * 4);
  L.counts = take(E * 4);
  L.offsets = take((E + 1) * 4);
  L.perm = take(R * 4);
  L.inv = take(R * 4);
  L.dscratch = take(moe::dispatch_scratch_bytes(s->n, s->k, s->E));
  // h holds the bf16 hidden, or (W4A8) the MXFP8 hidden; yp holds the pile
  // outputs and, before them, the MXFP8 expert input of the W4A8 mode.
  size_t hb = R * (size_t)s->d_ff * (wdt == MOE_F32 ? 4 : 2);
  size_t yb = R * (size_t)s->d * 4;
  if (wdt == MOE_MXFP4 && s->d % 32 == 0 && s->d_ff % 32 == 0) {
    hb = std::max(hb, moe::mx8_bytes(R, s->d_ff));
    yb = std::max(yb, moe::mx8_bytes(R, s->d));
  }
  L.h = take(hb);
  L.yp = take(yb);
  L.splits = moe::down_split_factor(plan_args(s, wdt));
  if (wdt == MOE_MXFP4 && s->d % 32 == 0 && s->d_ff % 32 == 0 && s->d <= moe::kW4A8MaxK &&
      s->d_ff <= moe::kW4A8MaxK) {
    moe::FfnArgs q = plan_args(s, wdt);  // the W4A8 mode may split K differently
    q.act_quant = true;
    L.splits = std::max(L.splits, moe::down_split_factor(q));
  }
  L.part = take(L.splits > 1 ? (size_t)L.splits * R * (size_t)s->d * 4 : 0);
  L.tail = take(moe::down_tail_bytes(plan_args(s, wdt)));
  L.total = o;
  return L;
}

// The W4A8 mode: MXFP4 weights, shapes the scaled-MFMA GEMM takes, and
// 32-bit offsets into the MXFP8 operands (the larger of n*k and n rows).
int check_w4a8(const moe_shape *s, const moe_expert_weights *w) {
  if (w->act_quant == 0) return MOE_OK;
  if (w->act_quant != MOE_MXFP8 || w->dtype != MOE_MXFP4) return MOE_ERR_DTYPE;
  if (s->d > moe::kW4A8MaxK || s->d_ff > moe::kW4A8MaxK) return MOE_ERR_SHAPE;
  if (((long long)s->d_ff * (s->d / 32)) % 4 || ((long long)s->d * (s->d_ff / 32)) % 4)
    return MOE_ERR_SHAPE;
  const long long R = (long long)s->n * s->k;
  if (R * std::max(s->d, s->d_ff) >= (1ll << 31)) return MOE_ERR_SHAPE;
  return MOE_OK;
}

// act_mx8: the activations handed in are already an MXFP8 matrix.
int check_weights(const moe_shape *s, int act, const moe_expert_weights *w,
                  bool act_mx8 = false) {
  if (!w) return MOE_ERR_NULL;
  if (act_mx8 && !w->act_quant) return MOE_ERR_DTYPE;
  const int st = check_dtypes(s, act_mx8 ? MOE_BF16 : act, w->dtype);
  if (st != MOE_OK) return st;
  const int sq = check_w4a8(s, w);
  if (sq != MOE_OK) return sq;
  if (!w->w1 || !w->w3 || !w->w2) return MOE_ERR_NULL;
  if (w->slot && w->n_slots < 1) return MOE_ERR_SHAPE;
  if (w->dtype == MOE_MXFP4 && (!w->s1 || !w->s3 || !w->s2)) return MOE_ERR_NULL;
  if (w->dtype != MOE_F32 && (!aligned16(w->w1) || !aligned16(w->w3) || !aligned16(w->w2)))
    return MOE_ERR_ALIGN;
  if (w->dtype == MOE_MXFP4 && (!aligned16(w->s1) || !aligned16(w->s3) || !aligned16(w->s2)))
    return MOE_ERR_ALIGN;
  return MOE_OK;
}

int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

moe::FfnArgs ffn_args(const moe_shape *s, const void *a, const int32_t *perm,
                      const int32_t *offsets, const moe_expert_weights *w, void *h, float *yp) {
  moe::FfnArgs f{};
  f.a = a;
  f.perm = perm;
  f.offsets = offsets;
  f.E = s->E;
  f.R = s->n * s->k;
  f.d = s->d;
  f.d_ff = s->d_ff;
  f.w_dtype = w->dtype;
  f.w1 = w->w1;
  f.w3 = w->w3;
  f.w2 = w->w2;
  f.s1 = w->s1;
  f.s3 = w->s3;
  f.s2 = w->s2;
  f.slot = w->slot;
  f.n_slots = w->slot ? w->n_slots : s->E;
  f.h = h;
  f.y_perm = yp;
  f.n = s->n;
  f.k = s->k;
  f.act_quant = w->act_quant == MOE_MXFP8;
  return f;
}

}  // namespace

extern "C" {

int moe_abi_version(void) { return MOE_ABI_VERSION; }

const char *moe_status_string(int status) {
  switch (status) {
    case MOE_OK: return "ok";
    case MOE_ERR_NULL: return "a required pointer is NULL";
    case MOE_ERR_SHAPE: return "shape out of range or inconsistent";
    case MOE_ERR_DTYPE: return "unsupported dtype or dtype combination";
    case MOE_ERR_ALIGN: return "pointer not 16-byte aligned";
    case MOE_ERR_WORKSPACE: return "workspace missing or too small";
    case MOE_ERR_HIP: return "HIP launch failed";
    default: return "unknown status";
  }
}

size_t moe_workspace_bytes(const moe_shape *s, int w_dtype) {
  if (check_shape(s) != MOE_OK) return 0;
  if (w_dtype != MOE_F32 && w_dtype != MOE_BF16 && w_dtype != MOE_MXFP4) return 0;
  return layout(s, w_dtype).total;
}

size_t moe_mxfp8_bytes(int64_t rows, int32_t cols) {
  if (rows < 0 || cols <= 0 || cols % 32) return 0;
  return moe::mx8_bytes((size_t)rows, cols);
}

int moe_quantize_mxfp8(int64_t rows, int32_t cols, const void *x, int act, void *q,
                       void *stream) {
  if (rows < 0 || rows > (1ll << 31) - 1 || cols <= 0 || cols % 32) return MOE_ERR_SHAPE;
  if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_DTYPE;
  if (rows == 0) return MOE_OK;
  if (!x || !q) return MOE_ERR_NULL;
  if (!aligned16(x) || !aligned16(q)) return MOE_ERR_ALIGN;
  uint8_t *qc = (uint8_t *)q;
  return hip_status(moe::launch_quantize_mx8(x, act == MOE_BF16, (int)rows, cols, qc,
                                             qc + moe::mx8_scale_offset((size_t)rows, cols),
                                             (hipStream_t)stream));
}

int moe_router_topk(const moe_shape *s, const void *x, int act, const void *wg,
                    const float *bias, float *logits, int32_t *topk_idx, float *topk_w,
                    void *stream) {
  int st = check_shape(s);
  if (st != MOE_OK) return st;
  if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_DTYPE;
  if (!x || !wg || !logits || !topk_idx || !topk_w) return MOE_ERR_NULL;
  if (act == MOE_BF16 && s->d % 8 == 0 && (!aligned16(x) || !aligned16(wg)))
    return MOE_ERR_ALIGN;
  hipStream_t hs = (hipStream_t)stream;
  hipError_t e = moe::launch_router_logits(x, wg, bias, logits, s->n, s->d, s->E,
                                           act == MOE_BF16, 1, hs);
  if (e != hipSuccess) return MOE_ERR_HIP;
  return hip_status(moe::launch_router_topk(logits, 1, s->n, s->E, s->k, renorm_of(s), topk_idx,
                                            topk_w, nullptr, hs));
}

size_t moe_router_stats_workspace_bytes(const moe_shape *s) {
  if (check_shape(s) != MOE_OK) return 0;
  return align_up((size_t)s->n * sizeof(float2));
}

int moe_router_stats(const moe_shape *s, const float *logits, const int32_t *topk_idx,
                     float alpha, float *P, float *f, float *loss, void *ws, size_t ws_bytes,
                     void *stream) {
  int st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!logits || !topk_idx || !P || !f || !loss) return MOE_ERR_NULL;
  if (!ws || ws_bytes < moe_router_stats_workspace_bytes(s)) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  return hip_status(moe::launch_router_stats(logits, topk_idx, s->n, s->E, s->k, alpha, P, f,
                                             loss, (float2 *)ws, (hipStream_t)stream));
}

size_t moe_dispatch_workspace_bytes(const moe_shape *s) {
  if (check_shape(s) != MOE_OK) return 0;
  return align_up(moe::dispatch_scratch_bytes(s->n, s->k, s->E));
}

int moe_dispatch(const moe_shape *s, const int32_t *topk_idx, int32_t *counts,
                 int32_t *offsets, int32_t *perm, int32_t *inv, const void *x, int act,
                 void *x_perm, void *ws, size_t ws_bytes, void *stream) {
  int st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!topk_idx || !counts || !offsets || !perm || !inv) return MOE_ERR_NULL;
  const int row_bytes = s->d * (act == MOE_F32 ? 4 : 2);
  if (x_perm) {
    if (!x) return MOE_ERR_NULL;
    if (act != MOE_F32 && act != MOE_BF16) return MOE_ERR_DTYPE;
    if (row_bytes % 4) return MOE_ERR_SHAPE;  // rows are copied in 4-byte words
    if (row_bytes % 16 == 0 && (!aligned16(x) || !aligned16(x_perm))) return MOE_ERR_ALIGN;
  }
  hipStream_t hs = (hipStream_t)stream;
  // the chunked form when the caller's scratch holds the per-chunk counts
  const size_t need = moe::dispatch_scratch_bytes(s->n, s->k, s->E);
  int32_t *scratch = (need > 0 && ws && ws_bytes >= need) ? (int32_t *)ws : nullptr;
  if (scratch && !aligned16(ws)) return MOE_ERR_ALIGN;
  hipError_t e = moe::launch_dispatch(topk_idx, s->n, s->k, s->E, counts, offsets, perm, inv,
                                      scratch, hs);
  if (e != hipSuccess) return MOE_ERR_HIP;
  if (x_perm) {
    e = moe::launch_gather_rows(x, perm, x_perm, s->n * s->k, s->n, row_bytes, hs);
    if (e != hipSuccess) return MOE_ERR_HIP;
  }
  return MOE_OK;
}

int moe_active_experts(const moe_shape *s, const int32_t *counts, int32_t *active,
                       int32_t *n_active, void *stream) {
  const int st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!counts || !active || !n_active) return MOE_ERR_NULL;
  return hip_status(
      moe::launch_active_experts(counts, s->E, active, n_active, (hipStream_t)stream));
}

int moe_grouped_ffn(const moe_shape *s, const void *x_perm, int act, const int32_t *offsets,
                    const moe_expert_weights *w, void *y_perm, int out, void *ws,
                    size_t ws_bytes, void *stream) {
  int st = check_shape(s);
  if (st != MOE_OK) return st;
  const bool mx8_in = act == MOE_MXFP8;
  st = check_weights(s, act, w, mx8_in);
  if (st != MOE_OK) return st;
  if (!x_perm || !offsets || !y_perm) return MOE_ERR_NULL;
  if (out != MOE_F32 && out != MOE_BF16) return MOE_ERR_DTYPE;
  if (act != MOE_F32 && (!aligned16(x_perm) || !aligned16(y_perm))) return MOE_ERR_ALIGN;
  if (out == MOE_BF16 && !aligned16(y_perm)) return MOE_ERR_ALIGN;
  const WsLayout L = layout(s, w->dtype);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  char *base = (char *)ws;
  hipStream_t hs = (hipStream_t)stream;
  const void *a = x_perm;
  if (w->act_quant && !mx8_in) {
    // encode the pile rows into the (not yet used) pile-output region
    uint8_t *xq = (uint8_t *)(base + L.yp);
    const size_t R = (size_t)s->n * s->k;
    hipError_t e = moe::launch_quantize_mx8(x_perm, true, (int)R, s->d, xq,
                                            xq + moe::mx8_scale_offset(R, s->d), hs);
    if (e != hipSuccess) return MOE_ERR_HIP;
    a = xq;
  }
  // BF16 output: the pile outputs are summed in f32 in the workspace, then
  // rounded once (nearest even) into y_perm.
  float *yp = out == MOE_BF16 ? (float *)(base + L.yp) : (float *)y_perm;
  moe::FfnArgs f = ffn_args(s, a, nullptr, offsets, w, base + L.h, yp);
  f.split_ok = true;
  f.split_part = (float *)(base + L.part);
  f.tail_part = (float *)(base + L.tail);
  hipError_t e = moe::launch_grouped_ffn(f, hs);
  if (e == hipSuccess && out == MOE_BF16)
    e = moe::launch_f32_to_bf16(yp, (uint16_t *)y_perm, (size_t)s->n * s->k * s->d, hs);
  return hip_status(e);
}

int moe_expert_up(const moe_shape *s, const void *a, int act, const int32_t *perm,
                  const int32_t *offsets, const moe_expert_weights *w, void *h, void *stream) {
  int st = check_shape(s);
  if (st != MOE_OK) return st;
  if (w && w->act_quant && act != MOE_MXFP8) return MOE_ERR_DTYPE;
  st = check_weights(s, act, w, act == MOE_MXFP8);
  if (st != MOE_OK) return st;
  if (!a || !offsets || !h) return MOE_ERR_NULL;
  if (act != MOE_F32 && (!aligned16(a) || !aligned16(h))) return MOE_ERR_ALIGN;
  const moe::FfnArgs f = ffn_args(s, a, perm, offsets, w, h, nullptr);
  return hip_status(moe::launch_expert_up(f, (hipStream_t)stream));
}

int moe_expert_down(const moe_shape *s, const void *h, const int32_t *offsets,
                    const moe_expert_weights *w, float *y_perm, void *stream) {
  int st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!w) return MOE_ERR_NULL;
  st = check_weights(s, w->dtype == MOE_F32 ? MOE_F32 : MOE_BF16, w);
  if (st != MOE_OK) return st;
  if (!h || !offsets || !y_perm) return MOE_ERR_NULL;
  if (w->dtype != MOE_F32 && (!aligned16(h) || !aligned16(y_perm))) return MOE_ERR_ALIGN;
  const moe::FfnArgs f = ffn_args(s, nullptr, nullptr, offsets, w, (void *)h, y_perm);
  return hip_status(moe::launch_expert_down(f, (hipStream_t)stream));
}

int moe_combine(const moe_shape *s, const void *y_perm, int in, const int32_t *inv,
                const float *topk_w, void *y, int out, void *stream) {
  int st = check_shape(s);
  if (st != MOE_OK) return st;
  if (!y_perm || !inv || !topk_w || !y) return MOE_ERR_NULL;
  if ((in != MOE_F32 && in != MOE_BF16) || (out != MOE_F32 && out != MOE_BF16))
    return MOE_ERR_DTYPE;
  if (in == MOE_BF16 && s->d % 8) return MOE_ERR_SHAPE;
  if ((in == MOE_BF16 || s->d % 4 == 0) && (!aligned16(y_perm) || !aligned16(y)))
    return MOE_ERR_ALIGN;
  return hip_status(moe::launch_combine(y_perm, in == MOE_BF16, inv, topk_w, s->n, s->k, s->d, y,
                                        out == MOE_BF16, (hipStream_t)stream));
}

int moe_forward(const moe_shape *s, const void *x, int act, const void *wg, const float *bias,
                const moe_expert_weights *w, void *y, int out, int32_t *topk_idx,
                float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  return moe::forward_impl(s, x, act, wg, bias, w, y, out, topk_idx, topk_w, ws, ws_bytes,
                           stream);
}

}  // extern "C"

namespace moe {

int forward_impl(const moe_shape *s, const void *x, int act, const void *wg, const float *bias,
                 const moe_expert_weights *w, void *y, int out, int32_t *topk_idx,
                 float *topk_w, void *ws, size_t ws_bytes, void *stream) {
  int st = check_shape(s);
  if (st != MOE_OK) return st;
  st = check_weights(s, act, w);
  if (st != MOE_OK) return st;
  if (!x || !wg || !y) return MOE_ERR_NULL;
  if (out != MOE_F32 && out != MOE_BF16) return MOE_ERR_DTYPE;
  if (act == MOE_BF16 && (!aligned16(x) || !aligned16(wg))) return MOE_ERR_ALIGN;
  if (s->d % 4 == 0 && !aligned16(y)) return MOE_ERR_ALIGN;
  const WsLayout L = layout(s, w->dtype);
  if (!ws || ws_bytes < L.total) return MOE_ERR_WORKSPACE;
  if (!aligned16(ws)) return MOE_ERR_ALIGN;
  char *base = (char *)ws;
  float *logits = (float *)(base + L.logits);
  int32_t *idx = topk_idx ? topk_idx : (int32_t *)(base + L.idx);
  float *wt = topk_w ? topk_w : (float *)(base + L.w);
  int32_t *counts = (int32_t *)(base + L.counts);
  int32_t *offsets = (int32_t *)(base + L.offsets);
  int32_t *perm = (int32_t *)(base + L.perm);
  int32_t *inv = (int32_t *)(base + L.inv);
  float *yp = (float *)(base + L.yp);
  hipStream_t hs = (hipStream_t)stream;

  const int splits = splits_of(s, w->dtype);
  hipError_t e = moe::launch_router_logits(x, wg, bias, logits, s->n, s->d, s->E,
                                           act == MOE_BF16, splits, hs);
  // planes of partial logits the routing sums (the router may sum them)
  const int planes = moe::router_planes(s->n, s->E, s->d, act == MOE_BF16, splits);
  // Small MXFP4 batches: the decode up kernel takes the top-k and the piles
  // itself (one launch fewer); otherwise top-k and dispatch run first.
  moe::FfnArgs fold = ffn_args(s, x, perm, offsets, w, nullptr, nullptr);
  const bool folded = moe::decode_route_fold_ok(fold);
  if (e == hipSuccess && folded) {
    // nothing to launch here: the up kernel routes
  } else if (e == hipSuccess && moe::route_small_ok(s->n, s->k, s->E)) {
    e = moe::launch_route_small(logits, planes, s->n, s->E, s->k, renorm_of(s), idx, wt, counts,
                                offsets, perm, inv, hs);
  } else if (e == hipSuccess) {
    e = moe::launch_router_topk(logits, planes, s->n, s->E, s->k, renorm_of(s), idx, wt,
                                nullptr, hs);
    if (e == hipSuccess)
      e = moe::launch_dispatch(idx, s->n, s->k, s->E, counts, offsets, perm, inv,
                               (int32_t *)(base + L.dscratch), hs);
  }
  const void *a = x;
  if (e == hipSuccess && w->act_quant) {
    // the experts' input: x as MXFP8, in the (not yet used) pile-output region
    uint8_t *xq = (uint8_t *)yp;
    e = moe::launch_quantize_mx8(x, true, s->n, s->d, xq,
                                 xq + moe::mx8_scale_offset((size_t)s->n, s->d), hs);
    a = xq;
  }
  bool fused = false, yp_bf16 = false;
  if (e == hipSuccess) {
    moe::FfnArgs f = ffn_args(s, a, perm, offsets, w, base + L.h, yp);
    f.split_ok = true;
    f.split_part = (float *)(base + L.part);
    f.tail_part = (float *)(base + L.tail);
    if (folded) {
      f.route_part = logits;
      f.route_S = planes;
      f.route_renorm = renorm_of(s) ? 1 : 0;
      f.r_idx = idx;
      f.r_w = wt;
      f.r_counts = counts;
      f.r_offsets = offsets;
      f.r_perm = perm;
      f.r_inv = inv;
    }
    f.comb_y = y;
    f.comb_inv = inv;
    f.comb_w = wt;
    f.comb_bf16 = out == MOE_BF16;
    f.yp_bf16_ok = true;  // the combine below reads either pile dtype
    if (s->k == 1 && out == MOE_BF16) {  // one expert per token: scale-and-scatter in the down pass
      f.fuse_y = y;
      f.fuse_perm = perm;
      f.fuse_w = wt;
    }
    e = moe::launch_grouped_ffn(f, hs, &fused, &yp_bf16);
  }
  if (e == hipSuccess && !fused)
    e = moe::launch_combine(yp, yp_bf16, inv, wt, s->n, s->k, s->d, y, out == MOE_BF16, hs);
  return hip_status(e);
}

}  // namespace moe
