/*
 * moe.h -- C ABI of libmoe_mi355x.so, the sparse Mixture-of-Experts layer
 * forward for AMD Instinct MI355X (gfx950).
 *
 * What is computed follows "How Mixture of Experts Scales Model Parameters"
 * (zhangchitc.github.io/posts/mixture-of-experts/):
 *   - section "Routing: a router scores the experts, and the top one runs":
 *     a d x E linear router W_g and a softmax over each row;
 *   - section "Top-K: several experts, added up by weight": the K best
 *     experts, weights renormalised over the K when K > 1;
 *   - section "The forward pass: dispatch, then combine": per-expert piles,
 *     each expert's FFN on its pile, weighted outputs put back in order;
 *   - section "Dense models: ...": the FFN is up-projection, activation,
 *     down-projection; here the SiLU-gated form silu(x W1) * (x W3) then W2.
 * MXFP4 weights (minseoc03.com feed, note "What is MXFP4?": 4-bit values in
 * blocks of 32 sharing one scale) use the OCP MX v1.0 encoding: E2M1
 * elements, one E8M0 scale per 32 consecutive elements along K.
 *
 * Conventions shared by every entry point
 *   - Data pointers are DEVICE pointers unless stated otherwise.  Structs
 *     (moe_shape, moe_expert_weights) live in HOST memory and are read
 *     during the call only.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every entry point only enqueues work on it and never synchronises
 *     with the host, so the sequence is capturable in a HIP graph.
 *   - The caller owns every buffer, including the workspace.  The library
 *     allocates no device memory and keeps no state between calls; calls on
 *     different streams with different buffers may run concurrently.
 *   - Inputs are never written.  Outputs are fully overwritten.
 *   - All argument checks run on the host before anything is enqueued: on
 *     an error return nothing has been launched.  A launch failure returns
 *     MOE_ERR_HIP.  Faults inside kernels surface at the caller's next
 *     synchronisation, as for any HIP work.
 *   - Row-major layouts.  bf16 is stored as its 16-bit pattern.  MXFP4
 *     matrices are [rows][K/2] bytes with the even-K element in the low
 *     nibble, plus [rows][K/32] E8M0 scale bytes.
 *   - MXFP8 matrices (rows x cols, cols % 32 == 0; the W4A8 mode below)
 *     are one buffer: E4M3 codes [rows][cols] at offset 0, then, from
 *     offset rows*cols rounded up to a multiple of 256, E8M0 scales
 *     [rows][sp] with sp = cols/32 rounded up to a multiple of 4 (padding
 *     bytes 0).  moe_mxfp8_bytes gives the size.  Encoding (OCP MX v1.0):
 *     per 32-block, X = floor(log2 amax) - 8 (the scale code X + 127,
 *     clamped at 0; an all-zero block has code 0); each element is v / 2^X
 *     rounded to the nearest E4M3 value, ties to even, clamped to +-448.
 *   - Rounding: products are accumulated in float32; the expert hidden
 *     activation is rounded to bf16 (round to nearest even) before the
 *     down-projection when the weights are bf16 or MXFP4 (to MXFP8 in the
 *     W4A8 mode); pile outputs are kept in float32 and rounded once in the
 *     combine.
 */
#ifndef MOE_MI355X_H
#define MOE_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define MOE_ABI_VERSION 4

typedef enum {
  MOE_OK = 0,
  MOE_ERR_NULL = -1,        /* a required pointer is NULL                    */
  MOE_ERR_SHAPE = -2,       /* n, d, E, k, d_ff out of range or inconsistent */
  MOE_ERR_DTYPE = -3,       /* unsupported dtype or dtype combination        */
  MOE_ERR_ALIGN = -4,       /* a pointer is not 16-byte aligned              */
  MOE_ERR_WORKSPACE = -5,   /* workspace NULL or smaller than required       */
  MOE_ERR_HIP = -6          /* a HIP launch failed                           */
} moe_status;

typedef enum { MOE_F32 = 0, MOE_BF16 = 1, MOE_MXFP4 = 2, MOE_MXFP8 = 3 } moe_dtype;

/* Layer shape.  n tokens of width d, E experts of hidden width d_ff, k
 * experts per token.  renorm: 1 = divide the k probabilities by their sum,
 * 0 = use the raw probabilities, -1 = renormalise iff k > 1.
 * Limits: n >= 1, d >= 1, d_ff >= 1, 1 <= E <= 1024, 1 <= k <= min(E, 32),
 * n * k < 2^31.  MXFP4 weights need d % 32 == 0 and d_ff % 32 == 0; bf16
 * activations need d % 8 == 0 and d_ff % 8 == 0.  With BF16 or MXFP4
 * weights the expert GEMMs address their operands with 32-bit byte
 * offsets: n * k * max(d, d_ff) < 2^30 and d * d_ff < 2^30 (MOE_ERR_SHAPE
 * otherwise; a larger batch is split by the caller). */
typedef struct {
  int32_t n, d, E, k, d_ff;
  int32_t renorm;
} moe_shape;

/* Expert weights (read only, caller owned).
 *   w1, w3: [E][d_ff][d]  (gate and value up-projections, K = d contiguous)
 *   w2:     [E][d][d_ff]  (down-projection, K = d_ff contiguous)
 * For MXFP4, w1/w3 are [E][d_ff][d/2] bytes and w2 is [E][d][d_ff/2] bytes,
 * with scales s1/s3 [E][d_ff][d/32] and s2 [E][d][d_ff/32]; s* are NULL for
 * the other dtypes.  F32 weights require F32 activations; BF16 and MXFP4
 * weights require BF16 activations.  BF16/MXFP4 weight and scale pointers
 * must be 16-byte aligned (MOE_ERR_ALIGN otherwise). */
typedef struct {
  int32_t dtype; /* moe_dtype */
  const void *w1, *w3, *w2;
  const uint8_t *s1, *s3, *s2;
  /* Logical -> physical expert slots (the hook for a partly resident expert
   * pool): with slot = NULL the arrays above hold E experts and expert e is
   * slot e.  Otherwise they hold n_slots physical slots ([n_slots][...] in
   * every layout above), slot is a DEVICE int32 [E] table read on the
   * device, and logical expert e (what the router scores and the piles are
   * keyed by) uses the weights of slot[e].  Entries outside [0, n_slots)
   * are clamped into it (the kernels never read outside the arrays).
   * n_slots >= 1 is required when slot is given. */
  const int32_t *slot;
  int32_t n_slots;
  /* 0, or MOE_MXFP8 for the W4A8 mode (MXFP4 weights only): the input of
   * each projection -- the token rows, then the hidden -- is encoded as
   * MXFP8 and the products run on the scaled MFMA with both operands in
   * their stored form.  The minseoc03.com feed's review of the vLLM paper
   * (section "What's Next") observes that quantised weights are usually
   * widened back before the arithmetic, which costs the speed-up; this
   * mode widens neither operand.  The router still sees the unencoded x.
   * Needs d and d_ff <= 7168, and d_ff*(d/32) and d*(d_ff/32) multiples of
   * 4 (MOE_ERR_SHAPE otherwise); scale arrays 16-byte aligned. */
  int32_t act_quant;
} moe_expert_weights;

/* ABI version of the loaded library (MOE_ABI_VERSION). */
int moe_abi_version(void);

/* Static, host-side description of a status code. */
const char *moe_status_string(int status);

/* Workspace bytes that moe_forward needs for this shape and weight dtype
 * (also enough for moe_grouped_ffn, and for MXFP4 in either mode).  The
 * activation dtype is implied by the weight dtype (F32 weights take F32
 * activations, BF16 and MXFP4 weights BF16), so it is not an argument.
 * Returns 0 for an invalid shape or dtype. */
size_t moe_workspace_bytes(const moe_shape *s, int w_dtype);

/* Bytes of an MXFP8 matrix of rows x cols (layout above); 0 when rows < 0
 * or cols is not a positive multiple of 32. */
size_t moe_mxfp8_bytes(int64_t rows, int32_t cols);

/* MXFP8 encoding of x [rows][cols] (act = MOE_F32 or MOE_BF16) into the
 * MXFP8 matrix q (moe_mxfp8_bytes(rows, cols) bytes), as described above;
 * the encoding of a W4A8 projection's input.  x and q 16-byte aligned;
 * cols % 32 == 0.  rows = 0 does nothing. */
int moe_quantize_mxfp8(int64_t rows, int32_t cols, const void *x, int act, void *q,
                       void *stream);

/* Router and top-k (routing and Top-K sections of the MoE page).
 *   x      [n][d]   activations (act = MOE_F32 or MOE_BF16)
 *   wg     [E][d]   router matrix W_g stored transposed, same dtype as x
 *   bias   [E] f32  added to every logit, or NULL
 *   logits [n][E] f32 output of x W_g (+ bias).  Required (MOE_ERR_NULL
 *          otherwise): the library keeps no device memory of its own, and
 *          the top-k pass reads the logits back from this buffer.
 *   topk_idx [n][k] int32 output: chosen experts, best first (descending
 *            logit, equal logits to the lower index)
 *   topk_w   [n][k] f32 output: softmax probability of each chosen expert
 *            over all E logits, divided by the sum over the k chosen when
 *            renormalising.
 * The softmax subtracts the row maximum before exponentiating ("Why
 * FlashAttention is So Fast", section "A fused kernel, and an overflow
 * problem").  A NaN logit ranks below every number (as -inf), so every
 * chosen id lies in [0, E) whatever x holds; a token whose logits are all
 * NaN gets experts 0 .. k-1 and NaN weights, and other tokens are not
 * affected.  The same rule holds inside moe_forward. */
int moe_router_topk(const moe_shape *s, const void *x, int act, const void *wg,
                    const float *bias, float *logits, int32_t *topk_idx,
                    float *topk_w, void *stream);

/* Router statistics and the load-balancing loss (load-balancing section of
 * the MoE page): P_i, the router probability of expert i averaged over the
 * n tokens; f_i, the fraction of tokens whose highest-scoring expert (the
 * first of its k) is i; and alpha * E * sum_i f_i P_i, which is 1 (times
 * alpha) when routing is uniform and E * P_1 when every token picks one
 * expert.  Per-expert counts over all k slots are moe_dispatch's counts.
 *   logits   [n][E] f32 input (as written by moe_router_topk; bias included)
 *   topk_idx [n][k] int32 input (every value in [0, E))
 *   P, f     [E] f32 outputs; loss: one f32 output
 *   ws / ws_bytes: device workspace of at least
 *           moe_router_stats_workspace_bytes(s) bytes (per-token softmax
 *           normalisers), 16-byte aligned.
 * Sums run in a fixed order (deterministic); the softmax subtracts each
 * row's maximum. */
size_t moe_router_stats_workspace_bytes(const moe_shape *s);
int moe_router_stats(const moe_shape *s, const float *logits, const int32_t *topk_idx,
                     float alpha, float *P, float *f, float *loss, void *ws, size_t ws_bytes,
                     void *stream);

/* Dispatch (forward-pass section of the MoE page): regroup the n*k
 * (token, slot) pairs into per-expert piles, expert by expert, each pile in
 * ascending token then slot order; empty piles are allowed.
 *   topk_idx [n][k] int32 input; a pair whose id is outside [0, E) is put
 *            in no pile: its inv entry is -1, offsets[E] counts only the
 *            piled pairs, and the pile rows from offsets[E] to n*k hold
 *            perm = -1 (x_perm zeros)
 *   counts   [E]    int32 output: pile sizes
 *   offsets  [E+1]  int32 output: pile e is rows offsets[e] .. offsets[e+1]
 *   perm     [n*k]  int32 output: token of each pile row
 *   inv      [n][k] int32 output: pile row of each (token, slot)
 *   x / x_perm: if x_perm is not NULL, x_perm[r] = x[perm[r]] ([n*k][d],
 *           dtype act) is gathered too (the row size d * sizeof(act) must be
 *           a multiple of 4 bytes); x may be NULL when x_perm is NULL.
 *   ws / ws_bytes: optional device scratch.  With at least
 *           moe_dispatch_workspace_bytes(s) bytes (16-byte aligned) the piles
 *           are built by many workgroups in two passes over chunks of 1024
 *           pairs; otherwise (NULL, or too small) by one workgroup.  The
 *           result is the same.
 * Results are deterministic (no order-dependent atomics). */
size_t moe_dispatch_workspace_bytes(const moe_shape *s);
int moe_dispatch(const moe_shape *s, const int32_t *topk_idx, int32_t *counts,
                 int32_t *offsets, int32_t *perm, int32_t *inv, const void *x,
                 int act, void *x_perm, void *ws, size_t ws_bytes, void *stream);

/* Active experts: the deduplicated, ascending list of the experts that a
 * batch routes at least one row to, read from moe_dispatch's counts.  It is
 * the set an expert cache must hold for the batch (the minseoc03.com feed's
 * review of FreeToken, sections "Decode: Exploit Expert Locality" and
 * "Dynamic Scheduling Without Giving Up CUDA Graphs": deduplicate the
 * experts and rewrite logical ids to physical cache slots on the GPU; the
 * slot table of moe_expert_weights is the second half).
 *   counts   [E] int32 input (device)
 *   active   [E] int32 output (device): active[j] for j < *n_active is the
 *            j-th expert with counts[e] > 0; the rest are set to -1
 *   n_active one int32 output (device)
 * One workgroup, no host synchronisation. */
int moe_active_experts(const moe_shape *s, const int32_t *counts, int32_t *active,
                       int32_t *n_active, void *stream);

/* Grouped expert FFN (forward-pass section): for every expert e, the rows
 * offsets[e] .. offsets[e+1] of x_perm go through expert e:
 *   y_perm[r] = (silu(x_perm[r] W1_e^T) * (x_perm[r] W3_e^T)) W2_e^T
 *   x_perm  [n*k][d] activations (act)
 *   offsets [E+1]    int32, device, as produced by moe_dispatch
 *   y_perm  [n*k][d] output, out = MOE_F32, or MOE_BF16 (the f32 pile
 *           outputs rounded once to nearest even; y_perm 16-byte aligned)
 *   ws      device workspace of at least moe_workspace_bytes(s, w->dtype).
 * offsets is read on the device only; empty experts cost nothing.
 * With BF16/MXFP4 weights, x_perm and y_perm must be 16-byte aligned.
 * W4A8 mode: x_perm is bf16 (encoded here) or already MXFP8
 * (act = MOE_MXFP8, an MXFP8 matrix of n*k rows). */
int moe_grouped_ffn(const moe_shape *s, const void *x_perm, int act,
                    const int32_t *offsets, const moe_expert_weights *w,
                    void *y_perm, int out, void *ws, size_t ws_bytes,
                    void *stream);

/* The two halves of moe_grouped_ffn, for callers that want them apart.
 *
 * moe_expert_up: h[r] = silu(a[src(r)] W1_e^T) * (a[src(r)] W3_e^T) for the
 *   rows r of every pile e ("Dense models" section: up-projection and
 *   activation).  src(r) = perm[r] when perm is not NULL (the rows are
 *   gathered from the token matrix x [n][d]), else r (a = x_perm [n*k][d]).
 *   h [n*k][d_ff] output: bf16 for BF16/MXFP4 weights (rounded to nearest
 *   even), f32 for F32 weights.
 * moe_expert_down: y_perm[r] = h[r] W2_e^T ("Dense models" section:
 *   down-projection), y_perm [n*k][d] f32.
 * offsets [E+1] as produced by moe_dispatch; read on the device only.
 * With BF16/MXFP4 weights, a, h and y_perm must be 16-byte aligned.
 * W4A8 mode: a is an MXFP8 matrix (act = MOE_MXFP8) of n rows (with perm)
 * or n*k rows, and h is an MXFP8 matrix of n*k rows x d_ff. */
int moe_expert_up(const moe_shape *s, const void *a, int act, const int32_t *perm,
                  const int32_t *offsets, const moe_expert_weights *w, void *h,
                  void *stream);
int moe_expert_down(const moe_shape *s, const void *h, const int32_t *offsets,
                    const moe_expert_weights *w, float *y_perm, void *stream);

/* Combine (forward-pass and Top-K sections): put the weighted pile rows
 * back in token order and add the k contributions:
 *   y[t] = sum_{j<k} topk_w[t][j] * y_perm[inv[t][j]]
 * summed in slot order in float32, then rounded to `out` (F32 or BF16).
 *   y_perm [n*k][d], in = MOE_F32 or MOE_BF16 (bf16 pile outputs, as
 *   moe_grouped_ffn writes with out = MOE_BF16; then d % 8 == 0, else
 *   MOE_ERR_SHAPE); inv, topk_w [n][k]; y [n][d].
 * A pair whose inv entry is outside [0, n*k) (moe_dispatch's -1 for an id
 * outside [0, E)) adds nothing. */
int moe_combine(const moe_shape *s, const void *y_perm, int in,
                const int32_t *inv, const float *topk_w, void *y, int out,
                void *stream);

/* The whole layer: router + top-k, dispatch, grouped FFN, combine.
 *   x [n][d] (act), wg [E][d] (act), bias [E] f32 or NULL, w: experts,
 *   y [n][d] output (out = act, or F32),
 *   topk_idx / topk_w: optional [n][k] outputs (NULL = keep internal),
 *   ws: workspace of at least moe_workspace_bytes(s, w->dtype) bytes,
 *       16-byte aligned; its contents on entry do not matter.
 * W4A8 mode: x must be bf16; it is encoded to MXFP8 for the experts. */
int moe_forward(const moe_shape *s, const void *x, int act, const void *wg,
                const float *bias, const moe_expert_weights *w, void *y,
                int out, int32_t *topk_idx, float *topk_w, void *ws,
                size_t ws_bytes, void *stream);

/* The whole layer, as moe_forward, without a workspace argument: for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The workspace is
 * a fixed array of MOE_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * per device, held from the first call on that device until the process
 * ends; the call itself allocates nothing.
 *   Arguments and results: as moe_forward.
 *   MOE_ERR_WORKSPACE when the shape needs more than the array holds
 *   (moe_workspace_bytes(s, w->dtype) > MOE_NOALLOC_SCRATCH_BYTES, e.g.
 *   the 128-expert MXFP4 layer at d = d_ff = 2880 up to about 400 tokens);
 *   argument errors are reported first, as by moe_forward.
 *   Every call on a device uses that device's one array, and the array
 *   keeps what the last call left in it (no call depends on that content).
 *   Calls that can overlap on one device -- on different streams without an
 *   order between them, or from several host threads -- race on the array;
 *   such callers use moe_forward with a workspace each. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_forward_noalloc(const moe_shape *s, const void *x, int act, const void *wg,
                        const float *bias, const moe_expert_weights *w, void *y, int out,
                        int32_t *topk_idx, float *topk_w, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_MI355X_H */
