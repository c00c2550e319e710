"""Float64 CPU oracle of the sparse MoE layer forward (TEST INFRASTRUCTURE).

Only tests, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may use this module.  It shares no code with the HIP library.

Sources, cited by page title and section:

* [MoE] "How Mixture of Experts Scales Model Parameters" (zhangchitc.github.io):
  - section "Dense models: every parameter in the FFN does work for every
    token": the FFN maps an n x d input to n x d through an up-projection W1
    (d x d_ff), an activation and a down-projection W2 (d_ff x d), token by
    token.
  - section "Routing: a router scores the experts, and the top one runs":
    the router is one d x E linear layer W_g followed by a softmax over each
    row; with one expert per token the chosen expert's output is scaled by
    its probability (0.45 in the page's example).
  - section "The forward pass: dispatch, then combine": tokens are regrouped
    into per-expert piles (possibly empty), each expert runs on its pile,
    rows are weighted and put back in token order.
  - section "Top-K: several experts, added up by weight": the K best experts
    are kept and their probabilities renormalised over the K before the
    weighted sum.
  - section "Load balancing: how collapse happens, and how it's kept in
    check": the equations for P_i, f_i and the auxiliary loss.
* [FA] "Why FlashAttention is So Fast", section "A fused kernel, and an
  overflow problem": safe softmax subtracts the row maximum before exp.
* [FT] minseoc03.com feed, review of the FreeToken paper: the GPU-side
  bookkeeping of an expert cache (deduplicated expert sets, logical ids
  rewritten to physical slots).
* [MX] minseoc03.com feed, note "What is MXFP4?": 4-bit floats in blocks of
  32 that share one scale.  The bit layout (e2m1 element, e8m0 scale) is not
  on the pages; it is read from the OCP Microscaling Formats v1.0
  specification.
* [VL] minseoc03.com feed, review of the vLLM paper, section "What's Next":
  quantised weights are usually expanded back to a wider type before the
  arithmetic, and that expansion eats the gain.  The W4A8 mode below is the
  alternative: activations are quantised too (to MXFP8) so that the matrix
  unit takes both operands in their narrow form.  The MXFP8 element (E4M3)
  and the rule that picks a block's shared scale are not on the pages; they
  are read from OCP Microscaling Formats v1.0 (the E4M3 element of the OCP
  8-bit floating point format: bias 7, no infinities, S.1111.111 is NaN,
  largest magnitude 448; shared exponent = floor(log2(block amax)) minus the
  element's largest exponent, 8; elements rounded to nearest even and
  clamped to +-448).

Readings where the pages are silent (each listed in the design notes):

* the activation is SwiGLU, ``silu(x W1) * (x W3)`` then ``W2``;
* with K = 1 the weight is the raw probability; with K > 1 it is
  renormalised over the chosen K;
* the softmax runs over all E logits (bias included), and selection is by
  descending float64 logit with ties to the lower expert index (generated
  inputs keep every top-(k+1) gap at >= 1e-4, so float32 kernels make the
  same choice);
* within a pile rows are ordered by token, then by slot.

Stored layouts read by this module (the HIP library reads the same bytes):

* ``x``   [n][d]       bf16 (uint16 bits) or float32
* ``wg``  [E][d]       same dtype as x (the page's W_g transposed)
* ``bias``[E]          float32 or None
* ``w1``, ``w3`` [E][d_ff][d] and ``w2`` [E][d][d_ff]: bf16 / float32, or
  MXFP4 packed bytes [E][N][K/2] (low nibble = even k) with e8m0 scales
  ``s1``, ``s3``, ``s2`` of shape [E][N][K/32].

Parity status: every function here is pinned by a test in
``tests/test_oracle_*.py`` (worked examples, closed forms, invariants,
library routines, brute force).
"""

from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# Decoders: raw bytes -> float64.  Independent of the HIP path.
# ---------------------------------------------------------------------------


def decode_bf16(u16: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns (uint16) -> float64.

    bfloat16 is the upper half of an IEEE binary32 word, so the value is the
    float32 whose top 16 bits are the pattern and whose low 16 bits are zero.
    """
    u16 = np.ascontiguousarray(u16, dtype=np.uint16)
    return (u16.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def decode_f32(a: np.ndarray) -> np.ndarray:
    """float32 -> float64 (exact)."""
    return np.asarray(a, dtype=np.float32).astype(np.float64)


def decode_e2m1(code: np.ndarray) -> np.ndarray:
    """FP4 E2M1 element codes (0..15) -> float64, from the format's definition.

    Bit 3 is the sign, bits 2..1 the exponent (bias 1), bit 0 the mantissa.
    Exponent field 0 is subnormal: value = m * 2^(1-1) * 0.5.  Otherwise
    value = 2^(e-1) * (1 + m/2).  No infinities or NaNs exist in E2M1.
    [MX]: the element type of an MXFP4 block.
    """
    code = np.asarray(code).astype(np.int64)
    sign = np.where((code >> 3) & 1, -1.0, 1.0)
    e = (code >> 1) & 3
    m = code & 1
    mag = np.where(e == 0, 0.5 * m, np.ldexp(1.0 + 0.5 * m, e - 1))
    return sign * mag


def decode_e8m0(s: np.ndarray) -> np.ndarray:
    """E8M0 shared-scale codes (0..255) -> float64: 2^(s-127); 255 is NaN.

    [MX]: one scale per block of 32 values.
    """
    s = np.asarray(s).astype(np.int64)
    v = np.ldexp(1.0, s - 127)
    return np.where(s == 255, np.nan, v)


def decode_mxfp4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP4 rows -> float64.

    ``packed`` [..., K/2] uint8 holds two E2M1 codes per byte, the element
    with the even K index in the low nibble.  ``scales`` [..., K/32] uint8
    holds one E8M0 scale per 32 consecutive elements along K.  Each value is
    ``e2m1(code) * 2^(scale-127)``  [MX].
    """
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    K = packed.shape[-1] * 2
    if scales.shape[-1] * 32 != K:
        raise ValueError("scale count does not match K/32")
    # Each of the 256 byte values decoded once into its two elements, the
    # low nibble (even K) first; the bytes then index that table.
    b = np.arange(256)
    pair = np.stack([decode_e2m1(b & 0x0F), decode_e2m1(b >> 4)], axis=-1)  # [256][2]
    vals = pair[packed].reshape(*packed.shape[:-1], K // 32, 32)
    vals *= decode_e8m0(scales)[..., None]
    return vals.reshape(*packed.shape[:-1], K)


def decode_e4m3(code: np.ndarray) -> np.ndarray:
    """FP8 E4M3 element codes (0..255) -> float64, from the format's definition.

    Bit 7 is the sign, bits 6..3 the exponent (bias 7), bits 2..0 the
    mantissa.  Exponent field 0 is subnormal: m/8 * 2^-6.  Otherwise
    2^(e-7) * (1 + m/8).  Exponent 15 with mantissa 7 is NaN; there are no
    infinities, so the largest magnitude is 1.75 * 2^8 = 448.  [VL] (OCP).
    """
    code = np.asarray(code).astype(np.int64)
    sign = np.where((code >> 7) & 1, -1.0, 1.0)
    e = (code >> 3) & 15
    m = code & 7
    mag = np.where(e == 0, np.ldexp(m / 8.0, -6), np.ldexp(1.0 + m / 8.0, e - 7))
    return np.where((code & 0x7F) == 0x7F, np.nan, sign * mag)


E4M3_MAX = 448.0
E4M3_EMAX = 8  # exponent of the largest power of two the element reaches


def _floor_log2(a: np.ndarray) -> np.ndarray:
    """floor(log2 a) for a > 0, exactly (frexp: a = f 2^e with f in [0.5, 1))."""
    return np.frexp(a)[1].astype(np.int64) - 1


def round_e4m3(a: np.ndarray) -> np.ndarray:
    """Non-negative float64 -> the nearest E4M3 magnitude, ties to even.

    In the binade [2^e, 2^(e+1)) (e >= -6) E4M3 has 8 steps of 2^(e-3);
    below 2^-6 the subnormal step is 2^-9.  Rounding a / step to the
    nearest integer with ties to even (numpy's round) and scaling back
    gives the nearest value; a carry into the next binade lands on its
    first value, which is exact.  Values above 448 saturate to 448.  [VL]
    """
    a = np.asarray(a, dtype=np.float64)
    e = np.where(a > 0, _floor_log2(np.where(a > 0, a, 1.0)), -6)
    step = np.ldexp(1.0, np.maximum(e, -6) - 3)
    return np.minimum(np.round(a / step) * step, E4M3_MAX)


def encode_e4m3(v: np.ndarray) -> np.ndarray:
    """Code of values that are exactly E4M3 magnitudes with a sign (float64,
    |v| <= 448); the sign bit is the sign bit of v, so -0.0 gives 0x80."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    sub = a < 2.0 ** -6
    e = np.where(sub, 0, _floor_log2(np.where(sub, 1.0, a)) + 7)
    m = np.where(sub, a / 2.0 ** -9, (a / np.ldexp(1.0, np.maximum(e, 1) - 7) - 1.0) * 8)
    code = (e.astype(np.int64) << 3) | np.rint(m).astype(np.int64)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


def quantize_mxfp8(v: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """MXFP8 encoding of float64 rows: blocks of 32 consecutive values along
    the last axis share one E8M0 scale 2^X, each element is an E4M3 code.

    X = floor(log2 amax) - 8 with amax the block's largest magnitude (the
    block's largest element lands in [256, 512) * 2^X, and values above
    448 * 2^X are clamped); an all-zero block takes the smallest scale,
    code 0.  X is clamped to the E8M0 range [-127, 127].  Each element is
    v / 2^X (exact: a power of two) rounded to the nearest E4M3 value, ties
    to even.  Returns (codes uint8 [..., K], scales uint8 [..., K/32]).  [VL]
    """
    v = np.asarray(v, dtype=np.float64)
    K = v.shape[-1]
    if K % 32:
        raise ValueError("the last axis must be a multiple of 32")
    blocks = v.reshape(*v.shape[:-1], K // 32, 32)
    amax = np.abs(blocks).max(axis=-1)
    X = np.where(amax > 0, _floor_log2(np.where(amax > 0, amax, 1.0)) - E4M3_EMAX, -127)
    X = np.clip(X, -127, 127)
    scaled = blocks / np.ldexp(1.0, X)[..., None]
    q = np.copysign(round_e4m3(np.abs(scaled)), scaled)
    codes = encode_e4m3(q).reshape(v.shape)
    return codes, (X + 127).astype(np.uint8)


def decode_mxfp8(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """MXFP8 rows -> float64: e4m3(code) * 2^(scale - 127) per 32-block."""
    codes = np.asarray(codes, dtype=np.uint8)
    K = codes.shape[-1]
    vals = decode_e4m3(codes).reshape(*codes.shape[:-1], K // 32, 32)
    return (vals * decode_e8m0(scales)[..., None]).reshape(codes.shape)


def mxfp8_round(v: np.ndarray) -> np.ndarray:
    """The value v takes after MXFP8 encoding and decoding."""
    return decode_mxfp8(*quantize_mxfp8(v))


def decode_matrix(raw: np.ndarray, dtype: str, scales: np.ndarray | None = None) -> np.ndarray:
    """Decode one stored operand ('bf16', 'f32' or 'mxfp4') to float64."""
    if dtype == "bf16":
        return decode_bf16(raw)
    if dtype == "f32":
        return decode_f32(raw)
    if dtype == "mxfp4":
        if scales is None:
            raise ValueError("mxfp4 needs scales")
        return decode_mxfp4(raw, scales)
    raise ValueError(f"unknown dtype {dtype!r}")


# ---------------------------------------------------------------------------
# Router: [MoE] "Routing: a router scores the experts, and the top one runs"
# ---------------------------------------------------------------------------


def router_logits(x: np.ndarray, wg_t: np.ndarray, bias: np.ndarray | None = None) -> np.ndarray:
    """Z = X W_g (+ b): one logit per (token, expert).

    ``x`` is n x d, ``wg_t`` is the stored E x d matrix (W_g transposed), so
    the product with the page's d x E matrix W_g is ``x @ wg_t.T``.  The bias
    is not on the pages; when present it is added to every row.
    """
    z = x @ wg_t.T
    if bias is not None:
        z = z + np.asarray(bias, dtype=np.float64)[None, :]
    return z


def softmax_rows(z: np.ndarray) -> np.ndarray:
    """Row softmax, computed the safe way.

    [MoE] routing section: softmax is applied to each row of the n x E
    matrix.  [FA] overflow section: subtract the row maximum m before
    exponentiating; numerator and denominator are both scaled by e^-m, so
    the value is unchanged.
    """
    m = z.max(axis=1, keepdims=True)
    ez = np.exp(z - m)
    return ez / ez.sum(axis=1, keepdims=True)


def topk_select(z: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest logits of each row, best first.

    [MoE] "Top-K: several experts, added up by weight": keep the K experts
    with the highest scores (K = 1 is the argmax of the routing section).
    Softmax is increasing, so ranking logits ranks probabilities.  The
    ranking is taken on the float64 logits as given, with no rounding;
    equal values go to the lower expert index (stable sort).
    """
    z64 = np.asarray(z, dtype=np.float64)
    order = np.argsort(-z64, axis=1, kind="stable")
    return order[:, :k].astype(np.int32)


def topk_weights(p: np.ndarray, idx: np.ndarray, renorm: bool) -> np.ndarray:
    """Combine weights of the chosen experts.

    Without renormalisation the weight is the chosen expert's probability
    (the routing section scales expert 1's output by 0.45).  With it, the K
    probabilities are divided by their sum (the Top-K section: 0.45/0.76 =
    0.59 and 0.31/0.76 = 0.41).
    """
    sel = np.take_along_axis(p, idx.astype(np.int64), axis=1)
    if renorm:
        sel = sel / sel.sum(axis=1, keepdims=True)
    return sel


# ---------------------------------------------------------------------------
# Expert body: [MoE] "Dense models: ..." -- up-projection, activation, down.
# ---------------------------------------------------------------------------


def _silu(g: np.ndarray) -> np.ndarray:
    """SiLU(g) = g * sigmoid(g) = g / (1 + e^-g)."""
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu_expert(x: np.ndarray, w1_t: np.ndarray, w3_t: np.ndarray, w2_t: np.ndarray,
                  act_quant: str | None = None) -> np.ndarray:
    """One expert's FFN on the rows of ``x`` (n x d -> n x d).

    Up-projection to d_ff through W1 (gate) and W3 (value), the SiLU-gated
    product, and the down-projection W2 back to d.  Stored matrices are the
    transposes: ``w1_t``/``w3_t`` are d_ff x d, ``w2_t`` is d x d_ff.

    ``act_quant='mxfp8'`` (the W4A8 mode, [VL]): each projection's input
    rows -- x before the up-projection, the hidden h before the
    down-projection -- are replaced by their MXFP8 values, blocks of 32
    along the row (the contraction axis).
    """
    if act_quant not in (None, "mxfp8"):
        raise ValueError(f"unknown act_quant {act_quant!r}")
    if act_quant:
        x = mxfp8_round(x)
    g = x @ w1_t.T
    u = x @ w3_t.T
    h = _silu(g) * u
    if act_quant:
        h = mxfp8_round(h)
    return h @ w2_t.T


# ---------------------------------------------------------------------------
# The layer, dense then masked.
# ---------------------------------------------------------------------------


def _expert_mats(layer: dict, e: int):
    wd = layer["w_dtype"]
    if wd == "mxfp4":
        w1 = decode_mxfp4(layer["w1"][e], layer["s1"][e])
        w3 = decode_mxfp4(layer["w3"][e], layer["s3"][e])
        w2 = decode_mxfp4(layer["w2"][e], layer["s2"][e])
    else:
        w1 = decode_matrix(layer["w1"][e], wd)
        w3 = decode_matrix(layer["w3"][e], wd)
        w2 = decode_matrix(layer["w2"][e], wd)
    return w1, w3, w2


def forward(layer: dict, k: int, renorm: bool | None = None, rows=None,
            act_quant: str | None = None) -> dict:
    """The MoE layer forward on (a subset of) the tokens, in float64.

    ``layer`` holds the raw stored arrays: 'x', 'x_dtype' ('bf16'|'f32'),
    'wg', 'bias' (float32 or None), 'w1', 'w3', 'w2', 'w_dtype'
    ('bf16'|'f32'|'mxfp4') and, for MXFP4, 's1', 's3', 's2'.

    Steps ([MoE] routing, forward-pass and Top-K sections):
      1. Z = X W_g (+ b);  2. P = softmax of each row;
      3. the top-k experts of each token;  4. their weights (raw p for K = 1,
      renormalised over the K otherwise);
      5. EVERY expert's FFN on EVERY token (dense), then
      6. Y[t] = sum_e M[t, e] * FFN_e(X[t]) with M[t, e] the weight of e if it
         was chosen for t, else 0.
    The FFN treats tokens independently ([MoE] dense-model section), so the
    result for a subset ``rows`` of tokens equals those rows of the full
    result.  ``act_quant='mxfp8'`` runs every expert in the W4A8 mode of
    :func:`swiglu_expert`; the router still sees the unquantised x.
    """
    if renorm is None:
        renorm = k > 1
    xr = layer["x"] if rows is None else layer["x"][np.asarray(rows)]
    x = decode_matrix(xr, layer["x_dtype"])
    wg = decode_matrix(layer["wg"], layer["x_dtype"])
    E = wg.shape[0]
    if not (1 <= k <= E):
        raise ValueError("need 1 <= k <= E")
    z = router_logits(x, wg, layer.get("bias"))
    p = softmax_rows(z)
    idx = topk_select(z, k)
    w = topk_weights(p, idx, renorm)
    n = x.shape[0]
    mask = np.zeros((n, E), dtype=np.float64)
    for j in range(k):
        mask[np.arange(n), idx[:, j]] += w[:, j]
    y = np.zeros_like(x)
    for e in range(E):
        w1, w3, w2 = _expert_mats(layer, e)
        y += mask[:, e:e + 1] * swiglu_expert(x, w1, w3, w2, act_quant)
    return {"y": y, "idx": idx, "w": w, "p": p, "z": z}


def dispatch(idx: np.ndarray, E: int) -> dict:
    """Regroup the (token, slot) pairs into per-expert piles by scanning.

    [MoE] "The forward pass: dispatch, then combine": tokens routed to the
    same expert are pulled out, in their original order, into that expert's
    input matrix; an expert with no tokens has an empty pile.  Expert by
    expert, the (token, slot) pairs are visited in ascending token then slot
    order and appended.

    Returns counts[E], offsets[E+1] (pile e is rows offsets[e]..offsets[e+1]),
    perm[R] (token of each pile row) and inv[n][k] (pile row of each pair).
    """
    idx = np.asarray(idx, dtype=np.int64)
    n, k = idx.shape
    flat = idx.reshape(-1)  # position t*k + j, ascending token then slot
    counts = np.zeros(E, dtype=np.int32)
    perm = []
    inv = np.full(n * k, -1, dtype=np.int32)
    for e in range(E):
        pos = np.nonzero(flat == e)[0]
        counts[e] = pos.size
        inv[pos] = np.arange(len(perm), len(perm) + pos.size)
        perm.extend((pos // k).tolist())
    offsets = np.zeros(E + 1, dtype=np.int32)
    offsets[1:] = np.cumsum(counts)
    return {
        "counts": counts,
        "offsets": offsets,
        "perm": np.asarray(perm, dtype=np.int32),
        "inv": inv.reshape(n, k),
    }


def aux_loss(p: np.ndarray, idx: np.ndarray, alpha: float = 1.0) -> dict:
    """Load-balancing auxiliary loss.

    [MoE] load-balancing section: P_i is the mean probability of expert i
    over the batch, f_i the fraction of tokens whose argmax is i, and the
    loss is alpha * E * sum_i f_i P_i.  The argmax is the first selected
    expert of each token.
    """
    n, E = p.shape
    P = p.mean(axis=0)
    top1 = np.asarray(idx)[:, 0]
    f = np.bincount(top1, minlength=E).astype(np.float64) / n
    return {"P": P, "f": f, "loss": alpha * E * float(np.sum(f * P))}


def active_experts(idx: np.ndarray, E: int) -> np.ndarray:
    """The distinct experts a batch is routed to, ascending.

    [FT] minseoc03.com feed, review of FreeToken, sections "Decode: Exploit
    Expert Locality" and "Dynamic Scheduling Without Giving Up CUDA Graphs":
    the experts a batch needs are the deduplicated set of its routing
    choices.  Written as a set over the (token, slot) choices.
    """
    seen = set(int(e) for e in np.asarray(idx).reshape(-1) if 0 <= int(e) < E)
    return np.array(sorted(seen), dtype=np.int32)


def resolve_slots(phys: dict, slot: np.ndarray) -> dict:
    """Logical expert weights from physical slots: expert e's matrices are
    those of slot[e].

    [FT] same review, section "Dynamic Scheduling Without Giving Up CUDA
    Graphs": logical expert ids are rewritten to physical cache slots.  The
    mapping is a plain gather of the stored operands (every array whose
    first axis is the slot axis); nothing is decoded or recomputed.
    """
    out = dict(phys)
    for key in ("w1", "w3", "w2", "s1", "s3", "s2"):
        if phys.get(key) is not None:
            out[key] = np.asarray(phys[key])[np.asarray(slot)]
    return out
