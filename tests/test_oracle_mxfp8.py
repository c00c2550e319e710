"""Pins of the oracle's MXFP8 activation quantisation and of its W4A8 mode
(MXFP8 activations times MXFP4 weights) to the E4M3 format's definition, a
library decoder, brute force over every code, and invariants of the layer.

The encoding rules are those of OCP Microscaling Formats v1.0 (E4M3
element of the OCP 8-bit floating point format; shared exponent =
floor(log2 amax) - 8; round to nearest even; clamp to +-448)."""

import math

import numpy as np
import pytest
import torch

import oracle
from mixture_experts_layer_wave_amd import workloads as W

# ------------------------------------------------------------ E4M3 element


def test_e4m3_decode_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.decode_e4m3(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert nan.sum() == 2 and nan[0x7F] and nan[0xFF]
    assert np.array_equal(got[~nan], ref[~nan])


def test_e4m3_spec_values():
    d = lambda c: float(oracle.decode_e4m3(np.array([c]))[0])
    assert d(0x7E) == 448.0            # largest magnitude, S.1111.110
    assert d(0x08) == 2.0 ** -6        # smallest normal
    assert d(0x01) == 2.0 ** -9        # smallest subnormal
    assert d(0x07) == 7 * 2.0 ** -9    # largest subnormal
    assert d(0x38) == 1.0 and d(0xB8) == -1.0
    assert d(0x00) == 0.0 and math.copysign(1.0, d(0x80)) == -1.0
    pos = oracle.decode_e4m3(np.arange(0x7F))
    assert np.all(np.diff(pos) > 0)    # monotone, all distinct


def test_encode_is_the_inverse_of_decode():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(oracle.encode_e4m3(oracle.decode_e4m3(codes)), codes)


# ------------------------------------------------------- the block encoder

# every finite non-negative E4M3 magnitude, and its code
_POS_CODES = np.arange(0x7F)
_POS_VALS = oracle.decode_e4m3(_POS_CODES)


def _brute_force_block(block):
    """Shared exponent by search, then each element by exhaustive nearest
    search over the 127 magnitudes (ties to the even code), clamped."""
    amax = np.abs(block).max()
    if amax == 0:
        s = 0
    else:
        # the scale 2^(s-127) that puts amax in [2^8, 2^9)
        s = next(s for s in range(0, 255) if amax < 2.0 ** (s - 127) * 512)
        s = max(s, 0)
    X = s - 127
    out = []
    for v in block:
        a = abs(v) / 2.0 ** X
        dist = np.abs(_POS_VALS - a)
        best = np.flatnonzero(dist == dist.min())
        code = int(best[0]) if len(best) == 1 else int([c for c in best if c % 2 == 0][0])
        out.append(code | (0x80 if math.copysign(1.0, v) < 0 else 0))
    return np.array(out, dtype=np.uint8), s


@pytest.mark.parametrize("seed", range(6))
def test_quantizer_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    rows = []
    for kind in range(8):
        b = rng.standard_normal(32) * 10.0 ** rng.uniform(-6, 6)
        if kind == 1:
            b[rng.integers(32)] *= 1e4          # wide dynamic range inside a block
        if kind == 2:
            b[:16] = 0.0                         # zeros and -0.0
            b[3] = -0.0
        if kind == 3:
            b[:] = 0.0                           # all-zero block
        if kind == 4:                            # exact ties between two E4M3 values
            b = np.ldexp(np.array([1 + (2 * i + 1) / 16 for i in range(8)] * 4), 3) * rng.choice([-1, 1], 32)
            b[0] = 256.0
        if kind == 5:                            # values that clamp at 448 * 2^X
            b = rng.uniform(-1, 1, 32)
            b[7] = 1.99
        rows.append(b)
    v = np.array(rows)
    codes, scales = oracle.quantize_mxfp8(v)
    for r in range(v.shape[0]):
        want_c, want_s = _brute_force_block(v[r])
        assert scales[r, 0] == want_s
        assert np.array_equal(codes[r], want_c), (r, codes[r], want_c)


def test_quantizer_closed_cases():
    blk = np.zeros(32)
    blk[0] = 1.0
    c, s = oracle.quantize_mxfp8(blk)
    assert s[0] == 127 - 8 and c[0] == 0x78      # 1.0 = 2^8 * 2^-8, S.1111.000
    blk[0] = 500.0                               # 500 in [256, 512): scale 1, clamps to 448
    c, s = oracle.quantize_mxfp8(blk)
    assert s[0] == 127 and c[0] == 0x7E
    blk[0] = -0.75                               # floor(log2 .75) = -1
    c, s = oracle.quantize_mxfp8(blk)
    assert s[0] == 127 - 9 and oracle.decode_e4m3(c[:1])[0] * 2.0 ** -9 == -0.75
    c, s = oracle.quantize_mxfp8(np.zeros(32))
    assert s[0] == 0 and np.all(c == 0)


def test_quantizer_agrees_with_torch_cast_in_range():
    """Inside +-448 * 2^X the element is the round-to-nearest-even cast of
    v / 2^X (torch's float8_e4m3fn conversion)."""
    rng = np.random.default_rng(9)
    v = rng.standard_normal((64, 256)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    codes, scales = oracle.quantize_mxfp8(v)
    scaled = v.reshape(64, 8, 32) / np.ldexp(1.0, scales.astype(np.int64) - 127)[..., None]
    t = torch.from_numpy(scaled).to(torch.float8_e4m3fn).view(torch.uint8).numpy().reshape(64, 256)
    inside = np.abs(scaled.reshape(64, 256)) <= 448
    assert inside.mean() > 0.9
    assert np.array_equal(codes[inside], t[inside])


def test_blocks_are_32_along_the_last_axis():
    """A block of large values next to blocks of small ones: each 32-block
    keeps its own relative precision (2^-4), and the scales follow each
    block's own amax.  (Magnitudes stay below 1.75 times a power of two, so
    no element reaches the clamp at 448 * 2^X.)"""
    rng = np.random.default_rng(4)
    v = rng.uniform(0.5, 0.85, (3, 128)) * 2.0 ** -10
    v[:, 32:64] *= 2.0 ** 30
    r = oracle.mxfp8_round(v)
    assert np.all(np.abs(r - v) <= np.abs(v) * 2.0 ** -4)
    _, s = oracle.quantize_mxfp8(v)
    assert np.all(s[:, 1] - s[:, 0] == 30) and np.all(s[:, 0] == s[:, 2])
    assert np.all(s[:, 0] == 127 - 11 - 8)


def test_round_is_idempotent():
    rng = np.random.default_rng(2)
    v = rng.standard_normal((16, 96))
    r = oracle.mxfp8_round(v)
    assert np.array_equal(oracle.mxfp8_round(r), r)


# -------------------------------------------------------- the W4A8 layer


def _small_mx_layer(n=12, d=64, E=4, k=2, f=96, seed=31):
    wl = W.scaled(W.WORKLOADS[W.PREFILL_ZIPF], f"w4a8-pin-{seed}", n=n, d=d, E=E, k=k, d_ff=f,
                  zipf_s=0.0, layer_seed=seed, x_seed=seed + 1)
    return W.make_layer(wl, use_fixture=False, cache=False)


def test_w4a8_quantises_the_expert_input():
    """Replacing x by its MXFP8 value changes nothing for the experts (the
    router sees x itself, so the routing is pinned to x's)."""
    L = _small_mx_layer()
    a = oracle.forward(L, k=2, act_quant="mxfp8")
    xq = oracle.mxfp8_round(oracle.decode_bf16(L["x"]))
    d = oracle.decode_bf16(L["x"])
    assert not np.array_equal(xq, d)
    # the expert outputs of the same routing, computed from the rounded x
    y = np.zeros_like(d)
    for e in range(L["E"]):
        w1 = oracle.decode_mxfp4(L["w1"][e], L["s1"][e])
        w3 = oracle.decode_mxfp4(L["w3"][e], L["s3"][e])
        w2 = oracle.decode_mxfp4(L["w2"][e], L["s2"][e])
        m = (a["idx"] == e) * a["w"]
        y += m.sum(axis=1, keepdims=True) * oracle.swiglu_expert(xq, w1, w3, w2, "mxfp8")
    np.testing.assert_allclose(a["y"], y, rtol=0, atol=1e-12)


def test_w4a8_hidden_is_on_the_mxfp8_grid():
    """With W2 the identity (exact in MXFP4: code 1.0, scale 2^0) one expert
    returns its quantised hidden activation: every 32-block of the output is
    on the MXFP8 grid, and within the format's 2^-4 relative step (plus the
    clamp of the block's top values) of the unquantised hidden."""
    L = _small_mx_layer(n=9, d=64, E=1, k=1, f=64, seed=7)
    eye_codes = np.where(np.eye(64) > 0, 2, 0).astype(np.uint8)
    L["w2"] = (eye_codes[:, 0::2] | (eye_codes[:, 1::2] << 4))[None]
    L["s2"] = np.full((1, 64, 2), 127, np.uint8)
    assert np.array_equal(oracle.decode_mxfp4(L["w2"][0], L["s2"][0]), np.eye(64))
    q = oracle.forward(L, k=1, act_quant="mxfp8")["y"]
    assert np.array_equal(oracle.mxfp8_round(q), q)
    xq = oracle.mxfp8_round(oracle.decode_bf16(L["x"]))
    w1 = oracle.decode_mxfp4(L["w1"][0], L["s1"][0])
    w3 = oracle.decode_mxfp4(L["w3"][0], L["s3"][0])
    h = oracle.swiglu_expert(xq, w1, w3, np.eye(64))       # no quantisation at all
    amax = np.repeat(np.abs(h).reshape(9, 2, 32).max(axis=2), 32, axis=1)
    assert np.all(np.abs(q - h) <= np.maximum(np.abs(h) * 2.0 ** -4, amax * 2.0 ** -3) + 1e-12)
    assert not np.array_equal(q, h)


def test_w4a8_is_token_permutation_equivariant():
    L = _small_mx_layer(seed=41)
    a = oracle.forward(L, k=2, act_quant="mxfp8")
    perm = np.random.default_rng(0).permutation(L["x"].shape[0])
    L2 = dict(L, x=L["x"][perm])
    b = oracle.forward(L2, k=2, act_quant="mxfp8")
    np.testing.assert_allclose(b["y"], a["y"][perm], rtol=0, atol=1e-12)


def test_w4a8_power_of_two_scaling_of_the_value_path():
    """h = silu(x W1) * (x W3) scales with W3; a power of two moves every
    block's shared exponent and leaves the codes alone, so y scales exactly.
    A factor of 1.3 does not (the hidden is re-rounded)."""
    L = _small_mx_layer(seed=51)
    a = oracle.forward(L, k=2, act_quant="mxfp8")["y"]
    L4 = dict(L, s3=(L["s3"].astype(np.int64) + 2).astype(np.uint8))  # W3 * 4
    b = oracle.forward(L4, k=2, act_quant="mxfp8")["y"]
    assert np.array_equal(b, 4 * a)
    # W2 is after the last rounding: any factor passes straight through
    L5 = dict(L, s2=(L["s2"].astype(np.int64) - 1).astype(np.uint8))  # W2 / 2
    c = oracle.forward(L5, k=2, act_quant="mxfp8")["y"]
    assert np.array_equal(c, a / 2)


def test_w4a8_is_close_to_the_unquantised_layer():
    L = _small_mx_layer(n=16, d=128, E=4, k=2, f=128, seed=61)
    q = oracle.forward(L, k=2, act_quant="mxfp8")["y"]
    p = oracle.forward(L, k=2)["y"]
    rel = np.abs(q - p).max(axis=1) / np.abs(p).max(axis=1)
    assert rel.max() < 0.1 and rel.max() > 1e-4
