"""GPU parity of the W4A8 mode (MXFP8 activations times MXFP4 weights on
the scaled MFMA) against the oracle's act_quant='mxfp8' layer, and of the
MXFP8 encoder against the oracle's, bit for bit."""

import numpy as np
import pytest

import oracle
from tests.gpu_support import TOL, oracle_routing, row_rel_err, sample_rows, say, small
from tests.golden import make_routing_fixtures as RF
from mixture_experts_layer_wave_amd import workloads as W

pytestmark = pytest.mark.gpu


def _split_mx8(buf: np.ndarray, rows: int, cols: int):
    off = (rows * cols + 255) // 256 * 256
    sp = (cols // 32 + 3) // 4 * 4
    return buf[: rows * cols].reshape(rows, cols), buf[off: off + rows * sp].reshape(rows, sp)


def _encode_case(rows, cols, seed):
    """Rows with a wide spread of magnitudes, all-zero blocks, negative zeros
    and tiny negatives next to large values (they round to -0)."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((rows, cols)) * np.exp(rng.uniform(-20, 20, (rows, 1)))
    x *= np.exp(rng.uniform(-3, 3, (rows, cols // 32))).repeat(32, axis=1)
    if cols >= 64:
        x[::3, 32:64] = 0.0
        x[1::5, 5] = -0.0
        x[2::7, 0] = -abs(x[2::7, 1]) * 1e-6
    return x


@pytest.mark.parametrize("rows,cols,act", [(1, 32, "bf16"), (37, 96, "bf16"), (300, 2880, "bf16"),
                                           (64, 160, "f32"), (5, 7168, "f32")])
def test_mxfp8_encoder_is_bit_exact(rows, cols, act):
    import torch

    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import to_device

    say(f"[w4a8 encode] rows {rows} cols {cols} {act}")
    x = _encode_case(rows, cols, rows * 7 + cols)
    if act == "bf16":
        xs = W.bf16_bits(x)
        xv = oracle.decode_bf16(xs)
    else:
        xs = x.astype(np.float32)
        xv = oracle.decode_f32(xs)
    q = torch.full((B.moe_mxfp8_bytes(rows, cols),), 0xAA, dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(rows, cols, to_device(xs), act, q)
    torch.cuda.synchronize()
    codes, scales = _split_mx8(q.cpu().numpy(), rows, cols)
    want_c, want_s = oracle.quantize_mxfp8(xv)
    nb = cols // 32
    assert np.array_equal(scales[:, :nb], want_s)
    assert np.all(scales[:, nb:] == 0)
    bad = np.argwhere(codes != want_c)
    assert bad.size == 0, (bad[:5], codes[tuple(bad[0])], want_c[tuple(bad[0])])


# Layers for the mode: K tails of 64 in both projections (d, d_ff = 64 mod
# 128), one expert per token, a single token, several row tiles per pile.
# Up to 1024 routed rows take the weight-streaming kernel, more the GEMM.
W4A8_SMALL = {
    "w4a8-ragged": small("w4a8-ragged", 300, 320, 8, 2, 448, "mxfp4", 21),
    "w4a8-k1": small("w4a8-k1", 200, 256, 4, 1, 384, "mxfp4", 22),
    "w4a8-n1": small("w4a8-n1", 1, 128, 16, 4, 96, "mxfp4", 23),
    "w4a8-deep": small("w4a8-deep", 700, 192, 3, 2, 2880, "mxfp4", 24),
    "w4a8-gemm-ragged": small("w4a8-gemm-ragged", 700, 320, 8, 2, 448, "mxfp4", 25),
}
STREAM_CASE, GEMM_CASE = "w4a8-ragged", "w4a8-gemm-ragged"


def _layer(name):
    if name in W.WORKLOADS:
        return W.make_layer(name, cache=True)
    wl = W4A8_SMALL[name]
    return W.make_layer(wl, redraws=RF.find_redraws(wl), use_fixture=False, cache=False)


def _device(L):
    import torch

    from mixture_experts_layer_wave_amd.device import DeviceLayer

    D = DeviceLayer(L, act_quant="mxfp8")
    D.forward()
    torch.cuda.synchronize()
    return D


@pytest.mark.parametrize("name", list(W4A8_SMALL) + list(W.DECODE) + [W.PREFILL_ZIPF])
def test_w4a8_forward_matches_oracle(name):
    say(f"[w4a8 forward] {name}")
    L = _layer(name)
    D = _device(L)
    ref = oracle_routing(L)
    assert np.array_equal(D.idx.cpu().numpy(), ref["idx"])
    rows = np.arange(L["n"]) if L["n"] <= 512 else sample_rows(L["n"], ref["idx"], ref["counts"])
    want = oracle.forward(L, L["k"], L["renorm"], rows=rows, act_quant="mxfp8")["y"]
    got = D.y_f64()[rows]
    err = row_rel_err(got, want)
    plain = oracle.forward(L, L["k"], L["renorm"], rows=rows[:8])["y"]
    say(f"    rows {len(rows)}  max row rel err {err:.3e} "
        f"(the unencoded layer differs by {row_rel_err(got[:8], plain):.3e})")
    assert err <= TOL["mxfp4"]
    assert np.isfinite(D.y_f64()).all()


@pytest.mark.parametrize("name", [STREAM_CASE, GEMM_CASE])
def test_w4a8_hidden_against_oracle(name):
    """The up projection alone: its MXFP8 hidden decodes to the oracle's
    encoded hidden up to a code flip where float32 and float64 round
    differently (rare, one E4M3 step); padding scale bytes are 0."""
    import torch

    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import to_device

    say(f"[w4a8 hidden] {name}")
    L = _layer(name)
    ref = oracle_routing(L)
    n, d, E, k, f = (L[key] for key in ("n", "d", "E", "k", "d_ff"))
    R = n * k
    D = _device(L)
    xq = torch.empty(B.moe_mxfp8_bytes(n, d), dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(n, d, D.x, "bf16", xq)
    off = to_device(ref["offsets"])
    perm = to_device(ref["perm"])
    h = torch.empty(B.moe_mxfp8_bytes(R, f), dtype=torch.uint8, device="cuda")
    B.moe_expert_up(D.shape, xq, "mxfp8", perm, off, D.weights, h)
    torch.cuda.synchronize()
    hc, hs = _split_mx8(h.cpu().numpy(), R, f)
    assert np.all(hs[:, f // 32:] == 0)
    got = oracle.decode_mxfp8(hc, hs[:, : f // 32])
    x = oracle.mxfp8_round(oracle.decode_bf16(L["x"]))
    want = np.zeros((R, f))
    for e in range(E):
        rs = slice(ref["offsets"][e], ref["offsets"][e + 1])
        w1 = oracle.decode_mxfp4(L["w1"][e], L["s1"][e])
        w3 = oracle.decode_mxfp4(L["w3"][e], L["s3"][e])
        xe = x[ref["perm"][rs]]
        g, u = xe @ w1.T, xe @ w3.T
        want[rs] = oracle.mxfp8_round(g / (1 + np.exp(-g)) * u)
    flips = np.mean(got != want)
    say(f"    hidden code flips {flips:.2e}, max row rel err {row_rel_err(got, want):.3e}")
    assert flips < 1e-2
    assert row_rel_err(got, want) <= 2 ** -3


@pytest.mark.parametrize("name", [STREAM_CASE, GEMM_CASE])
def test_w4a8_grouped_ffn_bf16_and_mxfp8_inputs_agree(name):
    """moe_grouped_ffn encodes bf16 pile rows itself; handing it the same
    rows already encoded gives the same bits."""
    import torch

    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import to_device

    say(f"[w4a8 grouped] {name}")
    L = _layer(name)
    ref = oracle_routing(L)
    n, d, k = L["n"], L["d"], L["k"]
    R = n * k
    D = _device(L)
    xp = to_device(L["x"][ref["perm"]])
    off = to_device(ref["offsets"])
    y1 = torch.empty((R, d), dtype=torch.float32, device="cuda")
    y2 = torch.empty_like(y1)
    B.moe_grouped_ffn(D.shape, xp, "bf16", off, D.weights, y1, "f32", D.ws, D.ws_bytes)
    xq = torch.empty(B.moe_mxfp8_bytes(R, d), dtype=torch.uint8, device="cuda")
    B.moe_quantize_mxfp8(R, d, xp, "bf16", xq)
    B.moe_grouped_ffn(D.shape, xq, "mxfp8", off, D.weights, y2, "f32", D.ws, D.ws_bytes)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    # and the pile outputs are the oracle's expert outputs
    x = oracle.mxfp8_round(oracle.decode_bf16(L["x"]))
    want = np.zeros((R, d))
    for e in range(L["E"]):
        rs = slice(ref["offsets"][e], ref["offsets"][e + 1])
        w1 = oracle.decode_mxfp4(L["w1"][e], L["s1"][e])
        w3 = oracle.decode_mxfp4(L["w3"][e], L["s3"][e])
        w2 = oracle.decode_mxfp4(L["w2"][e], L["s2"][e])
        want[rs] = oracle.swiglu_expert(x[ref["perm"][rs]], w1, w3, w2, "mxfp8")
    assert row_rel_err(y1.double().cpu().numpy(), want) <= TOL["mxfp4"]


@pytest.mark.parametrize("name", [STREAM_CASE, GEMM_CASE])
def test_w4a8_slots_are_bit_exact(name):
    """Weights stored in shuffled physical slots, with the slot table,
    give the same bits as the weights in expert order."""
    import torch

    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import DeviceLayer, to_device

    say(f"[w4a8 slots] {name}")
    L = _layer(name)
    E = L["E"]
    A = _device(L)
    slot = np.random.default_rng(3).permutation(E).astype(np.int32)
    phys = dict(L)
    for key in ("w1", "w3", "w2", "s1", "s3", "s2"):
        arr = np.empty_like(L[key])
        arr[slot] = L[key]
        phys[key] = arr
    P = DeviceLayer(phys, act_quant="mxfp8")
    st = to_device(slot)
    P.weights.slot = B._ptr(st)
    P.weights.n_slots = E
    P.forward()
    torch.cuda.synchronize()
    assert torch.equal(A.y, P.y)
