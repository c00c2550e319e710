"""Pins of the oracle to closed forms, library routines, invariants and brute
force, chosen so that a dropped term, a wrong sign or index, or a transposed
operand anywhere in it fails at least one test."""

import itertools
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from mixture_experts_layer_wave_amd import workloads as W

# ---------------------------------------------------------------- decoders


def test_bf16_decode_matches_torch():
    rng = np.random.default_rng(0)
    bits = rng.integers(0, 1 << 16, size=20000, dtype=np.uint64).astype(np.uint16)
    # drop NaN patterns (exponent all ones, nonzero mantissa): NaN != NaN
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    bits = bits[~((e == 0xFF) & (m != 0))]
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode_bf16(bits)
    assert np.array_equal(got, ref)
    assert oracle.decode_bf16(np.array([0x3F80, 0xC000, 0x0001], np.uint16)).tolist() == [1.0, -2.0, 2.0 ** -133]


# OCP Microscaling Formats v1.0, FP4 E2M1 element: the 8 magnitudes.
OCP_E2M1 = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def test_e2m1_table():
    got = oracle.decode_e2m1(np.arange(16))
    assert got[:8].tolist() == OCP_E2M1
    assert got[8:].tolist() == [-v for v in OCP_E2M1]


def test_e8m0_matches_torch():
    s = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(s).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    got = oracle.decode_e8m0(s)
    assert np.array_equal(got[:255], ref[:255])
    assert math.isnan(got[255]) and math.isnan(ref[255])


def test_mxfp4_nibble_order_and_block_scale():
    # one row of K = 64: two blocks; byte j holds k = 2j (low) and 2j + 1 (high)
    codes = np.arange(64) % 16
    packed = (codes[0::2] | (codes[1::2] << 4)).astype(np.uint8)[None]
    scales = np.array([[127 + 3, 127 - 2]], np.uint8)
    got = oracle.decode_mxfp4(packed, scales)[0]
    want = np.array([(1 if c < 8 else -1) * OCP_E2M1[c % 8] for c in codes], dtype=np.float64)
    want[:32] *= 8.0
    want[32:] *= 0.25
    assert np.array_equal(got, want)


def test_mxfp4_encoder_roundtrip_is_nearest():
    """The workload encoder picks, for each element, the representable value
    nearest to its scaled draw (checked with the oracle's decoder)."""
    rng = np.random.default_rng(3)
    w = (rng.standard_normal((8, 96)) / math.sqrt(96)).astype(np.float32)
    packed, s = W.mxfp4_encode(w)
    dec = oracle.decode_mxfp4(packed, s)
    scale = np.repeat(oracle.decode_e8m0(s), 32, axis=1)
    grid = np.array(OCP_E2M1)
    v = np.abs(w / scale)
    nearest = grid[np.argmin(np.abs(v[..., None] - grid), axis=-1)]
    assert np.array_equal(np.abs(dec / scale), nearest)
    assert np.all((dec == 0) | (np.sign(dec) == np.sign(w)))
    # the block amax lands in [4, 8) before rounding, as the shared-exponent rule intends
    amax = np.abs(w.reshape(8, 3, 32)).max(axis=2) / oracle.decode_e8m0(s)
    assert np.all((amax >= 4) & (amax < 8))


def test_bf16_encoder_is_round_to_nearest_even():
    rng = np.random.default_rng(1)
    a = rng.standard_normal(10000).astype(np.float32) * 10
    ref = torch.from_numpy(a).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(W.bf16_bits(a), ref)


# ---------------------------------------------------------------- router


def test_router_and_softmax_against_torch():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((7, 5))
    wg = rng.standard_normal((6, 5))
    b = rng.standard_normal(6)
    z = oracle.router_logits(x, wg, b)
    zt = F.linear(torch.tensor(x), torch.tensor(wg), torch.tensor(b)).numpy()
    np.testing.assert_allclose(z, zt, rtol=1e-13, atol=1e-13)
    p = oracle.softmax_rows(z)
    np.testing.assert_allclose(p, torch.softmax(torch.tensor(z), dim=1).numpy(), rtol=1e-13)
    np.testing.assert_allclose(p.sum(axis=1), 1.0, rtol=1e-14)
    # huge logits do not overflow (safe softmax)
    pb = oracle.softmax_rows(z + 1000.0)
    np.testing.assert_allclose(pb, p, rtol=1e-12)


@pytest.mark.parametrize("E,k", [(4, 1), (5, 2), (8, 2), (8, 3), (6, 6)])
def test_topk_matches_subset_brute_force(E, k):
    """Top-k = the k-subset with the largest logit sum (checked over all
    C(E, k) subsets), listed best first; ties go to the lower index."""
    rng = np.random.default_rng(E * 10 + k)
    z = rng.standard_normal((50, E))
    idx = oracle.topk_select(z, k)
    for t in range(z.shape[0]):
        best = max(itertools.combinations(range(E), k), key=lambda s: sum(z[t, list(s)]))
        assert sorted(idx[t].tolist()) == sorted(best)
        assert all(z[t, idx[t, j]] > z[t, idx[t, j + 1]] for j in range(k - 1))
    zt = np.zeros((1, E))
    zt[0, [1, 3]] = 2.0
    assert oracle.topk_select(zt, 2)[0].tolist() == [1, 3]
    assert oracle.topk_select(np.zeros((1, E)), 1)[0, 0] == 0


def test_topk_weights_closed_forms():
    rng = np.random.default_rng(4)
    z = rng.standard_normal((30, 8))
    p = oracle.softmax_rows(z)
    idx = oracle.topk_select(z, 3)
    w = oracle.topk_weights(p, idx, renorm=True)
    np.testing.assert_allclose(w.sum(axis=1), 1.0, rtol=1e-14)
    # renormalised weights are the softmax over the chosen logits only
    sel = np.take_along_axis(z, idx.astype(np.int64), axis=1)
    np.testing.assert_allclose(w, torch.softmax(torch.tensor(sel), dim=1).numpy(), rtol=1e-13)
    w1 = oracle.topk_weights(p, idx[:, :1], renorm=False)
    np.testing.assert_allclose(w1[:, 0], p.max(axis=1), rtol=0)


# ---------------------------------------------------------------- layer


def _f32_layer(n, d, E, k, f, seed, same_experts=False):
    rng = np.random.default_rng(seed)
    mk = lambda *s: (rng.standard_normal(s) / math.sqrt(s[-1])).astype(np.float32)
    w1, w3, w2 = mk(E, f, d), mk(E, f, d), mk(E, d, f)
    if same_experts:
        w1[:] = w1[0]
        w3[:] = w3[0]
        w2[:] = w2[0]
    return {"x": rng.standard_normal((n, d)).astype(np.float32), "x_dtype": "f32",
            "wg": mk(E, d), "bias": None, "w1": w1, "w3": w3, "w2": w2, "w_dtype": "f32"}


def _torch_ffn(x, w1, w3, w2):
    t = lambda a: torch.tensor(np.asarray(a, np.float64))
    return F.linear(F.silu(F.linear(t(x), t(w1))) * F.linear(t(x), t(w3)), t(w2)).numpy()


def test_single_expert_is_the_dense_ffn():
    L = _f32_layer(9, 6, 1, 1, 10, 11)
    out = oracle.forward(L, k=1)
    assert np.all(out["w"] == 1.0)
    np.testing.assert_allclose(out["y"], _torch_ffn(L["x"], L["w1"][0], L["w3"][0], L["w2"][0]), rtol=1e-12, atol=1e-14)


def test_k_equals_E_is_the_soft_mixture():
    L = _f32_layer(7, 5, 4, 4, 8, 12)
    out = oracle.forward(L, k=4)
    p = torch.softmax(torch.tensor(L["x"], dtype=torch.float64) @ torch.tensor(L["wg"], dtype=torch.float64).T, 1).numpy()
    mix = sum(p[:, e:e + 1] * _torch_ffn(L["x"], L["w1"][e], L["w3"][e], L["w2"][e]) for e in range(4))
    np.testing.assert_allclose(out["y"], mix, rtol=1e-11, atol=1e-14)


def test_identical_experts():
    L = _f32_layer(8, 4, 5, 2, 6, 13, same_experts=True)
    ffn = _torch_ffn(L["x"], L["w1"][0], L["w3"][0], L["w2"][0])
    np.testing.assert_allclose(oracle.forward(L, k=2)["y"], ffn, rtol=1e-12, atol=1e-14)
    o1 = oracle.forward(L, k=1)
    np.testing.assert_allclose(o1["y"], o1["p"].max(axis=1, keepdims=True) * ffn, rtol=1e-12, atol=1e-14)


def test_token_permutation_equivariance_and_rows_subset():
    L = _f32_layer(12, 6, 6, 2, 7, 14)
    full = oracle.forward(L, k=2)
    perm = np.random.default_rng(0).permutation(12)
    Lp = dict(L, x=L["x"][perm])
    outp = oracle.forward(Lp, k=2)
    np.testing.assert_allclose(outp["y"], full["y"][perm], rtol=1e-13, atol=1e-15)
    assert np.array_equal(outp["idx"], full["idx"][perm])
    sub = oracle.forward(L, k=2, rows=[3, 7, 1])
    np.testing.assert_allclose(sub["y"], full["y"][[3, 7, 1]], rtol=1e-13, atol=1e-15)


def test_linearity_in_w2_and_bias_shift():
    L = _f32_layer(10, 4, 4, 2, 6, 15)
    y = oracle.forward(L, k=2)["y"]
    L2 = dict(L, w2=L["w2"] * np.float32(4.0))
    np.testing.assert_allclose(oracle.forward(L2, k=2)["y"], 4.0 * y, rtol=1e-13, atol=1e-15)
    # a bias equal for every expert changes nothing; a large one on expert 2 forces it
    Lb = dict(L, bias=np.full(4, 3.0, np.float32))
    np.testing.assert_allclose(oracle.forward(Lb, k=2)["y"], y, rtol=1e-12, atol=1e-15)
    Lf = dict(L, bias=np.array([0, 0, 60, 0], np.float32))
    o = oracle.forward(Lf, k=2)
    assert np.all(o["idx"][:, 0] == 2)


def test_whole_layer_against_an_independent_sparse_loop():
    """Sparse evaluation (only chosen experts, token by token, in torch)
    equals the dense-then-masked oracle, on bf16 and MXFP4 weights."""
    for wdt in ("bf16", "mxfp4"):
        wl = W.Workload(f"t-{wdt}", 13, 64, 6, 3, 96, "bf16", wdt, 77, 78)
        L = W.make_layer(wl, use_fixture=False, cache=False)
        out = oracle.forward(L, k=3)
        x = oracle.decode_bf16(L["x"])
        wg = oracle.decode_bf16(L["wg"])
        p = torch.softmax(torch.tensor(x) @ torch.tensor(wg).T, 1).numpy()
        y = np.zeros_like(x)
        for t in range(13):
            top = np.argsort(-p[t])[:3]
            ws = p[t, top] / p[t, top].sum()
            for e, we in zip(top, ws):
                if wdt == "mxfp4":
                    m = [oracle.decode_mxfp4(L[a][e], L[s][e]) for a, s in (("w1", "s1"), ("w3", "s3"), ("w2", "s2"))]
                else:
                    m = [oracle.decode_bf16(L[a][e]) for a in ("w1", "w3", "w2")]
                y[t] += we * _torch_ffn(x[t:t + 1], *m)[0]
        np.testing.assert_allclose(out["y"], y, rtol=1e-10, atol=1e-13)


# ---------------------------------------------------------------- dispatch


def _dispatch_by_token_loop(idx, E):
    piles = [[] for _ in range(E)]
    for t in range(idx.shape[0]):
        for j in range(idx.shape[1]):
            piles[idx[t, j]].append((t, j))
    return piles


@pytest.mark.parametrize("n,E,k", [(6, 4, 1), (40, 8, 2), (33, 16, 4), (5, 8, 8), (20, 3, 1)])
def test_dispatch_brute_force(n, E, k):
    rng = np.random.default_rng(n + E + k)
    z = rng.standard_normal((n, E))
    if E == 16:
        z[:, 3] += 10  # every token hits expert 3; others sparse
    idx = oracle.topk_select(z, k)
    dp = oracle.dispatch(idx, E)
    piles = _dispatch_by_token_loop(idx, E)
    assert dp["counts"].tolist() == [len(p) for p in piles]
    assert dp["offsets"][0] == 0 and dp["offsets"][-1] == n * k
    for e in range(E):
        rows = list(range(dp["offsets"][e], dp["offsets"][e + 1]))
        assert [int(dp["perm"][r]) for r in rows] == [t for t, _ in piles[e]]
        for r, (t, j) in zip(rows, piles[e]):
            assert dp["inv"][t, j] == r
    assert sorted(dp["inv"].reshape(-1).tolist()) == list(range(n * k))


# ---------------------------------------------------------------- workloads


def test_workload_margins_hold_and_seeds_are_deterministic():
    import tests.golden.make_routing_fixtures as M

    for name in (W.SWITCH, W.PREFILL_ZIPF) + W.DECODE:
        wl = W.WORKLOADS[name]
        fx = W.routing_fixture(name)
        bias = W.bias_from_hex(fx["bias_f32_hex"]) if fx.get("bias_f32_hex") else None
        z = M.logits64(wl, fx["redraws"], bias)
        assert M.margin_violations(z, wl.k).size == 0
    a = W.draw_x(W.WORKLOADS[W.SWITCH])
    b = W.draw_x(W.WORKLOADS[W.SWITCH])
    assert np.array_equal(a, b)


def test_zipf_bias_skews_load():
    import tests.golden.make_routing_fixtures as M

    wl = W.WORKLOADS[W.PREFILL_ZIPF]
    fx = W.routing_fixture(wl.name)
    z = M.logits64(wl, fx["redraws"], W.bias_from_hex(fx["bias_f32_hex"]))
    load = np.bincount(oracle.topk_select(z, wl.k).reshape(-1), minlength=wl.E)
    tgt = W.zipf_targets(wl)
    assert np.abs(load - tgt).sum() < 0.06 * wl.R
    assert load.max() > 3000 and load.min() < 32
