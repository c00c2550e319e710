"""GPU behaviour on inputs outside the generated workloads: a token whose
activations are NaN, and expert ids outside [0, E) handed to moe_dispatch.
Nothing here may read or write outside the buffers; the checks are that
every chosen id stays in range and that the other tokens are unaffected."""

import numpy as np
import pytest

import oracle
from tests.gpu_support import TOL, layer_of, oracle_routing, row_rel_err, say
from mixture_experts_layer_wave_amd import workloads as W

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", ["bf16-ragged", "mxfp4-n4-e128", "mxfp4-gemm-ragged", W.DECODE[2]])
def test_nan_token_keeps_ids_in_range_and_others_unchanged(name):
    import torch
    from mixture_experts_layer_wave_amd.device import DeviceLayer

    say(f"[nan token] {name}")
    L = layer_of(name)
    ref = oracle_routing(L)
    t_bad = L["n"] // 2
    x = np.array(L["x"], copy=True)
    x[t_bad] = 0x7FC0 if L["x_dtype"] == "bf16" else np.float32("nan")  # quiet NaN
    Ln = dict(L, x=x)
    D = DeviceLayer(Ln)
    D.forward()
    torch.cuda.synchronize()
    idx = D.idx.cpu().numpy()
    assert ((idx >= 0) & (idx < L["E"])).all()
    # the NaN token's experts are the lowest k ids, its weights NaN
    assert idx[t_bad].tolist() == list(range(L["k"]))
    assert np.isnan(D.topw.cpu().numpy()[t_bad]).all()
    keep = np.array([t for t in range(L["n"]) if t != t_bad])
    assert np.array_equal(idx[keep], ref["idx"][keep])
    sel = keep if len(keep) <= 256 else np.unique(np.concatenate([keep[:64], keep[-64:], keep[::37]]))
    want = oracle.forward(L, L["k"], L["renorm"], rows=sel)["y"]
    got = D.y_f64()[sel]
    assert np.isfinite(got).all()
    assert row_rel_err(got, want) <= TOL[L["w_dtype"]]


@pytest.mark.parametrize("n,k,E,ws", [(2, 4, 128, False), (3, 2, 9, False), (40, 3, 9, False),
                                      (900, 2, 16, False), (1500, 4, 128, True),
                                      (1500, 4, 128, False), (5000, 4, 64, False)])
def test_dispatch_skips_ids_outside_range(n, k, E, ws):
    """Pairs with ids outside [0, E) go to no pile: inv = -1 for them, the
    piles of the others match the oracle's scan, the pile rows past the
    last pile hold perm = -1 and gather zeros, and the combine adds nothing
    for the skipped pairs."""
    import torch
    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import to_device

    say(f"[dispatch invalid ids] n={n} k={k} E={E} ws={ws}")
    rng = np.random.default_rng(n + E)
    idx = np.stack([rng.choice(E, size=k, replace=False) for _ in range(n)]).astype(np.int32)
    bad = rng.random(idx.shape) < 0.05
    if n * k <= 8:  # few pairs (the readlane dispatch): always some bad ids
        bad.flat[1] = bad.flat[-1] = True
    idx[bad] = rng.choice([-1, E, E + 7, -(1 << 30)], size=int(bad.sum()))
    want = oracle.dispatch(idx, E)  # scans ids 0..E-1 only
    R = n * k
    used = int(want["offsets"][-1])
    assert used == R - int(bad.sum())
    shape = (n, 8, E, k, 8)
    counts = torch.empty(E, dtype=torch.int32, device="cuda")
    offsets = torch.empty(E + 1, dtype=torch.int32, device="cuda")
    perm = torch.full((R,), 12345, dtype=torch.int32, device="cuda")
    inv = torch.full((n, k), 12345, dtype=torch.int32, device="cuda")
    d = 8
    x = torch.arange(n * d, dtype=torch.float32, device="cuda").reshape(n, d)
    xp = torch.full((R, d), 7.0, dtype=torch.float32, device="cuda")
    nws = B.moe_dispatch_workspace_bytes(shape) if ws else 0
    wsb = torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda")
    B.moe_dispatch(shape, to_device(idx), counts, offsets, perm, inv, x, "f32", xp,
                   wsb if ws else None, nws)
    torch.cuda.synchronize()
    assert np.array_equal(counts.cpu().numpy(), want["counts"])
    assert np.array_equal(offsets.cpu().numpy(), want["offsets"])
    p = perm.cpu().numpy()
    assert np.array_equal(p[:used], want["perm"])
    assert (p[used:] == -1).all()
    assert np.array_equal(inv.cpu().numpy(), want["inv"])
    xpn = xp.cpu().numpy()
    assert np.array_equal(xpn[:used], x.cpu().numpy()[want["perm"]])
    assert (xpn[used:] == 0).all()
    # combine: the skipped pairs add nothing
    yp = rng.standard_normal((R, d)).astype(np.float32)
    w = rng.random((n, k)).astype(np.float32)
    y = torch.empty((n, d), dtype=torch.float32, device="cuda")
    B.moe_combine(shape, to_device(yp), "f32", inv, to_device(w), y, "f32")
    torch.cuda.synchronize()
    inv_n = want["inv"]
    ref = np.zeros((n, d))
    for j in range(k):
        ok = inv_n[:, j] >= 0
        ref[ok] += w[ok, j:j + 1].astype(np.float64) * yp[inv_n[ok, j]].astype(np.float64)
    np.testing.assert_allclose(y.double().cpu().numpy(), ref, rtol=1e-5, atol=1e-6)
