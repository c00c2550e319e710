"""GPU parity of moe_dispatch: counts, offsets, perm, inv and the gathered
rows must equal the oracle's stable grouping exactly."""

import numpy as np
import pytest

import oracle
from tests.gpu_support import SMALL, layer_of, oracle_routing, say
from mixture_experts_layer_wave_amd import workloads as W

pytestmark = pytest.mark.gpu


def _run_dispatch(idx_np, E, x_np=None, chunked=False):
    import torch
    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import to_device

    n, k = idx_np.shape
    idx = to_device(idx_np.astype(np.int32))
    counts = torch.full((E,), -7, dtype=torch.int32, device="cuda")
    offsets = torch.full((E + 1,), -7, dtype=torch.int32, device="cuda")
    perm = torch.full((n * k,), -7, dtype=torch.int32, device="cuda")
    inv = torch.full((n, k), -7, dtype=torch.int32, device="cuda")
    xp = None
    x = None
    act = "bf16"
    if x_np is not None:
        x = to_device(x_np)
        act = "f32" if x_np.dtype == np.float32 else "bf16"
        xp = torch.empty((n * k, x_np.shape[1]), dtype=x.dtype, device="cuda")
    d = 1 if x_np is None else x_np.shape[1]
    shape = (n, d, E, k, 1, -1)
    ws, ws_bytes = None, 0
    if chunked:  # scratch for the two-pass form (used above 1024 pairs)
        ws_bytes = B.moe_dispatch_workspace_bytes(shape)
        ws = torch.full((max(ws_bytes, 16),), 0x5A, dtype=torch.uint8, device="cuda")
    B.moe_dispatch(shape, idx, counts, offsets, perm, inv, x, act, xp, ws, ws_bytes)
    torch.cuda.synchronize()
    out = {key: t.cpu().numpy() for key, t in
           (("counts", counts), ("offsets", offsets), ("perm", perm), ("inv", inv))}
    if xp is not None:
        out["x_perm"] = xp.cpu().numpy()
    return out


def _check(got, ref):
    for key in ("counts", "offsets", "perm", "inv"):
        assert np.array_equal(got[key], ref[key]), key


@pytest.mark.parametrize("chunked", [False, True])
@pytest.mark.parametrize("name", list(SMALL) + list(W.WORKLOADS))
def test_dispatch_of_routed_workloads(name, chunked):
    say(f"[dispatch] {name} chunked={chunked}")
    L = layer_of(name)
    ref = oracle_routing(L)
    got = _run_dispatch(ref["idx"], L["E"], L["x"], chunked)
    _check(got, ref)
    xp = got["x_perm"]
    want = L["x"][ref["perm"]]
    assert np.array_equal(xp.view(want.dtype) if xp.dtype != want.dtype else xp, want)


@pytest.mark.parametrize("chunked", [False, True])
@pytest.mark.parametrize("case", ["one-expert", "empty-experts", "many-chunks", "n1", "e1", "dup-slots",
                                  "small-256", "small-dups", "small-e1024", "small-257",
                                  "tiny-dups", "tiny-e128",
                                  "chunks-1025", "chunks-2048-e1024"])
def test_dispatch_edge_cases(case, chunked):
    say(f"[dispatch-edge] {case} chunked={chunked}")
    rng = np.random.default_rng(sum(map(ord, case)))
    if case == "one-expert":
        E, idx = 8, np.full((3000, 1), 5)
    elif case == "empty-experts":
        E = 64
        idx = rng.choice([3, 17, 40], size=(777, 2))
    elif case == "many-chunks":
        E = 1000
        idx = rng.integers(0, E, size=(4111, 4))
    elif case == "n1":
        E, idx = 128, np.array([[127, 0, 64, 63]])
    elif case == "e1":
        E, idx = 1, np.zeros((50, 1))
    elif case == "small-256":  # the one-wave path at its largest: 4 chunks of 64 pairs
        E, idx = 128, rng.integers(0, 128, size=(64, 4))
    elif case == "tiny-dups":  # at most 8 pairs (the readlane form): repeats, empty experts
        E, idx = 5, rng.choice([1, 3, 4], size=(4, 2))
    elif case == "tiny-e128":  # at most 8 pairs over 128 experts (two per lane)
        E, idx = 128, rng.integers(0, 128, size=(2, 4))
    elif case == "small-dups":  # one-wave path, few experts, repeated slots
        E, idx = 3, rng.integers(0, 3, size=(70, 3))
    elif case == "small-e1024":  # one-wave path, offsets scanned over 16 chunks of experts
        E, idx = 1024, rng.integers(0, 1024, size=(25, 4))
    elif case == "small-257":  # one pair past the one-wave path
        E, idx = 16, rng.integers(0, 16, size=(257, 1))
    elif case == "chunks-1025":  # one pair past a single chunk of the two-pass form
        E, idx = 8, rng.integers(0, 8, size=(1025, 1))
    elif case == "chunks-2048-e1024":  # two full chunks, most experts empty in each
        E, idx = 1024, rng.integers(0, 1024, size=(512, 4))
    else:  # a token may list the same expert twice: still a valid grouping input
        E = 4
        idx = rng.integers(0, E, size=(1500, 3))
    idx = idx.astype(np.int32)
    ref = oracle.dispatch(idx, E)
    got = _run_dispatch(idx, E, chunked=chunked)
    _check(got, ref)
