"""Logical -> physical expert slots and the active-expert list on the GPU.

The slot table only moves where an expert's weights are read from, so a
layer whose weights sit in shuffled physical slots (with decoy slots in
between) must give the same bits as the same layer stored in expert order,
and both must match the float64 oracle on the logical weights.  Out-of-range
table entries are clamped into the slot range.  The active-expert list must
equal the oracle's deduplicated routing choices."""

import numpy as np
import pytest

import oracle
from tests.gpu_support import TOL, layer_of, oracle_routing, row_rel_err, sample_rows, say
from mixture_experts_layer_wave_amd import workloads as W

pytestmark = pytest.mark.gpu

KEYS = ("w1", "w3", "w2", "s1", "s3", "s2")


def _physical(L, extra, seed):
    """Weights of L moved into E + extra slots in a random order; decoy
    slots hold other random bytes of the same dtype."""
    rng = np.random.default_rng(seed)
    E = L["E"]
    P = E + extra
    pos = rng.permutation(P)[:E].astype(np.int32)  # slot of logical expert e
    phys = {}
    for key in KEYS:
        a = L.get(key)
        if a is None:
            phys[key] = None
            continue
        a = np.asarray(a)
        out = np.empty((P,) + a.shape[1:], dtype=a.dtype)
        raw = rng.integers(0, 256, size=out.nbytes, dtype=np.uint8).view(a.dtype).reshape(out.shape)
        if key in ("s1", "s3", "s2"):
            raw = rng.integers(118, 124, size=out.shape, dtype=np.uint8)
        elif a.dtype == np.float32:
            raw = rng.standard_normal(out.shape).astype(np.float32)
        out[:] = raw
        out[pos] = a
        phys[key] = out
    return phys, pos, P


def _forward_with(D, phys, slot_dev, P):
    import torch
    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import to_device

    dw = {key: to_device(phys[key]) for key in KEYS}
    w = B.ExpertWeights(B.DTYPES[D.wdt], *(B._ptr(dw[key]) for key in KEYS), B._ptr(slot_dev), P)
    y = torch.empty_like(D.y)
    B.moe_forward(D.shape, D.x, D.act, D.wg, D.bias, w, y, D.act, D.idx, D.topw, D.ws, D.ws_bytes)
    torch.cuda.synchronize()
    return y


@pytest.mark.parametrize("name", ["f32-small", "bf16-ragged", "mxfp4-ragged", "mxfp4-n1",
                                  W.DECODE[1], W.SWITCH])
def test_slot_table_matches_expert_order(name):
    import torch
    from mixture_experts_layer_wave_amd.device import DeviceLayer

    say(f"[slots] {name}")
    L = layer_of(name)
    D = DeviceLayer(L)
    D.forward()
    torch.cuda.synchronize()
    y_ref = D.y.clone()
    phys, pos, P = _physical(L, 3, 7)
    slot = torch.tensor(pos, dtype=torch.int32, device="cuda")
    y = _forward_with(D, phys, slot, P)
    assert torch.equal(y, y_ref)
    # the oracle on the logical weights gathered back from the slots
    Lr = oracle.resolve_slots(dict(L, **phys), pos)
    ref = oracle_routing(L)
    rows = np.arange(L["n"]) if L["n"] <= 512 else sample_rows(L["n"], ref["idx"], ref["counts"])
    want = oracle.forward(Lr, L["k"], L["renorm"], rows=rows)["y"]
    assert row_rel_err(D.y_f64(y)[rows], want) <= TOL[L["w_dtype"]]


def test_slot_entries_are_clamped():
    import torch
    from mixture_experts_layer_wave_amd.device import DeviceLayer

    L = layer_of("mxfp4-ragged")
    D = DeviceLayer(L)
    phys, pos, P = _physical(L, 2, 11)
    wild = pos.copy()
    wild[0], wild[1] = -5, P + 7
    clamped = np.clip(wild, 0, P - 1).astype(np.int32)
    y_wild = _forward_with(D, phys, torch.tensor(wild, device="cuda"), P)
    y_clamped = _forward_with(D, phys, torch.tensor(clamped, device="cuda"), P)
    assert torch.equal(y_wild, y_clamped)


@pytest.mark.parametrize("name", ["bf16-ragged", "bf16-e1024-k32", W.DECODE[0], W.DECODE[2],
                                  W.PREFILL_ZIPF])
def test_active_experts_match_oracle(name):
    import torch
    from mixture_experts_layer_wave_amd import binding as B

    L = layer_of(name)
    ref = oracle_routing(L)
    E = L["E"]
    counts = torch.tensor(np.bincount(ref["idx"].reshape(-1), minlength=E).astype(np.int32), device="cuda")
    active = torch.full((E,), 12345, dtype=torch.int32, device="cuda")
    n_active = torch.full((1,), -7, dtype=torch.int32, device="cuda")
    B.moe_active_experts((L["n"], L["d"], E, L["k"], L["d_ff"]), counts, active, n_active)
    torch.cuda.synchronize()
    want = oracle.active_experts(ref["idx"], E)
    m = int(n_active.item())
    assert m == len(want)
    got = active.cpu().numpy()
    assert np.array_equal(got[:m], want) and (got[m:] == -1).all()
