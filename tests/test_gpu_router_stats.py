"""GPU parity of moe_router_stats (P_i, f_i and the load-balancing loss)
against the float64 oracle, and the page's two worked tables.

f_i comes from integer counts, so it matches to float32 rounding; P_i and the
loss are sums of float32 softmax values (relative error ~1e-6), held to 1e-4."""

import numpy as np
import pytest

import oracle
from tests.gpu_support import SMALL, layer_of, oracle_routing, say
from mixture_experts_layer_wave_amd import workloads as W

pytestmark = pytest.mark.gpu

NAMES = ["tiny-f32-n6-d3-e4-top1", "bf16-ragged", "mxfp4-ragged", "bf16-e1024-k32", W.SWITCH,
         W.DECODE[2], W.PREFILL_ZIPF]


def _stats(shape, logits, idx, alpha):
    import torch
    from mixture_experts_layer_wave_amd import binding as B

    E = B._shape(shape).E
    P = torch.full((E,), float("nan"), device="cuda")
    f = torch.full((E,), float("nan"), device="cuda")
    loss = torch.full((1,), float("nan"), device="cuda")
    nb = B.moe_router_stats_workspace_bytes(shape)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda")
    B.moe_router_stats(shape, logits, idx, alpha, P, f, loss, ws, nb)
    torch.cuda.synchronize()
    return P.double().cpu().numpy(), f.double().cpu().numpy(), float(loss.item())


@pytest.mark.parametrize("name", NAMES)
def test_router_stats_match_oracle(name):
    import torch
    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import DeviceLayer

    say(f"[router-stats] {name}")
    L = layer_of(name)
    D = DeviceLayer(L)
    logits = torch.empty((D.n, D.E), dtype=torch.float32, device="cuda")
    B.moe_router_topk(D.shape, D.x, D.act, D.wg, D.bias, logits, D.idx, D.topw)
    alpha = 0.01
    P, f, loss = _stats(D.shape, logits, D.idx, alpha)
    ref = oracle_routing(L)
    want = oracle.aux_loss(ref["p"], ref["idx"], alpha=alpha)
    np.testing.assert_allclose(f, want["f"], rtol=1e-6, atol=0)
    np.testing.assert_allclose(P, want["P"], rtol=1e-4, atol=1e-7)
    assert abs(loss - want["loss"]) <= 1e-4 * abs(want["loss"])
    # determinism: a second call gives the same bits
    P2, f2, loss2 = _stats(D.shape, logits, D.idx, alpha)
    assert np.array_equal(P, P2) and np.array_equal(f, f2) and loss == loss2


def test_router_stats_page_tables():
    """The page's tables: four tokens that all pick expert 1 with mean
    p_1 = 0.5825 give 4 x 0.5825 = 2.33 (x alpha = 0.0233); one argmax per
    expert gives exactly 1 (x alpha = 0.01)."""
    import json
    import os

    import torch

    gold = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "page_examples.json")))["aux_loss"]
    p = np.array([[0.60, 0.20, 0.10, 0.10],
                  [0.55, 0.15, 0.15, 0.15],
                  [0.63, 0.07, 0.20, 0.10],
                  [0.55, 0.25, 0.10, 0.10]])
    shape = (4, 8, 4, 1, 8)
    z = torch.tensor(np.log(p), dtype=torch.float32, device="cuda")
    idx = torch.zeros((4, 1), dtype=torch.int32, device="cuda")
    P, f, loss = _stats(shape, z, idx, gold["alpha"])
    assert f.tolist() == gold["unbalanced"]["f"]
    assert abs(P[0] - gold["unbalanced"]["P1"]) < 1e-6
    assert abs(loss - gold["terms_added"][0]) < 1e-6
    assert round(loss / gold["alpha"], 2) == gold["unbalanced"]["loss_over_alpha_2dp"]
    pb = np.full((4, 4), 0.2) + 0.2 * np.eye(4)
    zb = torch.tensor(np.log(pb), dtype=torch.float32, device="cuda")
    idxb = torch.arange(4, dtype=torch.int32, device="cuda").reshape(4, 1)
    P, f, loss = _stats(shape, zb, idxb, 1.0)
    assert f.tolist() == gold["balanced"]["f"]
    assert abs(loss - gold["balanced"]["loss_over_alpha"]) < 1e-6
