"""GPU parity of moe_router_topk against the float64 oracle.

Expert indices must match exactly (inputs are drawn with top-(k+1) logit
margins >= 1e-4); logits and weights within float32 accumulation error."""

import numpy as np
import pytest

from tests.gpu_support import SMALL, layer_of, oracle_routing, say
from mixture_experts_layer_wave_amd import workloads as W

pytestmark = pytest.mark.gpu

NAMES = list(SMALL) + list(W.WORKLOADS)


@pytest.mark.parametrize("name", NAMES)
def test_router_topk_matches_oracle(name):
    import torch
    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import DeviceLayer

    say(f"[router] {name}")
    L = layer_of(name)
    D = DeviceLayer(L)
    logits = torch.empty((D.n, D.E), dtype=torch.float32, device="cuda")
    B.moe_router_topk(D.shape, D.x, D.act, D.wg, D.bias, logits, D.idx, D.topw)
    torch.cuda.synchronize()
    ref = oracle_routing(L)
    z = logits.double().cpu().numpy()
    assert np.abs(z - ref["z"]).max() <= 1e-4 + 1e-5 * np.abs(ref["z"]).max()
    idx = D.idx.cpu().numpy()
    assert np.array_equal(idx, ref["idx"]), f"{(idx != ref['idx']).any(axis=1).sum()} tokens differ"
    w = D.topw.double().cpu().numpy()
    np.testing.assert_allclose(w, ref["w"], rtol=2e-5, atol=1e-7)
