"""Graph replay of the decode chain: four consecutive 128-expert MXFP4
decode layers (n = 1), each with its own weights and its own input token,
captured in one HIP graph.  The routing is dynamic (which experts a token
reads is decided on the device), yet the captured launches stay valid: no
entry point reads anything back to the host, and the FFN grids are sized
for the worst case.  Every replay must reproduce the eager outputs bit for
bit, and each layer must match the oracle."""

import numpy as np
import pytest

import oracle
from tests.gpu_support import TOL, layer_of, oracle_routing, row_rel_err, say
from tests.golden.make_routing_fixtures import find_redraws
from mixture_experts_layer_wave_amd import workloads as W

pytestmark = pytest.mark.gpu

N_LAYERS = 4


def _layers():
    base = W.WORKLOADS[W.DECODE[0]]
    out = [layer_of(W.DECODE[0])]
    for i in range(1, N_LAYERS):
        wl = W.scaled(base, f"decode-n1-layer{i}", layer_seed=base.layer_seed + 100 * i,
                      x_seed=base.x_seed + 100 * i)
        out.append(W.make_layer(wl, redraws=find_redraws(wl), use_fixture=False, cache=False))
    return out


def test_graph_of_four_decode_layers_matches_eager_and_oracle():
    import torch
    from mixture_experts_layer_wave_amd.device import DeviceLayer

    say("[graph] four decode n=1 layers")
    Ls = _layers()
    Ds = [DeviceLayer(L) for L in Ls]
    # eager, then the oracle per layer (routing exact, outputs within tolerance)
    for D in Ds:
        D.forward()
    torch.cuda.synchronize()
    eager = [(D.y.clone(), D.idx.clone(), D.topw.clone()) for D in Ds]
    for i, (L, D) in enumerate(zip(Ls, Ds)):
        ref = oracle_routing(L)
        assert np.array_equal(D.idx.cpu().numpy(), ref["idx"]), i
        want = oracle.forward(L, L["k"], L["renorm"])["y"]
        err = row_rel_err(D.y_f64(), want)
        say(f"    layer {i}: experts {D.idx.cpu().numpy()[0].tolist()}  row rel err {err:.3e}")
        assert err <= TOL["mxfp4"]
    # the four layers in one graph, captured on a side stream
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        for D in Ds:
            D.forward(stream=s)
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=s):
            for D in Ds:
                D.forward(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        for D in Ds:  # eager work between replays: clear every output
            D.y.fill_(0)
            D.idx.fill_(-1)
            D.topw.fill_(0)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (D, (y, idx, tw)) in enumerate(zip(Ds, eager)):
            assert torch.equal(D.y, y), (rep, i)
            assert torch.equal(D.idx, idx), (rep, i)
            assert torch.equal(D.topw.view(torch.int32), tw.view(torch.int32)), (rep, i)
