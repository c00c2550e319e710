"""moe_forward_noalloc (the entry point whose workspace is a fixed array in
the library) against moe_forward with a caller workspace: the same kernels,
so the outputs, expert ids and weights must be bit-identical -- on two calls
in a row, the second with a smaller batch, and after a shape too large for
the array has been refused."""

import numpy as np
import pytest

from tests.gpu_support import layer_of, say
from mixture_experts_layer_wave_amd import workloads as W

pytestmark = pytest.mark.gpu


def _run_both(L):
    import torch
    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import DeviceLayer

    D = DeviceLayer(L)
    D.forward()
    y_na = torch.full_like(D.y, -1)
    idx_na = torch.full_like(D.idx, -1)
    w_na = torch.full_like(D.topw, -1.0)
    B.moe_forward_noalloc(D.shape, D.x, D.act, D.wg, D.bias, D.weights, y_na, D.act, idx_na, w_na)
    torch.cuda.synchronize()
    assert torch.equal(D.y, y_na)
    assert torch.equal(D.idx, idx_na)
    assert torch.equal(D.topw.view(torch.int32), w_na.view(torch.int32))
    return D


@pytest.mark.parametrize("big,small", [(W.DECODE[2], W.DECODE[0]), ("mxfp4-gemm-ragged", "bf16-ragged")])
def test_noalloc_matches_forward_twice_then_smaller(big, small):
    say(f"[noalloc] {big} then {small}")
    _run_both(layer_of(big))
    _run_both(layer_of(small))


def test_noalloc_refuses_shapes_past_the_array():
    import torch
    from mixture_experts_layer_wave_amd import binding as B
    from mixture_experts_layer_wave_amd.device import DeviceLayer

    say("[noalloc] too large, then a valid call")
    L = layer_of(W.SWITCH)  # 4096 x 1024 bf16 with d_ff 4096: ~90 MB of workspace
    D = DeviceLayer(L)
    assert D.ws_bytes > (32 << 20)
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_noalloc(D.shape, D.x, D.act, D.wg, D.bias, D.weights, D.y, D.act, D.idx, D.topw)
    assert ei.value.status == -5
    # argument errors come first
    with pytest.raises(B.MoeError) as ei:
        B.moe_forward_noalloc(D.shape, None, D.act, D.wg, D.bias, D.weights, D.y, D.act, D.idx, D.topw)
    assert ei.value.status == -1
    torch.cuda.synchronize()
    _run_both(layer_of(W.DECODE[1]))
