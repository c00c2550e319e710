"""Device-side holder of one MoE layer for the C ABI (marshalling only).

Uploads the stored arrays of a layer (as produced by
:func:`mixture_experts_layer_wave_amd.workloads.make_layer`) to device
memory, sizes the workspace with ``moe_workspace_bytes`` and calls the
library's entry points.  torch provides device memory and streams only.
"""

from __future__ import annotations

import numpy as np
import torch

from . import binding as B


def to_device(a, device="cuda"):
    """numpy array -> device tensor with the same bytes (bf16 bits as int16)."""
    if a is None:
        return None
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def bf16_tensor_to_f64(t: torch.Tensor) -> np.ndarray:
    """int16 tensor of bf16 bit patterns -> float64 numpy (via torch's bf16)."""
    return t.view(torch.bfloat16).to(torch.float64).cpu().numpy()


class DeviceLayer:
    """One layer's inputs in HBM plus the output and workspace buffers."""

    def __init__(self, layer: dict, device: str = "cuda", renorm: int | None = None,
                 act_quant: str | None = None):
        self.layer = layer
        self.device = device
        self.n, self.d, self.E, self.k, self.d_ff = (layer[key] for key in ("n", "d", "E", "k", "d_ff"))
        self.act = layer["x_dtype"]
        self.wdt = layer["w_dtype"]
        rn = (1 if layer["renorm"] else 0) if renorm is None else renorm
        self.shape = B.Shape(self.n, self.d, self.E, self.k, self.d_ff, rn)
        self.x = to_device(layer["x"], device)
        self.wg = to_device(layer["wg"], device)
        self.bias = to_device(layer.get("bias"), device)
        self.w = {key: to_device(layer.get(key), device) for key in ("w1", "w3", "w2", "s1", "s3", "s2")}
        self.act_quant = act_quant
        self.weights = B.ExpertWeights(B.DTYPES[self.wdt], *(B._ptr(self.w[key]) for key in ("w1", "w3", "w2", "s1", "s3", "s2")),
                                       None, 0, B.DTYPES[act_quant] if act_quant else 0)
        self.ws_bytes = B.moe_workspace_bytes(self.shape, self.wdt)
        self.ws = torch.empty(self.ws_bytes, dtype=torch.uint8, device=device)
        ydt = torch.int16 if self.act == "bf16" else torch.float32
        self.y = torch.empty((self.n, self.d), dtype=ydt, device=device)
        self.idx = torch.empty((self.n, self.k), dtype=torch.int32, device=device)
        self.topw = torch.empty((self.n, self.k), dtype=torch.float32, device=device)

    def forward(self, stream=None, out: str | None = None, y=None):
        B.moe_forward(self.shape, self.x, self.act, self.wg, self.bias, self.weights,
                      self.y if y is None else y, out or self.act, self.idx, self.topw,
                      self.ws, self.ws_bytes, stream)
        return self.y if y is None else y

    def y_f64(self, y=None) -> np.ndarray:
        y = self.y if y is None else y
        if y.dtype == torch.int16:
            return bf16_tensor_to_f64(y)
        return y.to(torch.float64).cpu().numpy()
