"""ctypes binding of libmoe_mi355x.so (declared in include/moe.h).

Argument marshalling only: each function has the C entry point's name and
arguments, turns tensors into device pointers and the stream into a
hipStream_t, calls the library and raises :class:`MoeError` on a non-zero
status.  Every step of the layer runs in the library's HIP kernels; there is
no fallback.  Pointer arguments accept a torch tensor (its ``data_ptr()``),
a plain integer address, or None (NULL).  ``stream=None`` means torch's
current stream on the current device.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe_mi355x.so")

MOE_F32, MOE_BF16, MOE_MXFP4, MOE_MXFP8 = 0, 1, 2, 3
DTYPES = {"f32": MOE_F32, "bf16": MOE_BF16, "mxfp4": MOE_MXFP4, "mxfp8": MOE_MXFP8}

if not os.path.exists(LIB_PATH):
    raise ImportError(
        f"{LIB_PATH} is not built; run `python -m mixture_experts_layer_wave_amd.build` "
        "(the MoE layer has no non-HIP implementation)"
    )
lib = ctypes.CDLL(LIB_PATH)


class Shape(ctypes.Structure):
    _fields_ = [("n", ctypes.c_int32), ("d", ctypes.c_int32), ("E", ctypes.c_int32),
                ("k", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("renorm", ctypes.c_int32)]


class ExpertWeights(ctypes.Structure):
    # slot (device int32 [E]) / n_slots: logical -> physical expert slots;
    # left at NULL / 0, expert e is slot e.  act_quant: 0, or MOE_MXFP8 for
    # the W4A8 mode.
    _fields_ = [("dtype", ctypes.c_int32),
                ("w1", ctypes.c_void_p), ("w3", ctypes.c_void_p), ("w2", ctypes.c_void_p),
                ("s1", ctypes.c_void_p), ("s3", ctypes.c_void_p), ("s2", ctypes.c_void_p),
                ("slot", ctypes.c_void_p), ("n_slots", ctypes.c_int32),
                ("act_quant", ctypes.c_int32)]


class MoeError(RuntimeError):
    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn}: {lib.moe_status_string(status).decode()} (status {status})")


_P = ctypes.c_void_p
_I = ctypes.c_int
_SZ = ctypes.c_size_t
_SP = ctypes.POINTER(Shape)
_WP = ctypes.POINTER(ExpertWeights)

lib.moe_abi_version.restype = _I
lib.moe_abi_version.argtypes = []
lib.moe_status_string.restype = ctypes.c_char_p
lib.moe_status_string.argtypes = [_I]
lib.moe_workspace_bytes.restype = _SZ
lib.moe_workspace_bytes.argtypes = [_SP, _I]
lib.moe_mxfp8_bytes.restype = _SZ
lib.moe_mxfp8_bytes.argtypes = [ctypes.c_int64, ctypes.c_int32]
lib.moe_quantize_mxfp8.restype = _I
lib.moe_quantize_mxfp8.argtypes = [ctypes.c_int64, ctypes.c_int32, _P, _I, _P, _P]
lib.moe_router_topk.restype = _I
lib.moe_router_topk.argtypes = [_SP, _P, _I, _P, _P, _P, _P, _P, _P]
lib.moe_router_stats_workspace_bytes.restype = _SZ
lib.moe_router_stats_workspace_bytes.argtypes = [_SP]
lib.moe_router_stats.restype = _I
lib.moe_router_stats.argtypes = [_SP, _P, _P, ctypes.c_float, _P, _P, _P, _P, _SZ, _P]
lib.moe_active_experts.restype = _I
lib.moe_active_experts.argtypes = [_SP, _P, _P, _P, _P]
lib.moe_dispatch_workspace_bytes.restype = _SZ
lib.moe_dispatch_workspace_bytes.argtypes = [_SP]
lib.moe_dispatch.restype = _I
lib.moe_dispatch.argtypes = [_SP, _P, _P, _P, _P, _P, _P, _I, _P, _P, _SZ, _P]
lib.moe_grouped_ffn.restype = _I
lib.moe_grouped_ffn.argtypes = [_SP, _P, _I, _P, _WP, _P, _I, _P, _SZ, _P]
lib.moe_expert_up.restype = _I
lib.moe_expert_up.argtypes = [_SP, _P, _I, _P, _P, _WP, _P, _P]
lib.moe_expert_down.restype = _I
lib.moe_expert_down.argtypes = [_SP, _P, _P, _WP, _P, _P]
lib.moe_combine.restype = _I
lib.moe_combine.argtypes = [_SP, _P, _I, _P, _P, _P, _I, _P]
lib.moe_forward.restype = _I
lib.moe_forward.argtypes = [_SP, _P, _I, _P, _P, _WP, _P, _I, _P, _P, _P, _SZ, _P]
lib.moe_forward_noalloc.restype = _I
lib.moe_forward_noalloc.argtypes = [_SP, _P, _I, _P, _P, _WP, _P, _I, _P, _P, _P]

EXPORTS = ("moe_abi_version", "moe_status_string", "moe_workspace_bytes", "moe_mxfp8_bytes",
           "moe_quantize_mxfp8", "moe_router_topk",
           "moe_router_stats_workspace_bytes", "moe_router_stats", "moe_active_experts",
           "moe_dispatch_workspace_bytes", "moe_dispatch", "moe_grouped_ffn", "moe_expert_up", "moe_expert_down", "moe_combine",
           "moe_forward", "moe_forward_noalloc")


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch

        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


def _dt(d) -> int:
    return DTYPES[d] if isinstance(d, str) else int(d)


def _shape(s) -> Shape:
    if isinstance(s, Shape):
        return s
    return Shape(*s) if len(s) == 6 else Shape(*s, -1)


def _weights(w) -> ExpertWeights:
    if isinstance(w, ExpertWeights):
        return w
    aq = w.get("act_quant", 0)
    return ExpertWeights(_dt(w["dtype"]), _ptr(w["w1"]), _ptr(w["w3"]), _ptr(w["w2"]),
                         _ptr(w.get("s1")), _ptr(w.get("s3")), _ptr(w.get("s2")),
                         _ptr(w.get("slot")), int(w.get("n_slots", 0)), _dt(aq) if aq else 0)


def moe_abi_version() -> int:
    return lib.moe_abi_version()


def moe_status_string(status: int) -> str:
    return lib.moe_status_string(status).decode()


def moe_workspace_bytes(shape, w_dtype) -> int:
    return lib.moe_workspace_bytes(ctypes.byref(_shape(shape)), _dt(w_dtype))


def moe_mxfp8_bytes(rows, cols) -> int:
    return int(lib.moe_mxfp8_bytes(int(rows), int(cols)))


def moe_quantize_mxfp8(rows, cols, x, act, q, stream=None):
    _check("moe_quantize_mxfp8", lib.moe_quantize_mxfp8(
        int(rows), int(cols), _ptr(x), _dt(act), _ptr(q), _stream(stream)))


def moe_router_topk(shape, x, act, wg, bias, logits, topk_idx, topk_w, stream=None):
    _check("moe_router_topk", lib.moe_router_topk(
        ctypes.byref(_shape(shape)), _ptr(x), _dt(act), _ptr(wg), _ptr(bias), _ptr(logits),
        _ptr(topk_idx), _ptr(topk_w), _stream(stream)))


def moe_router_stats_workspace_bytes(shape) -> int:
    return int(lib.moe_router_stats_workspace_bytes(ctypes.byref(_shape(shape))))


def moe_router_stats(shape, logits, topk_idx, alpha, P, f, loss, ws, ws_bytes, stream=None):
    _check("moe_router_stats", lib.moe_router_stats(
        ctypes.byref(_shape(shape)), _ptr(logits), _ptr(topk_idx), float(alpha), _ptr(P), _ptr(f),
        _ptr(loss), _ptr(ws), int(ws_bytes), _stream(stream)))


def moe_dispatch_workspace_bytes(shape) -> int:
    return int(lib.moe_dispatch_workspace_bytes(ctypes.byref(_shape(shape))))


def moe_dispatch(shape, topk_idx, counts, offsets, perm, inv, x=None, act="bf16", x_perm=None,
                 ws=None, ws_bytes=0, stream=None):
    _check("moe_dispatch", lib.moe_dispatch(
        ctypes.byref(_shape(shape)), _ptr(topk_idx), _ptr(counts), _ptr(offsets), _ptr(perm),
        _ptr(inv), _ptr(x), _dt(act), _ptr(x_perm), _ptr(ws), ws_bytes, _stream(stream)))


def moe_active_experts(shape, counts, active, n_active, stream=None):
    _check("moe_active_experts", lib.moe_active_experts(
        ctypes.byref(_shape(shape)), _ptr(counts), _ptr(active), _ptr(n_active), _stream(stream)))


def moe_grouped_ffn(shape, x_perm, act, offsets, weights, y_perm, out, ws, ws_bytes, stream=None):
    w = _weights(weights)
    _check("moe_grouped_ffn", lib.moe_grouped_ffn(
        ctypes.byref(_shape(shape)), _ptr(x_perm), _dt(act), _ptr(offsets), ctypes.byref(w),
        _ptr(y_perm), _dt(out), _ptr(ws), ws_bytes, _stream(stream)))


def moe_expert_up(shape, a, act, perm, offsets, weights, h, stream=None):
    w = _weights(weights)
    _check("moe_expert_up", lib.moe_expert_up(
        ctypes.byref(_shape(shape)), _ptr(a), _dt(act), _ptr(perm), _ptr(offsets),
        ctypes.byref(w), _ptr(h), _stream(stream)))


def moe_expert_down(shape, h, offsets, weights, y_perm, stream=None):
    w = _weights(weights)
    _check("moe_expert_down", lib.moe_expert_down(
        ctypes.byref(_shape(shape)), _ptr(h), _ptr(offsets), ctypes.byref(w), _ptr(y_perm),
        _stream(stream)))


def moe_combine(shape, y_perm, in_dtype, inv, topk_w, y, out, stream=None):
    _check("moe_combine", lib.moe_combine(
        ctypes.byref(_shape(shape)), _ptr(y_perm), _dt(in_dtype), _ptr(inv), _ptr(topk_w),
        _ptr(y), _dt(out), _stream(stream)))


def moe_forward(shape, x, act, wg, bias, weights, y, out, topk_idx, topk_w, ws, ws_bytes,
                stream=None):
    w = _weights(weights)
    _check("moe_forward", lib.moe_forward(
        ctypes.byref(_shape(shape)), _ptr(x), _dt(act), _ptr(wg), _ptr(bias), ctypes.byref(w),
        _ptr(y), _dt(out), _ptr(topk_idx), _ptr(topk_w), _ptr(ws), ws_bytes, _stream(stream)))


def moe_forward_noalloc(shape, x, act, wg, bias, weights, y, out, topk_idx, topk_w, stream=None):
    w = _weights(weights)
    _check("moe_forward_noalloc", lib.moe_forward_noalloc(
        ctypes.byref(_shape(shape)), _ptr(x), _dt(act), _ptr(wg), _ptr(bias), ctypes.byref(w),
        _ptr(y), _dt(out), _ptr(topk_idx), _ptr(topk_w), _stream(stream)))
