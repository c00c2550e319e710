"""Seeded synthetic inputs for the MoE layer (shared by tests and bench).

This module only draws random numbers and encodes them into the stored
formats (bfloat16 bits, float32, MXFP4 bytes).  It holds none of the layer's
arithmetic: no router, softmax, selection, dispatch, expert or combine
step.  The two inputs that depend on routing -- which tokens must be
redrawn so that every top-k decision has a clear margin, and the router bias
that skews expert load -- are read from ``tests/golden/routing_fixtures.json``
(written by ``tests/golden/make_routing_fixtures.py`` from the float64
oracle) or passed in by the caller.

Recipe (stated once more in the design notes):

* every array comes from its own PCG64 stream,
  ``SeedSequence(seed, spawn_key=(tag, index...))``;
* X ~ N(0, 1); router and expert weights ~ N(0, 1) / sqrt(fan_in) with
  fan_in = d for W_g, W1, W3 and d_ff for W2; draws are float32 and are then
  rounded to bfloat16 (round to nearest even) or kept as float32;
* MXFP4 weights: the float32 draw of each 32-element block along K gets the
  shared exponent s = clamp(floor(log2(amax)) - 2 + 127, 1, 254) (E2M1's
  largest exponent is 2), each element is scaled by 2^-(s-127) and rounded to
  the nearest E2M1 magnitude {0, .5, 1, 1.5, 2, 3, 4, 6} (saturating; a value
  exactly half-way goes to the smaller magnitude) with its sign in bit 3;
  two codes per byte, the even K index in the low nibble;
* a redrawn token t (r-th redraw) takes its row from stream
  ``(seed, spawn_key=(REDRAW, t, r))``.
"""

from __future__ import annotations

import json
import math
import os
import threading
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, replace

import numpy as np

REPO_ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ROUTING_FIXTURES = os.path.join(REPO_ROOT, "tests", "golden", "routing_fixtures.json")

# stream tags
_X, _WG, _W1, _W3, _W2, _REDRAW = 1, 2, 3, 4, 5, 6


@dataclass(frozen=True)
class Workload:
    """Shape, formats and seeds of one synthetic MoE layer + batch."""

    name: str
    n: int          # tokens
    d: int          # model width
    E: int          # experts
    k: int          # experts per token
    d_ff: int       # expert hidden width
    act: str        # 'f32' | 'bf16' (X, W_g, output)
    wdt: str        # 'f32' | 'bf16' | 'mxfp4' (expert weights)
    layer_seed: int  # weights (W_g, W1, W3, W2)
    x_seed: int      # tokens
    zipf_s: float = 0.0  # > 0: router bias skews load toward Zipf(s)

    @property
    def renorm(self) -> bool:
        return self.k > 1

    @property
    def R(self) -> int:
        return self.n * self.k


def _wl(name, n, d, E, k, d_ff, act, wdt, layer_seed, x_seed, zipf_s=0.0):
    return Workload(name, n, d, E, k, d_ff, act, wdt, layer_seed, x_seed, zipf_s)


# The five workloads: a tiny float32 layer the size of the page's worked
# example, a Switch-style top-1 layer, a Mixtral-shaped top-2 layer, and a
# 128-expert top-4 MXFP4 layer (gpt-oss-120b's expert count, top-k and
# weight format) at decode and at prefill with a Zipf-skewed router.
WORKLOADS = {
    w.name: w
    for w in (
        _wl("tiny-f32-n6-d3-e4-top1", 6, 3, 4, 1, 12, "f32", "f32", 1000, 1000),
        _wl("switch-top1-n4096-d1024-e8-ff4096-bf16", 4096, 1024, 8, 1, 4096, "bf16", "bf16", 1001, 1001),
        _wl("mixtral-top2-n8192-d4096-e8-ff14336-bf16", 8192, 4096, 8, 2, 14336, "bf16", "bf16", 1002, 1002),
        _wl("e128-top4-mxfp4-decode-n1", 1, 2880, 128, 4, 2880, "bf16", "mxfp4", 1003, 2001),
        _wl("e128-top4-mxfp4-decode-n8", 8, 2880, 128, 4, 2880, "bf16", "mxfp4", 1003, 2008),
        _wl("e128-top4-mxfp4-decode-n64", 64, 2880, 128, 4, 2880, "bf16", "mxfp4", 1003, 2064),
        _wl("e128-top4-mxfp4-prefill-zipf-n4096", 4096, 2880, 128, 4, 2880, "bf16", "mxfp4", 1003, 2409, 1.1),
    )
}

TINY = "tiny-f32-n6-d3-e4-top1"
SWITCH = "switch-top1-n4096-d1024-e8-ff4096-bf16"
MIXTRAL = "mixtral-top2-n8192-d4096-e8-ff14336-bf16"
DECODE = ("e128-top4-mxfp4-decode-n1", "e128-top4-mxfp4-decode-n8", "e128-top4-mxfp4-decode-n64")
PREFILL_ZIPF = "e128-top4-mxfp4-prefill-zipf-n4096"


def scaled(base: Workload, name: str, **kw) -> Workload:
    """A smaller (or otherwise altered) variant of a workload."""
    return replace(base, name=name, **kw)


# ---------------------------------------------------------------------------
# Encoders (input generation only).
# ---------------------------------------------------------------------------


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round to nearest even (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    return ((u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)).astype(np.uint16)


_E2M1_MIDS = np.array([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0], dtype=np.float32)


def mxfp4_encode(w: np.ndarray) -> tuple[np.ndarray, np.ndarray]:
    """float32 [N][K] -> (packed codes [N][K/2] uint8, e8m0 scales [N][K/32])."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    if K % 32:
        raise ValueError("MXFP4 needs K % 32 == 0")
    blk = w.reshape(N, K // 32, 32)
    amax = np.abs(blk).max(axis=2)
    with np.errstate(divide="ignore"):
        ex = np.floor(np.log2(amax))
    ex = np.where(np.isfinite(ex), ex, -127.0)
    s = np.clip(ex - 2.0 + 127.0, 1, 254).astype(np.int32)
    inv_scale = np.ldexp(np.float32(1.0), (127 - s)).astype(np.float32)
    v = blk * inv_scale[:, :, None]
    mag = np.abs(v)
    code = np.zeros(v.shape, dtype=np.uint8)
    tmp = np.empty(v.shape, dtype=bool)
    for mid in _E2M1_MIDS:
        np.greater(mag, mid, out=tmp)
        code += tmp
    np.less(v, 0, out=tmp)
    code |= tmp.astype(np.uint8) << 3
    code = code.reshape(N, K)
    packed = (code[:, 0::2] | (code[:, 1::2] << 4)).astype(np.uint8)
    return packed, s.astype(np.uint8)


# ---------------------------------------------------------------------------
# Draws
# ---------------------------------------------------------------------------


def _rng(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def _normal(seed: int, key: tuple, shape, scale: float = 1.0) -> np.ndarray:
    out = np.empty(shape, dtype=np.float32)
    _rng(seed, *key).standard_normal(out=out, dtype=np.float32)
    if scale != 1.0:
        out *= np.float32(scale)
    return out


def _encode_act(a: np.ndarray, act: str) -> np.ndarray:
    return a if act == "f32" else bf16_bits(a)


def draw_x(wl: Workload, redraws: dict | None = None) -> np.ndarray:
    """Token matrix X [n][d] (stored dtype), with per-token redraws applied."""
    x = _normal(wl.x_seed, (_X,), (wl.n, wl.d))
    for t, r in (redraws or {}).items():
        x[int(t)] = _normal(wl.x_seed, (_REDRAW, int(t), int(r)), (wl.d,))
    return _encode_act(x, wl.act)


def draw_router(wl: Workload) -> np.ndarray:
    """W_g stored as [E][d] (stored dtype), N(0,1)/sqrt(d)."""
    return _encode_act(_normal(wl.layer_seed, (_WG,), (wl.E, wl.d), 1.0 / math.sqrt(wl.d)), wl.act)


_tls = threading.local()


def _expert_matrix(wl: Workload, tag: int, e: int):
    N, K = (wl.d_ff, wl.d) if tag in (_W1, _W3) else (wl.d, wl.d_ff)
    w = _normal(wl.layer_seed, (tag, e), (N, K), 1.0 / math.sqrt(K))
    if wl.wdt == "mxfp4":
        return mxfp4_encode(w)
    if wl.wdt == "bf16":
        return bf16_bits(w), None
    return w, None


def draw_experts(wl: Workload, threads: int | None = None) -> dict:
    """W1, W3 [E][d_ff][d] and W2 [E][d][d_ff] (+ MXFP4 scales)."""
    E, d, f = wl.E, wl.d, wl.d_ff
    if wl.wdt == "mxfp4":
        w1 = np.empty((E, f, d // 2), np.uint8)
        w3 = np.empty((E, f, d // 2), np.uint8)
        w2 = np.empty((E, d, f // 2), np.uint8)
        s1 = np.empty((E, f, d // 32), np.uint8)
        s3 = np.empty((E, f, d // 32), np.uint8)
        s2 = np.empty((E, d, f // 32), np.uint8)
    else:
        dt = np.uint16 if wl.wdt == "bf16" else np.float32
        w1 = np.empty((E, f, d), dt)
        w3 = np.empty((E, f, d), dt)
        w2 = np.empty((E, d, f), dt)
        s1 = s3 = s2 = None
    outs = {_W1: (w1, s1), _W3: (w3, s3), _W2: (w2, s2)}

    def job(te):
        tag, e = te
        v, s = _expert_matrix(wl, tag, e)
        outs[tag][0][e] = v
        if s is not None:
            outs[tag][1][e] = s

    tasks = [(tag, e) for e in range(E) for tag in (_W1, _W3, _W2)]
    nthr = threads or min(16, os.cpu_count() or 1)
    if nthr <= 1 or len(tasks) == 1:
        for t in tasks:
            job(t)
    else:
        with ThreadPoolExecutor(nthr) as ex:
            list(ex.map(job, tasks))
    return {"w1": w1, "w3": w3, "w2": w2, "s1": s1, "s3": s3, "s2": s2}


def zipf_targets(wl: Workload) -> np.ndarray:
    """Target rows per expert for a Zipf(s) load: rank r gets R r^-s / H.

    Ranks are assigned to experts by a seeded permutation.
    """
    r = np.arange(1, wl.E + 1, dtype=np.float64)
    share = r ** (-wl.zipf_s)
    share /= share.sum()
    perm = _rng(wl.layer_seed, 99).permutation(wl.E)
    tgt = np.empty(wl.E)
    tgt[perm] = wl.R * share
    return tgt


# ---------------------------------------------------------------------------
# Routing fixtures (redraw maps and the Zipf bias) produced by the oracle.
# ---------------------------------------------------------------------------

_fixture_cache: dict | None = None


def routing_fixture(name: str) -> dict:
    """{'redraws': {token: count}, 'bias_f32_hex': [...] or None} for a workload."""
    global _fixture_cache
    if _fixture_cache is None:
        if os.path.exists(ROUTING_FIXTURES):
            with open(ROUTING_FIXTURES) as f:
                _fixture_cache = json.load(f)
        else:
            _fixture_cache = {}
    return _fixture_cache.get(name, {})


def bias_from_hex(hexes) -> np.ndarray:
    return np.array([int(h, 16) for h in hexes], dtype=np.uint32).view(np.float32)


_layer_cache: dict = {}


def make_layer(wl: Workload | str, redraws: dict | None = None, bias: np.ndarray | None = None,
               use_fixture: bool = True, cache: bool = True) -> dict:
    """All stored arrays of one workload, in the layout the oracle and the
    library read: x, x_dtype, wg, bias, w1, w3, w2, w_dtype, s1, s3, s2,
    plus n, d, E, k, d_ff, renorm, name."""
    if isinstance(wl, str):
        wl = WORKLOADS[wl]
    fx = routing_fixture(wl.name) if use_fixture else {}
    if redraws is None:
        redraws = fx.get("redraws", {})
    if bias is None and fx.get("bias_f32_hex") is not None:
        bias = bias_from_hex(fx["bias_f32_hex"])
    key = (wl.layer_seed, wl.E, wl.d, wl.d_ff, wl.wdt, wl.act)
    if cache and key in _layer_cache:
        wts = _layer_cache[key]
    else:
        wts = {"wg": draw_router(wl), **draw_experts(wl)}
        if cache:
            _layer_cache[key] = wts
    return {
        "name": wl.name, "n": wl.n, "d": wl.d, "E": wl.E, "k": wl.k, "d_ff": wl.d_ff,
        "renorm": wl.renorm,
        "x": draw_x(wl, redraws), "x_dtype": wl.act,
        "bias": None if bias is None else np.asarray(bias, dtype=np.float32),
        "w_dtype": wl.wdt, **wts,
    }
