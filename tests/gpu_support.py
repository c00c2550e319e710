"""Shared helpers of the GPU parity tests (imported by tests/test_gpu_*.py)."""

from __future__ import annotations

import functools
import sys

import numpy as np

import oracle
from mixture_experts_layer_wave_amd import workloads as W
from tests.golden import make_routing_fixtures as RF

# Output tolerances, as max over tokens of the row-normalised infinity norm
# of the error: |y - y_ref|_inf / |y_ref|_inf per token.
TOL = {"bf16": 2e-2, "mxfp4": 2e-2, "f32": 1e-5}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def row_rel_err(y: np.ndarray, ref: np.ndarray) -> float:
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return float((np.abs(y - ref).max(axis=1) / den).max())


def small(name, n, d, E, k, d_ff, wdt, seed, act="bf16", zipf_s=0.0) -> W.Workload:
    return W.Workload(name, n, d, E, k, d_ff, act, wdt, seed, seed + 1, zipf_s)


# Small and edge-case layers: several tiles, ragged tails, degenerate cases.
SMALL = {
    "bf16-ragged": small("bf16-ragged", 300, 136, 5, 2, 200, "bf16", 11),
    "mxfp4-ragged": small("mxfp4-ragged", 260, 96, 7, 3, 160, "mxfp4", 12),
    "bf16-e1": small("bf16-e1", 70, 64, 1, 1, 72, "bf16", 13),
    "bf16-k-eq-e": small("bf16-k-eq-e", 50, 64, 6, 6, 64, "bf16", 14),
    "bf16-e1024-k32": small("bf16-e1024-k32", 40, 64, 1024, 32, 32, "bf16", 15),
    "mxfp4-n1": small("mxfp4-n1", 1, 128, 16, 4, 96, "mxfp4", 16),
    # more than 1024 routed rows: the prefill GEMM with MXFP4 codes in LDS;
    # K tails in both projections (320 and 448 are not multiples of 128)
    "mxfp4-gemm-ragged": small("mxfp4-gemm-ragged", 700, 320, 8, 2, 448, "mxfp4", 18),
    # piles of about 25 rows on the GEMM path (the 64-row tile shape)
    "mxfp4-gemm-small-piles": small("mxfp4-gemm-small-piles", 600, 192, 48, 2, 320, "mxfp4", 19),
    "f32-small": small("f32-small", 33, 12, 5, 2, 20, "f32", 17, act="f32"),
    # top-k and dispatch in one workgroup: one pass of 4 tokens x 64 lanes,
    # and the 16-slot top-k instance (1024 experts, top-32) at n = 1
    "mxfp4-n4-e128": small("mxfp4-n4-e128", 4, 128, 128, 4, 96, "mxfp4", 20),
    "bf16-n1-e1024-k32": small("bf16-n1-e1024-k32", 1, 64, 1024, 32, 32, "bf16", 21),
    # MXFP4 with K past what the GEMM with codes in LDS keeps (7168) and more
    # than 1024 routed rows: the large-tile GEMM dequantising the codes in
    # registers, on the up projection (K = d) and on the down (K = d_ff)
    "mxfp4-wide-d": small("mxfp4-wide-d", 600, 7232, 4, 2, 96, "mxfp4", 22),
    "mxfp4-wide-ff": small("mxfp4-wide-ff", 600, 128, 4, 2, 7232, "mxfp4", 23),
    # more than two rounds of down blocks whose last row tiles fill at most
    # half of the chip: the down pass splits those tiles along K
    "bf16-tail-split": small("bf16-tail-split", 42000, 512, 2, 2, 256, "bf16", 24),
}


@functools.lru_cache(maxsize=None)
def layer_of(name: str) -> dict:
    """Stored arrays of a named workload (fixture redraws applied); layers
    sharing weights (the 128-expert decode and prefill batches) share them."""
    if name in W.WORKLOADS:
        return W.make_layer(name, cache=True)
    wl = SMALL[name]
    red = RF.find_redraws(wl)
    return W.make_layer(wl, redraws=red, use_fixture=False, cache=False)


def oracle_routing(layer: dict) -> dict:
    """Oracle logits, idx, weights and dispatch for every token."""
    x = oracle.decode_matrix(layer["x"], layer["x_dtype"])
    wg = oracle.decode_matrix(layer["wg"], layer["x_dtype"])
    bias = layer.get("bias")
    z = oracle.router_logits(x, wg, None if bias is None else oracle.decode_f32(bias))
    p = oracle.softmax_rows(z)
    idx = oracle.topk_select(z, layer["k"])
    w = oracle.topk_weights(p, idx, layer["renorm"])
    dp = oracle.dispatch(idx, layer["E"])
    return {"z": z, "p": p, "idx": idx, "w": w, **dp}


def sample_rows(n: int, idx: np.ndarray, counts: np.ndarray, m: int = 40) -> np.ndarray:
    """Deterministic token sample: first, last, spread, and tokens of the
    smallest non-empty piles."""
    rng = np.random.default_rng(n)
    rows = {0, n - 1}
    rows.update(rng.choice(n, size=min(n, m), replace=False).tolist())
    nz = np.nonzero(counts)[0]
    for e in nz[np.argsort(counts[nz])][:4]:
        t = np.nonzero((idx == e).any(axis=1))[0]
        rows.add(int(t[0]))
    return np.array(sorted(rows))


def pile_rows(lo: int, hi: int, e: int, step: int = 32) -> np.ndarray:
    """Rows of the pile [lo, hi) that touch every `step`-row group of it:
    the first and last row, plus one row of each group at a phase that
    varies from group to group.  Row tiles start at a pile's first row and
    are multiples of 32 rows, so with step = 32 every 32-row MFMA group of
    every row tile of the pile is compared (all output columns of a row)."""
    m = hi - lo
    if m <= 0:
        return np.zeros(0, dtype=np.int64)
    rows = {lo, hi - 1}
    for j in range((m + step - 1) // step):
        r = lo + j * step + (j * 13 + e * 7) % step
        rows.add(min(r, hi - 1))
    return np.array(sorted(rows), dtype=np.int64)


def pile_tokens(offsets: np.ndarray, perm: np.ndarray, step: int = 32) -> np.ndarray:
    """Tokens behind pile_rows of every pile (deduplicated, ascending)."""
    E = len(offsets) - 1
    rows = [pile_rows(int(offsets[e]), int(offsets[e + 1]), e, step) for e in range(E)]
    rows = np.concatenate(rows) if rows else np.zeros(0, dtype=np.int64)
    return np.unique(np.asarray(perm)[rows])
