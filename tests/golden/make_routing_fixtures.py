"""Write tests/golden/routing_fixtures.json from the float64 oracle.

Two inputs of the synthetic workloads depend on routing, and both are found
here with the oracle only (nothing from the HIP library):

* margins -- every token's top-(k+1) float64 logits (bias included) must be
  separated by at least 1e-4, so that the float32 kernels and the float64
  oracle choose the same experts in the same order.  Tokens that fail are
  redrawn from their own stream until all pass; the redraw counts are stored.
* Zipf skew -- the prefill workload adds a per-expert router bias so that
  expert load follows Zipf(1.1).  It is calibrated by the fixed-point
  iteration b_e += 0.5 (ln target_e - ln max(load_e, 0.5)) on float64
  routing until the L1 load error is below 5% of the routed rows, then
  frozen as float32 (stored as hex bit patterns).

Run:  python tests/golden/make_routing_fixtures.py
"""

from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

import oracle  # noqa: E402
from mixture_experts_layer_wave_amd import workloads as W  # noqa: E402

MARGIN = 1e-4


def logits64(wl: W.Workload, redraws: dict, bias) -> np.ndarray:
    x = oracle.decode_matrix(W.draw_x(wl, redraws), wl.act)
    wg = oracle.decode_matrix(W.draw_router(wl), wl.act)
    return oracle.router_logits(x, wg, None if bias is None else oracle.decode_f32(bias))


def margin_violations(z: np.ndarray, k: int, margin: float = MARGIN) -> np.ndarray:
    """Tokens whose top-(k+1) sorted logits have an adjacent gap < margin."""
    top = -np.sort(-z, axis=1)[:, : min(k + 1, z.shape[1])]
    gaps = top[:, :-1] - top[:, 1:]
    if gaps.shape[1] == 0:
        return np.zeros(0, dtype=np.int64)
    return np.nonzero((gaps < margin).any(axis=1))[0]


def find_redraws(wl: W.Workload, bias=None, max_rounds: int = 50) -> dict:
    redraws: dict[int, int] = {}
    for _ in range(max_rounds):
        bad = margin_violations(logits64(wl, redraws, bias), wl.k)
        if bad.size == 0:
            return redraws
        for t in bad.tolist():
            redraws[t] = redraws.get(t, 0) + 1
    raise RuntimeError(f"{wl.name}: margins not reached after {max_rounds} rounds")


def calibrate_zipf_bias(wl: W.Workload, tol: float = 0.05, max_iter: int = 500) -> np.ndarray:
    x = oracle.decode_matrix(W.draw_x(wl, {}), wl.act)
    wg = oracle.decode_matrix(W.draw_router(wl), wl.act)
    z0 = oracle.router_logits(x, wg, None)
    tgt = W.zipf_targets(wl)
    b = np.zeros(wl.E)
    for _ in range(max_iter):
        idx = oracle.topk_select(z0 + b[None, :], wl.k)
        load = np.bincount(idx.reshape(-1), minlength=wl.E).astype(np.float64)
        if np.abs(load - tgt).sum() < tol * wl.R:
            return b.astype(np.float32)
        b += 0.5 * (np.log(tgt) - np.log(np.maximum(load, 0.5)))
    raise RuntimeError("Zipf bias calibration did not converge")


def bias_hex(b: np.ndarray) -> list:
    return [f"{v:08x}" for v in np.asarray(b, np.float32).view(np.uint32).tolist()]


def main():
    out = {}
    for name, wl in W.WORKLOADS.items():
        bias = calibrate_zipf_bias(wl) if wl.zipf_s > 0 else None
        red = find_redraws(wl, bias)
        out[name] = {
            "redraws": {str(t): c for t, c in sorted(red.items())},
            "bias_f32_hex": None if bias is None else bias_hex(bias),
        }
        print(name, "redrawn tokens:", len(red), "bias:", bias is not None, flush=True)
    out["_about"] = (
        "Written by tests/golden/make_routing_fixtures.py from the float64 oracle: "
        "per-workload token redraw counts enforcing top-(k+1) logit margins >= 1e-4, "
        "and the float32 router bias giving Zipf(1.1) expert load on the prefill workload."
    )
    with open(os.path.join(HERE, "routing_fixtures.json"), "w") as f:
        json.dump(out, f, indent=1, sort_keys=True)


if __name__ == "__main__":
    main()
