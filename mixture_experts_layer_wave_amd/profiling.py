"""Summaries of rocprofv3 output for the files under profiles/.

    python -m mixture_experts_layer_wave_amd.profiling stats \
        --csv DIR/run_kernel_stats.csv --title T --command CMD --out profiles/X.md
    python -m mixture_experts_layer_wave_amd.profiling traffic --workload NAME \
        --kernel SUBSTRING --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \
        --copy-bytes N --command CMD --out profiles/Y.md

    python -m mixture_experts_layer_wave_amd.profiling mfma --workload NAME \
        --kernel SUBSTRING --pmc DIR --peak-tflops P --command CMD --out profiles/Z.md

`traffic` turns two counter runs (FETCH_SIZE, then WRITE_SIZE; rocprofv3
reports KiB per dispatch) into HBM bytes per launch of one kernel.  Each
counter is scaled by what it reads for a plain device copy of known size
(copy bytes / counter bytes), measured in the same way.  The summary records
a digest of the sources that define the kernel; bench.py reports the
traffic only while those sources are unchanged.

`mfma` reads one counter run (MFMA math ops, MFMA busy cycles and
GRBM_GUI_ACTIVE, with each dispatch's start and end time) and sets the
flops the matrix cores executed beside the kernel's algorithmic flops
(4 R d d_ff for the up projection: routed rows only), with the average
clock over the dispatch and the fraction of the peak at that clock.
"""

from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import os
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")

# Sources that define each profiled kernel family (relative to the package).
KERNEL_SOURCES = {
    "big_gemm_kernel": ["csrc/gemm_big.hip", "csrc/gemm_big.h", "csrc/gemm_common.h",
                        "csrc/common.h"],
    "mxw_gemm_kernel": ["csrc/gemm_mxw.hip", "csrc/gemm_mxw.h", "csrc/gemm_common.h",
                        "csrc/common.h"],
    "mxw16_mixed_kernel": ["csrc/gemm_mxw.hip", "csrc/gemm_mxw.h", "csrc/gemm_common.h",
                           "csrc/common.h"],
    "mxw16_pair_kernel": ["csrc/gemm_mxw.hip", "csrc/gemm_mxw.h", "csrc/gemm_common.h",
                          "csrc/common.h", "csrc/ffn.hip"],
    "mx_decode_kernel": ["csrc/decode.hip", "csrc/gemm_mxw.h", "csrc/common.h",
                         "csrc/route_dev.h"],
}


def family(kernel: str) -> str:
    for fam in KERNEL_SOURCES:
        if fam in kernel:
            return fam
    raise KeyError(f"no source list for kernel {kernel!r}")


def sources_digest(fam: str) -> str:
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[fam]:
        with open(os.path.join(PKG, rel), "rb") as f:
            h.update(rel.encode() + b"\0" + f.read())
    return h.hexdigest()


def _csv(path_or_dir: str, suffix: str) -> str:
    if os.path.isdir(path_or_dir):
        hits = sorted(glob.glob(os.path.join(path_or_dir, "**", f"*{suffix}"), recursive=True))
        if not hits:
            raise FileNotFoundError(f"no *{suffix} under {path_or_dir}")
        return hits[0]
    return path_or_dir


def short_name(name: str) -> str:
    name = name.replace("moe::(anonymous namespace)::", "").replace("void ", "")
    if name.endswith(")"):  # drop the parameter list (the last balanced group)
        depth = 0
        for i in range(len(name) - 1, -1, -1):
            depth += {")": 1, "(": -1}.get(name[i], 0)
            if depth == 0:
                name = name[:i]
                break
    return name


def kernel_stats(path: str):
    rows = list(csv.DictReader(open(_csv(path, "kernel_stats.csv"))))
    out = []
    for r in rows:
        out.append({"name": short_name(r["Name"]), "calls": int(r["Calls"]),
                    "avg_us": float(r["AverageNs"]) / 1e3, "total_us": float(r["TotalDurationNs"]) / 1e3,
                    "pct": float(r["Percentage"])})
    return out


def counter_means(path: str, counter: str):
    """Mean counter value per dispatch, per kernel name."""
    acc = defaultdict(list)
    for r in csv.DictReader(open(_csv(path, "counter_collection.csv"))):
        if r["Counter_Name"] == counter:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: (sum(v) / len(v), len(v)) for k, v in acc.items()}


def dispatch_counters(path: str, substring: str):
    """{counter: mean value per dispatch} and the mean dispatch time (ns) of
    the one kernel whose name contains substring."""
    acc, times, names = defaultdict(list), {}, set()
    for r in csv.DictReader(open(_csv(path, "counter_collection.csv"))):
        if substring not in r["Kernel_Name"]:
            continue
        names.add(r["Kernel_Name"])
        acc[r["Counter_Name"]].append(float(r["Counter_Value"]))
        times[r["Dispatch_Id"]] = int(r["End_Timestamp"]) - int(r["Start_Timestamp"])
    if len(names) != 1:
        raise ValueError(f"{len(names)} kernels match {substring!r}: {[short_name(k) for k in names]}")
    means = {k: sum(v) / len(v) for k, v in acc.items()}
    return names.pop(), means, sum(times.values()) / len(times), len(times)


def _pick(means, substring):
    hits = [(k, v) for k, v in means.items() if substring in k]
    if len(hits) != 1:
        raise ValueError(f"{len(hits)} kernels match {substring!r}: {[short_name(k) for k, _ in hits]}")
    return hits[0]


def cmd_stats(a):
    rows = kernel_stats(a.csv)
    lines = [f"# {a.title}", "", "Command:", "", "```", a.command, "```", "",
             "| kernel | calls | avg us | total us | % |", "|---|---:|---:|---:|---:|"]
    for r in rows[: a.top]:
        lines.append(f"| `{r['name']}` | {r['calls']} | {r['avg_us']:.2f} | {r['total_us']:.1f} | {r['pct']:.1f} |")
    if a.note:
        lines += ["", a.note]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {a.out}")


def cmd_traffic(a):
    copy_kib_f = max(v for v, _ in counter_means(a.copy_fetch, "FETCH_SIZE").values())
    copy_kib_w = max(v for v, _ in counter_means(a.copy_write, "WRITE_SIZE").values())
    f_scale = a.copy_bytes / (copy_kib_f * 1024.0)
    w_scale = a.copy_bytes / (copy_kib_w * 1024.0)
    kname, (fetch_kib, nf) = _pick(counter_means(a.fetch, "FETCH_SIZE"), a.kernel)
    _, (write_kib, nw) = _pick(counter_means(a.write, "WRITE_SIZE"), a.kernel)
    fetch_b = fetch_kib * 1024.0 * f_scale
    write_b = write_kib * 1024.0 * w_scale
    fam = family(kname)
    lines = [
        f"# HBM traffic of `{short_name(kname)}` ({a.workload})", "",
        "Commands (counters in separate passes, then this summary):", "", "```", a.command, "```", "",
        "| quantity | value |", "|---|---:|",
        f"| copy calibration: bytes copied | {a.copy_bytes} |",
        f"| copy FETCH_SIZE (KiB) | {copy_kib_f:.1f} |",
        f"| copy WRITE_SIZE (KiB) | {copy_kib_w:.1f} |",
        f"| FETCH scale (bytes per counted byte) | {f_scale:.4f} |",
        f"| WRITE scale (bytes per counted byte) | {w_scale:.4f} |",
        f"| kernel FETCH_SIZE per dispatch (KiB, mean of {nf}) | {fetch_kib:.1f} |",
        f"| kernel WRITE_SIZE per dispatch (KiB, mean of {nw}) | {write_kib:.1f} |",
        f"| HBM bytes read per launch (scaled) | {fetch_b:.0f} |",
        f"| HBM bytes written per launch (scaled) | {write_b:.0f} |",
        "",
        f"workload: {a.workload}",
        f"act_quant: {a.act_quant or 'none'}",
        f"kernel: {short_name(kname)}",
        f"traffic_bytes_per_launch: {fetch_b + write_b:.0f}",
        f"sources_sha256: {sources_digest(fam)}",
    ]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {a.out}: {fetch_b + write_b:.0f} bytes per launch")


# MI355X: 8 XCDs, 256 CUs of 4 SIMDs; spec clock 2.4 GHz.
N_XCD, N_SIMD, SPEC_GHZ = 8, 1024, 2.4


def up_flops(workload: str) -> float:
    from mixture_experts_layer_wave_amd import workloads as W
    wl = W.WORKLOADS[workload]
    return 4.0 * wl.n * wl.k * wl.d * wl.d_ff


def projection_flops(workload: str, kernel: str) -> float:
    """Algorithmic flops of one launch of an expert GEMM: the up projection
    (W1 and W3, first template argument true) or the down projection (W2,
    half the up projection's)."""
    up = short_name(kernel).split("<", 1)[1].startswith("true")
    return up_flops(workload) if up else up_flops(workload) / 2.0


def cmd_mfma(a):
    kname, c, dur_ns, nd = dispatch_counters(a.pmc, a.kernel)
    mops = sum(v for k, v in c.items() if k.startswith("SQ_INSTS_VALU_MFMA_MOPS_"))
    counted = mops * 512.0
    alg = projection_flops(a.workload, kname) if a.flops is None else a.flops
    # GRBM_GUI_ACTIVE is summed over the XCDs: cycles of one XCD = sum / 8.
    cycles = c["GRBM_GUI_ACTIVE"] / N_XCD
    ghz = cycles / dur_ns
    busy = c["SQ_VALU_MFMA_BUSY_CYCLES"] / (cycles * N_SIMD)
    achieved = alg / (dur_ns * 1e-9) / 1e12
    peak_clk = a.peak_tflops * ghz / SPEC_GHZ
    rows = [("dispatches averaged", f"{nd}"),
            ("dispatch duration (us)", f"{dur_ns / 1e3:.1f}"),
            ("algorithmic flops per launch", f"{alg:.4e}"),
            ("MFMA flops counted (MOPS x 512)", f"{counted:.4e}"),
            ("counted / algorithmic", f"{counted / alg:.3f}"),
            ("achieved (algorithmic, TFLOP/s)", f"{achieved:.1f}"),
            ("fraction of the spec peak", f"{achieved / a.peak_tflops:.3f}"),
            ("average clock (GRBM_GUI_ACTIVE / duration, GHz)", f"{ghz:.3f}"),
            ("peak at that clock (TFLOP/s)", f"{peak_clk:.1f}"),
            ("fraction of the peak at that clock", f"{achieved / peak_clk:.3f}"),
            ("MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs))", f"{busy:.3f}")]
    rows += [(f"{k} (per dispatch)", f"{v:.4e}") for k, v in sorted(c.items())]
    lines = [f"# MFMA counters of `{short_name(kname)}` ({a.workload})", "",
             "Commands (one counter pass, then this summary):", "", "```", a.command, "```", "",
             "| quantity | value |", "|---|---:|"] + [f"| {k} | {v} |" for k, v in rows]
    lines += ["", f"workload: {a.workload}", f"act_quant: {a.act_quant or 'none'}",
              f"kernel: {short_name(kname)}", f"spec_peak_tflops: {a.peak_tflops}",
              f"sources_sha256: {sources_digest(family(kname))}"]
    open(a.out, "w").write("\n".join(lines) + "\n")
    print(f"wrote {a.out}: {achieved:.0f} TFLOP/s, clock {ghz:.2f} GHz, MFMA busy {busy:.3f}, "
          f"counted/alg {counted / alg:.3f}")


def read_traffic(workload: str, kernel_family: str, act_quant: str | None = None, up: bool = True):
    """(bytes per launch, path) of the up (or down) kernel of the family from
    profiles/ if its sources digest still matches the current sources of the
    kernel, else (None, reason).  Every kernel family takes UP as its first
    template argument, so the up kernel is `family<true`."""
    want = f"{kernel_family}<{'true' if up else 'false'}"
    for path in sorted(glob.glob(os.path.join(PROFILES, "*traffic*.md"))):
        kv = {}
        for line in open(path):
            if ":" in line and not line.startswith(("|", "#", " ")):
                k, _, v = line.partition(":")
                kv[k.strip()] = v.strip()
        if kv.get("workload") != workload or not kv.get("kernel", "").startswith(want):
            continue
        if kv.get("act_quant", "none") != (act_quant or "none"):
            continue
        if kv.get("sources_sha256") != sources_digest(kernel_family):
            return None, f"{os.path.relpath(path, ROOT)}: kernel sources changed since measured"
        return float(kv["traffic_bytes_per_launch"]), os.path.relpath(path, ROOT)
    return None, "no traffic profile for this workload"


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--csv", required=True)
    s.add_argument("--title", required=True)
    s.add_argument("--command", required=True)
    s.add_argument("--out", required=True)
    s.add_argument("--top", type=int, default=12)
    s.add_argument("--note", default="")
    t = sub.add_parser("traffic")
    for k in ("workload", "kernel", "fetch", "write", "copy_fetch", "copy_write", "command", "out"):
        t.add_argument("--" + k.replace("_", "-"), required=True)
    t.add_argument("--copy-bytes", type=int, required=True)
    t.add_argument("--act-quant", default=None)
    m = sub.add_parser("mfma")
    for k in ("workload", "kernel", "pmc", "command", "out"):
        m.add_argument("--" + k, required=True)
    m.add_argument("--peak-tflops", type=float, required=True)
    m.add_argument("--flops", type=float, default=None)
    m.add_argument("--act-quant", default=None)
    a = ap.parse_args()
    {"stats": cmd_stats, "traffic": cmd_traffic, "mfma": cmd_mfma}[a.cmd](a)


if __name__ == "__main__":
    main()
