"""Host-side checks of the rocprofv3 summary helpers used by bench.py."""

import os

from mixture_experts_layer_wave_amd import profiling as P


def test_short_name_drops_parameters_and_namespace():
    raw = "void moe::(anonymous namespace)::big_gemm_kernel<true, false, 256, 256>(moe::BigGemmParams)"
    assert P.short_name(raw) == "big_gemm_kernel<true, false, 256, 256>"
    assert P.short_name("__amd_rocclr_copyBuffer") == "__amd_rocclr_copyBuffer"


def test_read_traffic_follows_the_kernel_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(P, "PROFILES", str(tmp_path))
    fam = "mx_decode_kernel"
    good = P.sources_digest(fam)
    body = "# x\n\n| a | b |\n\nworkload: w1\nkernel: mx_decode_kernel<true, 6>\n"
    (tmp_path / "a_traffic_w1.md").write_text(body + f"traffic_bytes_per_launch: 1234\nsources_sha256: {good}\n")
    (tmp_path / "b_traffic_w2.md").write_text(body.replace("w1", "w2") + "traffic_bytes_per_launch: 99\nsources_sha256: 00\n")
    assert P.read_traffic("w1", fam)[0] == 1234.0
    val, why = P.read_traffic("w2", fam)
    assert val is None and "changed" in why
    assert P.read_traffic("w3", fam)[0] is None


def test_committed_traffic_profiles_parse():
    import glob, os
    for path in glob.glob(os.path.join(P.ROOT, "profiles", "*traffic*.md")):
        kv = dict(l.split(":", 1) for l in open(path) if l.startswith(("workload:", "kernel:", "traffic_bytes_per_launch:", "sources_sha256:")))
        assert float(kv["traffic_bytes_per_launch"]) > 0
        assert len(kv["sources_sha256"].strip()) == 64


def test_read_traffic_keeps_the_modes_apart(tmp_path, monkeypatch):
    monkeypatch.setattr(P, "PROFILES", str(tmp_path))
    fam = "mx_decode_kernel"
    good = P.sources_digest(fam)
    tail = f"kernel: mx_decode_kernel<true, 6, true>\nsources_sha256: {good}\n"
    (tmp_path / "a_traffic.md").write_text("workload: w1\nact_quant: mxfp8\ntraffic_bytes_per_launch: 7\n" + tail)
    (tmp_path / "b_traffic.md").write_text("workload: w1\ntraffic_bytes_per_launch: 5\n" + tail)
    assert P.read_traffic("w1", fam, "mxfp8")[0] == 7.0
    assert P.read_traffic("w1", fam)[0] == 5.0


def test_read_traffic_keeps_up_and_down_apart(tmp_path, monkeypatch):
    # the down kernel's summary sorts first; the roofline line needs the up kernel's
    monkeypatch.setattr(P, "PROFILES", str(tmp_path))
    fam = "big_gemm_kernel"
    good = P.sources_digest(fam)
    (tmp_path / "big_gemm_kernel_down_traffic_w1.md").write_text(
        f"workload: w1\nkernel: big_gemm_kernel<false, false, 320>\ntraffic_bytes_per_launch: 3\nsources_sha256: {good}\n")
    (tmp_path / "big_gemm_kernel_up_traffic_w1.md").write_text(
        f"workload: w1\nkernel: big_gemm_kernel<true, false, 320>\ntraffic_bytes_per_launch: 15\nsources_sha256: {good}\n")
    assert P.read_traffic("w1", fam) == (15.0, os.path.relpath(str(tmp_path / "big_gemm_kernel_up_traffic_w1.md"), P.ROOT))
    assert P.read_traffic("w1", fam, up=False)[0] == 3.0


def test_committed_up_traffic_is_the_up_kernel():
    for wl in ("mixtral-top2-n8192-d4096-e8-ff14336-bf16", "e128-top4-mxfp4-decode-n1"):
        fam = "big_gemm_kernel" if "mixtral" in wl else "mx_decode_kernel"
        val, src = P.read_traffic(wl, fam)
        if val is not None:
            assert "_up_traffic_" in src


def test_mfma_summary_arithmetic(tmp_path):
    # Two dispatches of one kernel, 100 us each, with counters chosen so the
    # derived figures are round: 2.0 GHz (GRBM_GUI_ACTIVE is summed over 8
    # XCDs), half the SIMD cycles busy, 1.5x the algorithmic flops counted.
    import csv
    wl = "switch-top1-n4096-d1024-e8-ff4096-bf16"
    alg = P.up_flops(wl)
    cycles = 2.0e9 * 100e-6
    vals = {"GRBM_GUI_ACTIVE": cycles * 8, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cycles * 1024,
            "SQ_INSTS_VALU_MFMA_MOPS_BF16": 1.5 * alg / 512, "SQ_INSTS_VALU_MFMA_MOPS_F8": 0.0}
    d = tmp_path / "run"
    d.mkdir()
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"])
        for disp, t0 in ((1, 1000), (2, 500000)):
            for k, v in vals.items():
                w.writerow([disp, "void moe::big_gemm_kernel<true, false>(p)", k, v, t0, t0 + 100000])
            w.writerow([disp + 10, "other_kernel", "GRBM_GUI_ACTIVE", 1, 0, 1])
    out = tmp_path / "m.md"
    import argparse
    P.cmd_mfma(argparse.Namespace(workload=wl, kernel="big_gemm_kernel<true", pmc=str(d), command="c",
                                  out=str(out), peak_tflops=2500.0, flops=None, act_quant=None))
    rows = {}
    for line in open(out):
        if line.startswith("| ") and line.count("|") == 3:
            k, v = line.strip().strip("|").split("|")
            rows[k.strip()] = v.strip()
    assert rows["counted / algorithmic"].strip() == "1.500"
    assert rows["average clock (GRBM_GUI_ACTIVE / duration, GHz)"].strip() == "2.000"
    assert rows["MFMA busy (SQ_VALU_MFMA_BUSY_CYCLES / (cycles x 1024 SIMDs))"].strip() == "0.500"
    ach = alg / 100e-6 / 1e12
    assert abs(float(rows["fraction of the peak at that clock"]) - ach / (2500.0 * 2.0 / 2.4)) < 1e-3


def test_projection_flops_by_kernel():
    # the up projection runs W1 and W3 (4 R d f flops), the down projection W2
    wl = "mixtral-top2-n8192-d4096-e8-ff14336-bf16"
    up = P.projection_flops(wl, "void moe::(anonymous namespace)::big_gemm_kernel<true, true, false, 320, 256, false>(moe::BigGemmParams)")
    down = P.projection_flops(wl, "void moe::(anonymous namespace)::big_gemm_kernel<false, false, false, 320, 256, true>(moe::BigGemmParams)")
    assert up == 4.0 * 8192 * 2 * 4096 * 14336
    assert down == up / 2
