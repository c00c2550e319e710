"""Host-side checks of the rocprofv3 summary helpers used by bench.py."""

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
