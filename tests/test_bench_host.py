"""Host-side checks of bench.py's bookkeeping (no GPU needed)."""
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_source_digest_ignores_comments_only(tmp_path):
    a = tmp_path / "a.hip"
    a.write_text("// header\nint f(int x) {\n  return x + 1;  // one\n}\n/* block\n comment */\n")
    b = tmp_path / "b.hip"
    b.write_text("// another header\nint f(int x)   {\n    return x + 1;\n}\n")
    c = tmp_path / "c.hip"
    c.write_text("int f(int x) {\n  return x + 2;\n}\n")
    assert bench.source_digest(str(a)) == bench.source_digest(str(b))
    assert bench.source_digest(str(a)) != bench.source_digest(str(c))


def _record(path, kernel, src, traffic):
    path.write_text(f"# header\nkernel: {kernel}\nsource_sha256: {bench.source_digest(str(src))}\n"
                    f"traffic_bytes_per_launch: {traffic}\n")


def test_recorded_traffic_per_kernel(tmp_path, monkeypatch):
    # a record is found under either decode kernel's name, is voided by a
    # change to that kernel's source, and is not used while a decode
    # variant is forced through the environment
    src_m = tmp_path / "m.hip"
    src_m.write_text("int m() { return 1; }\n")
    src_s = tmp_path / "s.hip"
    src_s.write_text("int s() { return 2; }\n")
    prof = tmp_path / "profiles"
    prof.mkdir()
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "DECODE_SOURCES", {"decode_mfma": str(src_m), "decode_split": str(src_s)})
    monkeypatch.delenv("TQ_DECODE_VARIANT", raising=False)
    _record(prof / "decode_mfma_wa_hbm_traffic.txt", "decode_mfma_kernel", src_m, 1000)
    _record(prof / "decode_split_wb_hbm_traffic.txt", "decode_split_kernel", src_s, 2000)
    assert bench.recorded_traffic("wa") == 1000
    assert bench.recorded_traffic("wb") == 2000
    assert bench.recorded_traffic("wc") is None
    monkeypatch.setenv("TQ_DECODE_VARIANT", "ref")
    assert bench.recorded_traffic("wa") is None
    monkeypatch.delenv("TQ_DECODE_VARIANT")
    src_s.write_text("int s() { return 3; }\n")
    assert bench.recorded_traffic("wb") is None
    assert bench.recorded_traffic("wa") == 1000


def test_committed_traffic_records_parse():
    # every committed counter summary names its kernel's source and carries
    # the fields the bench reads
    prof = os.path.join(ROOT, "profiles")
    for name in sorted(os.listdir(prof)):
        if not name.endswith("_hbm_traffic.txt"):
            continue
        fields = {}
        with open(os.path.join(prof, name)) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        assert name.split("_")[0] + "_" + name.split("_")[1] in bench.DECODE_SOURCES, name
        assert len(fields["source_sha256"]) == 64, name
        assert int(float(fields["traffic_bytes_per_launch"])) > 0, name
        # above a megabyte the fixed costs (partials, counters, whole cache
        # lines) must stay small; the tiny d = 64 case is all fixed cost
        if int(fields["algorithmic_bytes_per_launch"]) > 1 << 20:
            assert float(fields["traffic_over_algorithmic"]) < 1.5, name


def test_trace_summary_keeps_the_timed_dispatches(tmp_path):
    # six decode dispatches: two warm-up ones of 100 us, then four of 30 us;
    # with steps 2 and layers 2 only the last four enter the average
    import bench
    path = tmp_path / "trace.csv"
    name = "void tq::(anonymous namespace)::decode_mfma_kernel<3, 4, false, false>(tq::DecodeParams)"
    with open(path, "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        t = 0
        for dur in (100000, 100000, 30000, 30000, 30000, 30000):
            f.write(f"\"{name}\",{t},{t + dur}\n")
            t += dur + 1000
    out = bench.trace_summary(str(path), "c4_tq35_32k", 4, ["cmd"])
    line = next(ln for ln in out.splitlines() if ln.startswith("decode_mfma_kernel"))
    calls, avg = line.split()[-5], float(line.split()[-4])
    assert calls == "4" and avg == 30.0
    gbs = bench.decode_bytes(bench.WORKLOADS["c4_tq35_32k"]) / 30e-6 / 1e9
    assert f"{gbs:.1f} GB/s" in out


def test_pmc_summary_per_chunk(tmp_path):
    import bench
    path = tmp_path / "pmc.csv"
    name = "void tq::(anonymous namespace)::decode_mfma_kernel<3, 4, false, false>(tq::DecodeParams)"
    chunks = 4 * 8 * 32768 // 32
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for v in (2.0, 4.0):
            f.write(f"\"{name}\",SQ_INSTS_VALU,{v * chunks}\n")
            f.write(f"\"{name}\",SQ_WAVE_CYCLES,{10 * v * chunks}\n")
            f.write(f"\"{name}\",SQ_ACTIVE_INST_VALU,{v * chunks}\n")
    out = bench.pmc_summary([str(path)], "c4_tq35_32k", ["cmd"], "test")
    assert "per chunk       3.00" in out
    assert "SQ_ACTIVE_INST_VALU / SQ_WAVE_CYCLES = 0.1000" in out


def test_traffic_key_separates_sparse_v():
    # a sparse-V decode fetches fewer bytes, so its record is its own
    assert bench.traffic_key("c4_tq35_32k") == "c4_tq35_32k"
    assert bench.traffic_key("c4_tq35_32k", 0.0) == "c4_tq35_32k"
    assert bench.traffic_key("c4_tq35_32k_peaked", 0.001) == "c4_tq35_32k_peaked_sparse_v0.001"
