"""The measurement records bench.py reads (profiles/*.json): they are reported only while
they were taken on the current kernel source, and their derived figures follow from the
raw counter readings they hold."""
import json
import os

import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
WL = "gqa_causal_h32_kv8_n32768_d128"


def _write(tmp_path, name, rec):
    d = tmp_path / "profiles"
    d.mkdir(exist_ok=True)
    (d / name).write_text(json.dumps(rec))


def test_records_follow_the_source_hash(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda *a: "abc")
    assert bench.measured_traffic(WL) is None
    _write(tmp_path, f"traffic_fwd_counted_{WL}.json", {"kernel_source_hash": "abc", "hbm_bytes_per_launch": 123})
    assert bench.measured_traffic(WL) == 123
    # a record of another kernel source is not reported
    monkeypatch.setattr(bench, "kernel_source_hash", lambda *a: "def")
    assert bench.measured_traffic(WL) is None


def test_committed_traffic_record_is_consistent():
    with open(os.path.join(ROOT, "profiles", f"traffic_fwd_counted_{WL}.json")) as f:
        rec = json.load(f)
    cal = rec["calibration"]
    # the factors are what make the copy's counters read its known size
    assert cal["fetch_factor"] == pytest.approx(cal["copy_bytes"] / 1024 / cal["copy_fetch_size_kib"], rel=1e-3)
    assert cal["write_factor"] == pytest.approx(cal["copy_bytes"] / 1024 / cal["copy_write_size_kib"], rel=1e-3)
    hbm = 1024 * (rec["fetch_size_kib_per_launch"] * cal["fetch_factor"]
                  + rec["write_size_kib_per_launch"] * cal["write_factor"])
    assert rec["hbm_bytes_per_launch"] == pytest.approx(hbm, rel=1e-6)
    assert rec["hbm_over_algorithmic"] == pytest.approx(rec["hbm_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"],
                                                        rel=1e-3)
    # the write side is O (fp32) at least
    from precision_attention_amd import inputs as I
    w = I.WORKLOADS[WL]
    assert rec["algorithmic_bytes_per_launch"] == w.bytes()
    assert 1024 * rec["write_size_kib_per_launch"] * cal["write_factor"] >= 4 * w.B * w.H * w.N * w.d
    for cmd in rec["commands"]:
        assert cmd.startswith("rocprofv3 ") and " -- python -u bench.py " in cmd


def test_committed_sq_record_is_consistent():
    with open(os.path.join(ROOT, "profiles", f"sq_fwd_counted_{WL}.json")) as f:
        rec = json.load(f)
    c = rec["counters_per_launch"]
    cycles = c["GRBM_GUI_ACTIVE"] / 8
    assert rec["sclk_ghz"] == pytest.approx(cycles / rec["kernel_median_ns"], rel=1e-3)
    assert 1.0 < rec["sclk_ghz"] < 2.5
    assert rec["mfma_per_wave_step"] == pytest.approx(c["SQ_INSTS_MFMA"] / rec["wave_steps_per_launch"], rel=1e-3)
    assert rec["mfma_busy_frac"] == pytest.approx(c["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / cycles, rel=1e-2)
    # 8 MFMAs per wave-step (4 for S, 4 for P.V at d = 128), 64 cycles each
    assert rec["mfma_per_wave_step"] == pytest.approx(8.0)
    assert c["SQ_VALU_MFMA_BUSY_CYCLES"] == pytest.approx(64 * c["SQ_INSTS_MFMA"], rel=0.01)
    assert 0.0 < rec["coexec_frac_of_mfma"] <= 1.0
    # the vector-ALU share of the modelled vector work per wave-step over the launch's SIMD cycles
    assert rec["valu_busy_frac_model"] == pytest.approx(
        rec["valu_cycles_per_wave_step_model"] * rec["wave_steps_per_launch"] / 1024 / cycles, rel=1e-3)
    assert 0.0 < rec["valu_busy_frac_model"] <= 1.0
    for cmd in rec["commands"]:
        assert cmd.startswith("rocprofv3 ") and " -- python -u bench.py " in cmd


def test_source_hash_ignores_comments_only(tmp_path, monkeypatch):
    code = "// header\nint f(int a) { /* note */ return a + 1; }  // tail\n"
    assert bench.strip_comments(code) == "int f(int a) { return a + 1; }"
    srcs = []
    for i, rel in enumerate(bench.KERNEL_SOURCES):
        path = tmp_path / rel
        path.parent.mkdir(parents=True, exist_ok=True)
        path.write_text(f"int x{i} = {i};\n")
        srcs.append(path)
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    h0 = bench.kernel_source_hash()
    srcs[0].write_text("// a comment\nint x0 =   0; /* more */\n")
    assert bench.kernel_source_hash() == h0
    srcs[0].write_text("int x0 = 1;\n")
    assert bench.kernel_source_hash() != h0



@pytest.mark.parametrize("wl", ["decode_gqa_h32_kv8_n131072_d128", "decode_b8_gqa_h32_kv8_n32768_d128"])
def test_committed_decode_traffic_records_are_consistent(wl):
    from precision_attention_amd import inputs as I

    with open(os.path.join(ROOT, "profiles", f"traffic_decode_{wl}.json")) as f:
        rec = json.load(f)
    cal = rec["calibration"]
    fetch = 1024 * sum(rec["fetch_size_kib_per_call"].values()) * cal["fetch_factor"]
    write = 1024 * sum(rec["write_size_kib_per_call"].values()) * cal["write_factor"]
    assert rec["hbm_bytes_per_launch"] == pytest.approx(fetch + write, rel=1e-6)
    w = I.WORKLOADS[wl]
    assert rec["algorithmic_bytes_per_launch"] == w.bytes()
    # K and V are read at least once; the split records (d + 4 floats per head and split)
    # and O are written at least once
    assert fetch >= 2 * w.B * w.Hkv * w.N * w.d
    assert rec["hbm_over_algorithmic"] == pytest.approx((fetch + write) / w.bytes(), rel=1e-3)
    for cmd in rec["commands"]:
        assert cmd.startswith("rocprofv3 ") and " -- python -u bench.py " in cmd
    # taken at the split count the bench runs
    from precision_attention_amd import binding

    assert rec["n_split"] == binding.decode_default_splits(w.B, w.Hkv, w.H, w.N)


def test_decode_record_follows_the_split_count(tmp_path, monkeypatch):
    wl = "decode_b8_gqa_h32_kv8_n32768_d128"
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda *a: "abc")
    _write(tmp_path, f"traffic_decode_{wl}.json", {"kernel_source_hash": "abc", "n_split": 8, "hbm_bytes_per_launch": 7})
    assert bench.measured_traffic(wl, "decode", n_split=8) == 7
    assert bench.measured_traffic(wl, "decode", n_split=16) is None


def test_quality_heads_exist_for_every_workload():
    import bench
    from precision_attention_amd import inputs as I

    for w in I.WORKLOADS.values():
        heads = bench.quality_heads(w.H)
        assert heads and all(b == 0 and 0 <= h < w.H for b, h in heads), w.name
    assert bench.quality_heads(32) == ((0, 0), (0, 9), (0, 22), (0, 31))
