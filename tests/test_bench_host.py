"""Host logic of bench.py (CPU, no device): the one-GPU refusal, the sha-tied
reading of rocprofv3 traffic summaries, and the per-kernel statistics and
roofline arithmetic the JSON line reports."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused_before_any_device_work():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""


def test_every_counter_summary_names_known_sources():
    names = [f[len("counters_"):-4] for f in os.listdir(os.path.join(ROOT, "profiles"))
             if f.startswith("counters_") and f.endswith(".txt")]
    assert names
    for n in names:
        assert n in bench.KERNEL_SOURCES, n
        text = open(os.path.join(ROOT, "profiles", f"counters_{n}.txt")).read()
        assert "kernel_sources_sha256:" in text and "hbm_bytes_per_launch:" in text, n


def _fake_tree(tmp_path, sha, nbytes):
    csrc = tmp_path / "optimizer_step_adamw_amd" / "csrc"
    csrc.mkdir(parents=True)
    for f in bench.KERNEL_SOURCES["adamw_fp32"]:
        shutil.copy(os.path.join(ROOT, "optimizer_step_adamw_amd", "csrc", f), csrc / f)
    prof = tmp_path / "profiles"
    prof.mkdir()
    (prof / "counters_adamw_fp32.txt").write_text(
        f"HBM traffic\n\nhbm_bytes_per_launch: {nbytes}\nkernel_sources_sha256: {sha}\n")
    return tmp_path


def test_traffic_is_reported_only_for_the_sources_it_was_measured_on(tmp_path, monkeypatch):
    real = bench.kernel_sources_sha256("adamw_fp32")
    monkeypatch.setattr(bench, "ROOT", str(_fake_tree(tmp_path, real, 471103258)))
    assert bench.kernel_sources_sha256("adamw_fp32") == real
    assert bench.traffic_from_profile("adamw_fp32") == 471103258.0
    # a changed kernel source: the summary no longer applies
    src = tmp_path / "optimizer_step_adamw_amd" / "csrc" / "kernels_adam.hip"
    src.write_text(src.read_text() + "\n// edited\n")
    assert bench.traffic_from_profile("adamw_fp32") is None
    # unknown kernels and missing summaries give None too
    assert bench.traffic_from_profile("no_such_kernel") is None


def test_kernel_stats_and_roofline_arithmetic():
    recs = [("adam_kernel", 4096, 0.080), ("adam_kernel", 4096, 0.078), ("other", 1, 5.0),
            ("adam_kernel", 4096, 0.082)]
    st = bench.kernel_stats(recs, "adam_kernel")
    assert st["launches"] == 3 and st["workgroups"] == [4096]
    assert st["mean_ms"] == pytest.approx(0.080) and st["median_ms"] == pytest.approx(0.080)
    assert st["p10_ms"] == pytest.approx(0.078) and st["p90_ms"] == pytest.approx(0.082)
    assert bench.kernel_stats(recs, "missing") is None
    nbytes = 28.0 * 4096 * 4096
    e = bench.roofline_entry("adam_kernel", "w", nbytes, st, ceiling=dict(gbs=5800.0), traffic=nbytes * 1.003)
    assert e["achieved"] == pytest.approx(nbytes / 0.080e-3 / 1e9)
    assert e["frac"] == pytest.approx(e["achieved"] / 8000.0)
    assert e["frac_of_ceiling"] == pytest.approx(e["achieved"] / 5800.0)
    assert e["bound"] == "hbm" and e["unit"] == "GB/s" and e["peak"] == 8000.0


def test_read_write_bound_model():
    """(R + W) / (R / read + W / write): a pure read stays at the read rate, a
    pure write at the better of the two write probes, and a mix lies between
    them, nearer the side that moves more bytes."""
    ceil = {"read_fp32_268M": {"gbs": 6600.0}, "write_fp32_268M": {"gbs": 5400.0},
            "write_fp32_ordinary_268M": {"gbs": 5500.0}}
    assert bench.rw_bound(ceil, (4.0, 0.0))["gbs"] == pytest.approx(6600.0)
    assert bench.rw_bound(ceil, (0.0, 4.0))["gbs"] == pytest.approx(5500.0)
    adamw = bench.rw_bound(ceil, (16.0, 12.0))["gbs"]
    assert adamw == pytest.approx(28.0 / (16.0 / 6600.0 + 12.0 / 5500.0))
    assert 5500.0 < adamw < 6600.0
    assert bench.rw_bound({}, (16.0, 12.0)) is None and bench.rw_bound(ceil, None) is None
    # every roofline workload's split adds up to its algorithmic bytes per element
    assert sum(bench.RW_SPLIT["adamw_fp32_4096x4096"]) == bench.B_ADAMW_F32
    assert sum(bench.RW_SPLIT["ademamix_fp32_4096x4096"]) == bench.B_ADEMAMIX_F32
    assert sum(bench.RW_SPLIT["adamw_bf16_remainder_llama1b"]) == bench.B_BF16R
    assert sum(bench.RW_SPLIT["blockwise_8bit_268M"]) == pytest.approx(bench.B_8BIT)
    assert sum(bench.RW_SPLIT["blockwise_4bit_268M"]) == pytest.approx(bench.B_4BIT)
