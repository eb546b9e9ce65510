"""bench.py's host logic on the CPU: the one-GPU contract, the roofline
accounting of the method, the algorithmic bytes of the normal operator, and
the counter tables (each names a committed profile; an entry taken on the
current kernel sources yields traffic, a stale one none)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr


def test_method_roofline():
    # F^H D, one vector: 14 FLOP and 2 sincos per pair; transcendental-bound
    m = bench.method_roofline("fhd", 1)
    assert m["flop_per_voxel_sample"] == 14 and m["bound"] == "trans"
    assert m["p_roof_pairs_per_s"] == pytest.approx(bench.R_TRANS_PER_S / 2)
    # 16 vectors share the phase: 6 + 8 x 16 FLOP per (voxel, sample); FP32-bound
    m16 = bench.method_roofline("fhd", 16)
    assert m16["flop_per_voxel_sample"] == 134 and m16["bound"] == "fp32"
    assert m16["p_roof_pairs_per_s"] == pytest.approx(16 * bench.FP32_PEAK_TFLOPS * 1e12 / 134)
    assert bench.method_roofline("q", 1)["flop_per_voxel_sample"] == 10


def test_normal_operator_bytes():
    # 128^3: x pass (first iteration form), y, z with the spectrum, inverse y,
    # crop with the image and Ap: 520.1 MB, the count the CG profile uses
    assert bench.normal_operator_bytes(128, 128, 128) == pytest.approx(520.1e6, rel=1e-3)


@pytest.mark.parametrize("table", ["TRAFFIC", "MFMA_BUSY"])
def test_counter_tables_name_committed_profiles(table):
    for key, e in getattr(bench, table).items():
        assert os.path.exists(os.path.join(ROOT, e["profile"])), (key, e["profile"])
        assert len(e["kernel_sha256"]) == 16


def test_traffic_only_for_current_sources():
    for (config, trig, summ, engine, group), e in bench.TRAFFIC.items():
        rate, detail = bench.traffic_for(config, trig, summ, engine, group, 10.0)
        if e["kernel_sha256"] == bench.kernel_source_sha(e["source"]):
            assert detail["bytes_per_launch"] == pytest.approx(e["fetch_bytes"] + e["write_bytes"])
            assert rate == pytest.approx(detail["bytes_per_launch"] / 10e-3 / 1e9)
        else:
            assert rate is None and detail is None
    assert bench.traffic_for("no such workload", "hw", "blocked", "mfma", 128, 10.0) == (None, None)
