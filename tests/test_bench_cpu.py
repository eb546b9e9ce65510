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


def _plan_workspace(nbytes, offset, header):
    import torch
    ws = torch.zeros(nbytes, dtype=torch.uint8)
    ws[offset:offset + 4 * len(header)] = torch.tensor(header, dtype=torch.int32).view(torch.uint8)
    return ws


def test_mirror_pair_work_reads_the_plan():
    """The adjoint's pair plan sits at the end of the workspace; 128^3 with
    8,064 pairs and 256 groups alone: 520 wave slots of 32 MFMAs per block of
    four samples against 1,024 waves of 24 -> 4.0625 executed FLOP per pair."""
    from types import SimpleNamespace
    G = 16384
    pair_bytes = ((64 + 8 * G + 15) // 16 * 16 + 16 * G + 255) // 256 * 256
    nbytes = 10 * pair_bytes
    ws = _plan_workspace(nbytes, nbytes - pair_bytes, [8320, 8064, 31, 8464, 520, 130, 16512])
    p = SimpleNamespace(N=128 ** 3, M=262144, B=1)
    plan = {"voxels_per_lane": 128, "padded_samples": 262144, "passes": 1}
    w = bench.mirror_pair_work(ws, nbytes, p, plan)
    assert (w["paired_groups"], w["groups_alone"], w["launch_rows"], w["wave_slots"]) == (8064, 256, 31, 520)
    assert w["executed_flop_per_pair"] == pytest.approx(4.0625)
    assert w["mfma_ratio_to_unpaired"] == pytest.approx(520 * 32 / (1024 * 24), abs=1e-4)


def test_forward_pair_work_reads_the_plan():
    """The forward's pair plan follows the entry headers, entries, list and
    wave flags of the pass; 8,320 entries over 16,384 groups -> 4.0625."""
    from types import SimpleNamespace
    G, gpad = 16384, 16384
    a256 = lambda b: (b + 255) // 256 * 256
    off = a256(gpad * 16) + a256(gpad * 64 * 8 * 4) + a256(4 * (gpad + 1)) + a256(4 * (G // 16))
    ws = _plan_workspace(off + 4096, off, [8320, 8064, 1, 0, 520, 130, 16512])
    p = SimpleNamespace(N=128 ** 3, M=262144, B=1)
    plan = {"voxels_per_lane": 128, "passes": 1, "sample_splits": 1}
    w = bench.forward_pair_work(ws, p, plan)
    assert (w["paired_groups"], w["groups_alone"]) == (8064, 256)
    assert w["executed_flop_per_pair"] == pytest.approx(4.0625)
    assert w["mfma_ratio_to_unpaired"] == pytest.approx(8320 * 32 / (16384 * 24), abs=1e-4)
