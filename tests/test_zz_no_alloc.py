"""fhd_compute_noalloc (the entry point for callers that cannot allocate)
against fhd_compute, through the C ABI.

Two calls in a row on the library's fixed device array, the second with a
smaller problem (so it runs on what the first left in the array), each
compared bitwise with fhd_compute given the same plan (same kernels, same
launch shape, so the same bits); then the 128^3 x 262,144 benchmark workload,
whose automatic plan needs more than the array holds, so the entry point
lowers the sample-row count: bitwise equal to fhd_compute with that row count
and within the trig path's bar of fhd_compute's default plan.
"""
import numpy as np
import pytest
import torch

from non_cartesian_mri_amd import _lib, inputs
from tests.gpu_util import TOL, assert_close, dev_problem, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _both(p, d, **opts):
    from non_cartesian_mri_amd import fhd_compute, fhd_compute_noalloc
    args = (d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], d["D"])
    out = torch.empty((p.B, p.N), dtype=torch.complex64, device="cuda:0")
    got = fhd_compute_noalloc(*args, out=out, **opts)
    want = fhd_compute(*args, **opts)
    torch.cuda.synchronize()
    return got.cpu().numpy().reshape(p.B, p.N), want.cpu().numpy().reshape(p.B, p.N)


@pytest.mark.parametrize("engine", ["auto", "mfma16"])
@pytest.mark.parametrize("trig", ["hw", "accurate"])
def test_two_calls_in_a_row_second_smaller(oracle_mod, trig, engine):
    # engine "mfma16": the half-split kernels, whose scale, factor parts and Mu
    # also live in the array
    big = inputs.make_config("fhd_64cube_65536_radial")
    small = inputs.random_problem(901, M=2047, L=16, B=3)
    for p in (big, small):
        print(f"[noalloc] {p.name} trig={trig} engine={engine} N={p.N} M={p.M} B={p.B}", flush=True)
        got, want = _both(p, dev_problem(p), trig=trig, engine=engine)
        assert np.array_equal(got, want), f"{p.name}: noalloc differs from fhd_compute"
    ref = oracle_mod.fhd(small.kx, small.ky, small.kz, small.x, small.y, small.z, small.phi, small.D)
    assert_close(got, ref, TOL[trig], f"noalloc {small.name} {trig} {engine}")


def test_plan_lowered_to_fit_the_array():
    from non_cartesian_mri_amd import fhd_describe_plan, fhd_workspace_bytes
    p = inputs.make_config("fhd_128cube_262144_spirals")
    cap = _lib.NOALLOC_SCRATCH_BYTES
    auto = fhd_describe_plan(p.M, p.N, 1, trig="hw")
    assert auto["workspace_bytes"] > cap    # the default plan does not fit
    s = auto["sample_splits"]
    while s > 1 and fhd_workspace_bytes(p.M, p.N, 1, trig="hw", sample_splits=s) > cap:
        s -= 1
    assert fhd_workspace_bytes(p.M, p.N, 1, trig="hw", sample_splits=s) <= cap
    print(f"[noalloc] {p.name}: {auto['sample_splits']} rows planned, {s} fit", flush=True)
    d = dev_problem(p)
    got, want = _both(p, d, trig="hw", sample_splits=s)
    assert np.array_equal(got, want)
    from non_cartesian_mri_amd import fhd_compute_noalloc, fhd_compute
    args = (d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], d["D"])
    auto_rows = fhd_compute_noalloc(*args, trig="hw")
    default = fhd_compute(*args, trig="hw")
    torch.cuda.synchronize()
    assert np.array_equal(auto_rows.cpu().numpy().reshape(-1), got.reshape(-1))
    assert_close(auto_rows.cpu().numpy(), default.cpu().numpy(), TOL["hw"], "noalloc lowered rows vs default")
