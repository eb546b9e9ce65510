"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default options: automatic group size and tile).

The oracle evaluates seeded voxel subsets (all voxels for the 32^3 and 64^3
cases), the
phantom round trip compares PSNR of the GPU and oracle images on the three
central slices, and Q is also checked at its closed forms: Q(0) = sum |phi|^2
and Hermitian symmetry on the grid.
"""
import math

import numpy as np
import pytest
import torch

from non_cartesian_mri_amd import inputs
from tests.gpu_util import TOL, assert_close, dev_problem, gpu_fhd, gpu_q, require_gpu

pytestmark = pytest.mark.gpu

TRIGS = ["accurate", "hw"]
# oracle voxels per workload (None: every voxel)
SUBSET = {"fhd_32cube_2048_uniform": None, "fhd_64cube_65536_radial": None, "fhd_512cube_262144_spirals": 1024,
          "fhd_128cube_262144_spirals": 4096, "fhd_128cube_262144_spirals_jittered": 4096,
          "q_128cube_halfstep_1048576_uniform": 4096, "q_128cube_unitstep_1048576_uniform": 2048,
          "fhd16_96cube_500001_radial": 2048}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


_cache = {}


def _problem_and_ref(name, oracle_mod):
    if name not in _cache:
        p = inputs.make_config(name)
        idx = None if SUBSET[name] is None else inputs.subset_indices(p.N, SUBSET[name], p.seed)
        if p.kind == "q":
            ref = oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, idx=idx)
        else:
            ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D, idx=idx)
        print(f"[oracle] {name}: {oracle_mod.last.seconds:.1f}s on {oracle_mod.last.threads} threads", flush=True)
        _cache[name] = (p, idx, ref, dev_problem(p))
    return _cache[name]


ENGINES = ["auto", "valu", "mfma16"]   # auto = the matrix-core engine for these options; mfma16 the half-split one


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("name", ["fhd_32cube_2048_uniform", "fhd_64cube_65536_radial", "fhd_128cube_262144_spirals",
                                  "fhd16_96cube_500001_radial", "fhd_512cube_262144_spirals"])
def test_fhd_config(oracle_mod, name, trig, engine):
    p, idx, ref, d = _problem_and_ref(name, oracle_mod)
    print(f"[gpu] {name} trig={trig} engine={engine} N={p.N} M={p.M} B={p.B}", flush=True)
    got = gpu_fhd(p, d, trig=trig, engine=engine)
    if idx is not None:
        got = got[:, idx]
    assert_close(got, ref, TOL[trig], f"{name} {trig} {engine}")


@pytest.mark.parametrize("trig", TRIGS)
def test_fhd_per_pair_kernel_full_size(oracle_mod, trig):
    """The pages' own form of the gather (one voxel per lane, one phase, sine,
    cosine and complex multiply-accumulate per voxel-sample pair: the VALU
    engine with one voxel per lane) at 128^3 x 262,144 with its planned
    launch rows."""
    name = "fhd_128cube_262144_spirals"
    p, idx, ref, d = _problem_and_ref(name, oracle_mod)
    got = gpu_fhd(p, d, trig=trig, engine="valu", voxels_per_lane=1)
    assert_close(got[:, idx], ref, TOL[trig], f"{name} {trig} per-pair")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("trig", TRIGS)
def test_fhd_off_grid_full_size(oracle_mod, trig, engine):
    """2,097,152 voxel centres off the grid (the 128^3 centres displaced by up
    to a quarter voxel per axis): no voxel group shares common offsets, so
    every wave takes the direct per-voxel evaluation of its engine."""
    name = "fhd_128cube_262144_spirals_jittered"
    p, idx, ref, d = _problem_and_ref(name, oracle_mod)
    print(f"[gpu] {name} trig={trig} engine={engine}", flush=True)
    got = gpu_fhd(p, d, trig=trig, engine=engine)
    assert_close(got[:, idx], ref, TOL[trig], f"{name} {trig} {engine}")


@pytest.mark.parametrize("engine", ENGINES)
@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("name", ["q_128cube_halfstep_1048576_uniform", "q_128cube_unitstep_1048576_uniform"])
def test_q_config(oracle_mod, name, trig, engine):
    p, idx, ref, d = _problem_and_ref(name, oracle_mod)
    print(f"[gpu] {name} trig={trig} engine={engine} N={p.N} M={p.M}", flush=True)
    got = gpu_q(p, d, trig=trig, engine=engine)
    assert_close(got[idx], ref, TOL[trig], f"{name} {trig}")
    # closed forms at full size
    w = np.abs(p.phi.astype(np.complex128)) ** 2
    o = np.nonzero((p.x == 0) & (p.y == 0) & (p.z == 0))[0][0]
    assert abs(got[o] - w.sum()) <= TOL[trig] * w.sum()
    # Hermitian pairs: voxel (i,j,k) and its mirror through the origin
    L = 128
    rng = np.random.Generator(np.random.PCG64(7))
    ii = rng.integers(1, L, size=(512, 3))
    n = (ii[:, 2] * L + ii[:, 1]) * L + ii[:, 0]
    mi = L - ii
    nm = (mi[:, 2] * L + mi[:, 1]) * L + mi[:, 0]
    assert np.all(p.x[nm] == -p.x[n]) and np.all(p.z[nm] == -p.z[n])
    rms = np.sqrt(np.mean(np.abs(ref) ** 2))
    assert np.max(np.abs(got[nm] - np.conj(got[n]))) <= 6 * TOL[trig] * rms


def test_phantom_round_trip_psnr(oracle_mod):
    """Ellipsoid phantom -> analytic k-space on the radial trajectory -> F^H D with
    density weights |k|^2: PSNR of the GPU image may drop at most 0.1 dB from the oracle's
    (the drop the pages report for hardware trigonometry, tests/golden/pages_figures.json)."""
    from tests.test_golden_cpu import psnr_drop_gate_db
    gate = psnr_drop_gate_db()
    p = inputs.make_config("phantom_96cube_500001_radial")
    sl = p.extra["slices"]
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D, idx=sl)[0]
    print(f"[oracle] phantom slices ({sl.size} voxels): {oracle_mod.last.seconds:.1f}s", flush=True)
    I0 = inputs.phantom_image(p.x[sl], p.y[sl], p.z[sl])
    alpha = oracle_mod.ls_scale(I0, ref)
    ps_ref = oracle_mod.psnr_db(I0, ref, alpha)
    d = dev_problem(p)
    for engine in ENGINES:
        for trig in TRIGS:
            got = gpu_fhd(p, d, trig=trig, engine=engine)[0, sl]
            ps = oracle_mod.psnr_db(I0, got, alpha)
            print(f"[psnr] oracle {ps_ref:.3f} dB, gpu {trig}/{engine} {ps:.3f} dB", flush=True)
            assert math.isfinite(ps_ref) and ps_ref > 5.0
            assert ps_ref - ps <= gate
            assert_close(got, ref, TOL[trig], f"phantom {trig} {engine}")
