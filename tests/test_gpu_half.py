"""GPU parity of the half-split matrix-core engine (engine="mfma16": every fp32
product formed from fp16 parts on the fp16 matrix cores, fp32 accumulation)
against the double-precision oracle, at the same bars as the fp32 engines
(tests/gpu_util.TOL: rel-L2 1e-5 accurate, 2e-3 HW, plus the per-element bar).

  - grids whose groups of 128 / vectors voxels line up with x rows (the
    factored path), with ragged voxel and sample tails (a partial last wave,
    M not a multiple of the 32-sample chunk), one and several launch rows,
    both trig paths, F^H D, batched F^H D and Q;
  - irregular voxels (every wave takes the fp32 direct kernel), and a grid
    with one displaced voxel (that wave direct, the other factored);
  - data whose Mu spans nine orders of magnitude (the power-of-two factor
    scale and the fp16 parts' range);
  - M = 0 and M = 1; two runs bitwise equal.
The full-size workloads (32^3 to 512^3, off-grid, Q, the batched 96^3 case)
run in tests/test_gpu_configs.py beside the other engines.
"""
import numpy as np
import pytest

from non_cartesian_mri_amd import inputs
from tests.gpu_util import TOL, assert_close, dev_problem, gpu_fhd, gpu_q, require_gpu

pytestmark = pytest.mark.gpu

TRIGS = ["accurate", "hw"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _rows(ny, nz, n=None, nx=128):
    """Voxel coordinates of an nx x ny x nz grid (x fastest), the first n."""
    iz, iy, ix = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")
    x, y, z = ((a.ravel() - s // 2).astype(np.float32) for a, s in ((ix, nx), (iy, ny), (iz, nz)))
    return (x, y, z) if n is None else (x[:n], y[:n], z[:n])


def _problem(seed, M, coords, B=1, kind="fhd", mu_range=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    kx, ky, kz = inputs.uniform_k(M, rng)
    x, y, z = coords
    phi = inputs.complex_normal(rng, M)
    D = None
    if kind == "fhd":
        D = np.stack([inputs.complex_normal(rng, M) for _ in range(B)]).reshape(B, M)
        if mu_range is not None:   # per-sample magnitudes 10^U(-r, r)
            D = (D * (10.0 ** rng.uniform(-mu_range, mu_range, M))).astype(np.complex64)
    return inputs.Problem(f"half{seed}", kind, kx, ky, kz, x, y, z, phi, D, seed)


def _check(oracle_mod, p, what, **opts):
    ref = (oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi) if p.kind == "q"
           else oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D))
    d = dev_problem(p)
    got = gpu_q(p, d, engine="mfma16", **opts) if p.kind == "q" else gpu_fhd(p, d, engine="mfma16", **opts)
    assert_close(got, ref, TOL[opts.get("trig", "accurate")], what)
    return got


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("M,splits,tile", [(1001, 0, 0), (1001, 3, 0), (32, 1, 0), (4099, 0, 0), (4099, 1, 0),
                                           (4099, 1, 64), (4099, 2, 96)])
def test_grid(oracle_mod, trig, M, splits, tile):
    # 128 x 5 x 3 voxels cut to 1900: one wave of 16 groups, the last partial;
    # tile > 0: tiles folded into running totals (the accurate path's default
    # is ~sqrt(M), the HW path's the whole launch row)
    p = _problem(301, M, _rows(5, 3, n=1900))
    _check(oracle_mod, p, f"mfma16 grid M={M} splits={splits} tile={tile} {trig}", trig=trig,
           sample_splits=splits, tile=tile)


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("B", [2, 16, 19])
def test_batch(oracle_mod, trig, B):
    # passes of 16, 8, 4, 2, 1 vectors: groups of 8 to 128 voxels
    p = _problem(302, 777, _rows(4, 2), B=B)
    _check(oracle_mod, p, f"mfma16 batch B={B} {trig}", trig=trig)


@pytest.mark.parametrize("trig", TRIGS)
def test_q(oracle_mod, trig):
    p = _problem(303, 2049, _rows(6, 2), kind="q")
    _check(oracle_mod, p, f"mfma16 Q {trig}", trig=trig)


@pytest.mark.parametrize("trig", TRIGS)
def test_irregular_voxels(oracle_mod, trig):
    rng = np.random.Generator(np.random.PCG64(304))
    c = ((rng.random((3, 1500)) - 0.5) * 24).astype(np.float32)
    p = _problem(304, 1200, (c[0], c[1], c[2]))
    _check(oracle_mod, p, f"mfma16 irregular {trig}", trig=trig)


@pytest.mark.parametrize("trig", TRIGS)
def test_one_displaced_voxel(oracle_mod, trig):
    # two waves of 2048 voxels; a voxel of the second is moved off the grid
    x, y, z = _rows(8, 4)
    x = x.copy()
    x[3000] += 0.3
    p = _problem(305, 900, (x, y, z))
    _check(oracle_mod, p, f"mfma16 one displaced voxel {trig}", trig=trig)


def test_wide_dynamic_range(oracle_mod):
    # |Mu| over nine orders of magnitude: the factors' power-of-two scale puts
    # the largest near 2^14; the smallest parts fall to fp16 subnormals
    p = _problem(306, 3000, _rows(4, 2), mu_range=4.5)
    _check(oracle_mod, p, "mfma16 |Mu| over 1e9", trig="accurate")


@pytest.mark.parametrize("M", [0, 1])
def test_tiny_M(oracle_mod, M):
    p = _problem(307, M, _rows(2, 1))
    got = gpu_fhd(p, dev_problem(p), engine="mfma16", trig="accurate")
    if M == 0:
        assert np.all(got == 0)
    else:
        ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
        assert_close(got, ref, TOL["accurate"], "mfma16 M=1")


def test_deterministic():
    p = _problem(308, 2500, _rows(8, 2))
    d = dev_problem(p)
    a = gpu_fhd(p, d, engine="mfma16", trig="hw")
    b = gpu_fhd(p, d, engine="mfma16", trig="hw")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
