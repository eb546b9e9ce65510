"""GPU parity of the half-split forward operator (fhd_forward with
engine="mfma16": the four-group engine's sum over voxel groups with every
fp32 product formed from fp16 hi/lo parts on the fp16 matrix cores, fp32
accumulation) against the double-precision oracle, at the fp32 engines' bars
(tests/gpu_util.TOL).

  - grids whose groups of 128 / vectors voxels line up with x rows, with a
    partial last group and chunk of 32 groups, ragged sample counts (a
    partial last wave of 16), one and several launch rows, tiles folded into
    running totals and a tile that spans the launch row, blocked and plain
    sums, both trig paths;
  - batches of 2 to 19 images (passes of 16, 8, 4, 2 and 1 vectors);
  - irregular voxels (every group off the common offsets: all direct), one
    displaced voxel, tiny voxel counts, an all-zero image (scale 1);
  - an image whose magnitudes span nine orders of magnitude (the power-of-two
    scale and the fp16 parts' range);
  - x rows whose octets of groups are equally spaced (phases stepped by
    rotations) in the identity order or a strided chunk order, not at all
    (evaluated per group), or both in one wave;
  - the 128^3 and 512^3 x 262,144 workloads on sampled outputs; adjointness
    with the half-split F^H D; two runs bitwise equal.
"""
import numpy as np
import pytest
import torch

from non_cartesian_mri_amd import inputs
from tests.gpu_util import TOL, assert_close, dev_problem, require_gpu

pytestmark = pytest.mark.gpu

TRIGS = ["accurate", "hw"]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _images(seed, B, N, mag_range=None):
    rng = np.random.Generator(np.random.PCG64(seed))
    r = np.stack([inputs.complex_normal(rng, N) for _ in range(B)]).reshape(B, N)
    if mag_range is not None:   # per-voxel magnitudes 10^U(-r, r)
        r = (r * (10.0 ** rng.uniform(-mag_range, mag_range, (B, N)))).astype(np.complex64)
    return r


def _forward(p, rho, d=None, **opts):
    from non_cartesian_mri_amd import fhd_forward
    d = d or dev_problem(p)
    r = torch.from_numpy(np.ascontiguousarray(rho)).to("cuda:0")
    out = fhd_forward(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], r, engine="mfma16", **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(rho.shape[0], p.M)


def _ref(oracle_mod, p, rho, idx=None):
    return oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho, idx=idx)


@pytest.fixture(scope="module")
def grid(oracle_mod):
    # 30,000 of the 32^3 voxels: 235 groups of 128 (the last partial), 8
    # chunks of 32 groups (the last partial); 1001 samples (a partial wave)
    p = inputs.random_problem(501, M=1001, L=32, N=30000)
    rho = _images(502, 1, p.N)
    return p, dev_problem(p), rho, _ref(oracle_mod, p, rho)


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("tile", [32, 64, 0, 1 << 20])
def test_grid(grid, trig, splits, tile):
    p, d, rho, ref = grid
    got = _forward(p, rho, d, trig=trig, tile=tile, sample_splits=splits)
    assert_close(got, ref, TOL[trig], f"half forward grid {trig} rows={splits} tile={tile}")


@pytest.mark.parametrize("trig", TRIGS)
def test_plain_sum(grid, trig):
    p, d, rho, ref = grid
    assert_close(_forward(p, rho, d, trig=trig, sum="plain"), ref, TOL[trig], f"half forward plain {trig}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("B", [2, 3, 16, 19])
def test_batch(oracle_mod, trig, B):
    p = inputs.random_problem(503, M=777, L=16)
    rho = _images(504, B, p.N)
    assert_close(_forward(p, rho, trig=trig), _ref(oracle_mod, p, rho), TOL[trig], f"half forward B={B} {trig}")


@pytest.mark.parametrize("trig", TRIGS)
def test_irregular_voxels(oracle_mod, trig):
    p = inputs.random_problem(505, M=900, L=12, N=1500, coords="random")
    rho = _images(506, 2, p.N)
    assert_close(_forward(p, rho, trig=trig), _ref(oracle_mod, p, rho), TOL[trig], f"half forward irregular {trig}")


@pytest.mark.parametrize("trig", TRIGS)
def test_one_displaced_voxel(oracle_mod, trig):
    p = inputs.random_problem(507, M=700, L=16)
    x = p.x.copy()
    x[1000] += np.float32(0.3)   # its group of 128 goes to the direct kernel, the others stay regular
    p.x = x
    rho = _images(508, 1, p.N)
    assert_close(_forward(p, rho, trig=trig), _ref(oracle_mod, p, rho), TOL[trig], f"half forward displaced {trig}")


def _rows(ys, nz, nx=128):
    """Voxel coordinates of x rows of nx voxels at the y values ys on nz planes."""
    iz, iy, ix = np.meshgrid(np.arange(nz), np.asarray(ys), np.arange(nx), indexing="ij")
    return tuple((a.ravel() - 8).astype(np.float32) for a in (ix, iy, iz))


def _rows_problem(seed, M, coords):
    rng = np.random.Generator(np.random.PCG64(seed))
    kx, ky, kz = inputs.uniform_k(M, rng)
    x, y, z = coords
    return inputs.Problem(f"rows{seed}", "fhd", kx, ky, kz, x, y, z, inputs.complex_normal(rng, M), None, seed)


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("ys,nz,nx,B", [(range(8), 5, 128, 1), (range(12), 3, 128, 1),
                                        ([0, 1, 2, 3, 4, 6, 7, 8, 9, 10, 11, 12, 15], 4, 128, 1),
                                        (range(8), 5, 128, 2), (range(12), 3, 128, 3), (range(9), 2, 512, 1),
                                        (range(10), 2, 256, 1), (range(6), 3, 256, 4)])
def test_octet_spacing(oracle_mod, trig, ys, nz, nx, B):
    """Voxels on x rows of nx.  A lane steps its phase over an octet of
    groups by rotations where the octet's bases are equally spaced; a chunk
    of 32 groups takes them in the order (stride 1, 2 or 4 over the chunk)
    that makes most octets so.  128-voxel groups: one per 128-row (8 rows per
    plane: every octet; 12 rows per plane or rows missing from the sequence:
    some octets, the others evaluated per group, in one wave), four per
    512-row and two per 256-row (stride 4 and 2, with a ragged plane end);
    two vectors: 64-voxel groups, two per 128-row; three: a pass of two and
    one; four: 32-voxel groups, eight per 256-row (no stride fits: evaluated
    per group)."""
    p = _rows_problem(521, 1500, _rows(list(ys), nz, nx=nx))
    rho = _images(522, B, p.N)
    assert_close(_forward(p, rho, trig=trig), _ref(oracle_mod, p, rho), TOL[trig],
                 f"half forward rows ys={list(ys)[:3]}... nz={nz} nx={nx} B={B} {trig}")


@pytest.mark.parametrize("N", [1, 3, 129])
def test_tiny_voxel_counts(oracle_mod, N):
    p = inputs.random_problem(509, M=321, L=16, N=N)
    rho = _images(510, 1, N)
    for trig in TRIGS:
        assert_close(_forward(p, rho, trig=trig), _ref(oracle_mod, p, rho), TOL[trig], f"half forward N={N} {trig}")


@pytest.mark.parametrize("M", [1, 15, 16, 17, 4099])
def test_sample_count_tails(oracle_mod, M):
    p = inputs.random_problem(511, M=M, L=8)
    rho = _images(512, 2, p.N)
    ref = _ref(oracle_mod, p, rho)
    for trig in TRIGS:
        assert_close(_forward(p, rho, trig=trig), ref, TOL[trig], f"half forward M={M} {trig}")


def test_zero_image():
    p = inputs.random_problem(513, M=200, L=8)
    got = _forward(p, np.zeros((1, p.N), np.complex64), trig="accurate")
    assert np.all(got == 0)


def test_wide_dynamic_range(oracle_mod):
    # |rho| over nine orders of magnitude: the parts' power-of-two scale puts
    # the largest entry near 2^14; the smallest fall to fp16 subnormals
    p = inputs.random_problem(514, M=1500, L=16)
    rho = _images(515, 1, p.N, mag_range=4.5)
    assert_close(_forward(p, rho, trig="accurate"), _ref(oracle_mod, p, rho), TOL["accurate"],
                 "half forward |rho| over 1e9")


@pytest.mark.parametrize("trig", TRIGS)
def test_full_size_sampled(oracle_mod, trig):
    """128^3 voxels x 262,144 stack-of-spirals samples in the default launch
    plan; the oracle evaluates 256 seeded samples."""
    p = inputs.make_config("fhd_128cube_262144_spirals")
    rho = _images(516, 1, p.N)
    idx = inputs.subset_indices(p.M, 256, p.seed)
    ref = _ref(oracle_mod, p, rho, idx=idx)
    print(f"[oracle] forward 128^3 x 256 samples: {oracle_mod.last.seconds:.1f}s", flush=True)
    got = _forward(p, rho, trig=trig)
    assert_close(got[:, idx], ref, TOL[trig], f"half forward 128^3 {trig}")


@pytest.mark.parametrize("trig", TRIGS)
def test_512cubed_sampled(oracle_mod, trig):
    """512^3 voxels x 262,144 spiral samples (rows of 1.6 GB of packed groups:
    tiles folded on both trig paths): 16 seeded samples against the oracle."""
    p = inputs.make_config("fhd_512cube_262144_spirals")
    rho = _images(523, 1, p.N)
    idx = inputs.subset_indices(p.M, 16, p.seed)
    ref = _ref(oracle_mod, p, rho, idx=idx)
    print(f"[oracle] forward 512^3 x 16 samples: {oracle_mod.last.seconds:.1f}s", flush=True)
    got = _forward(p, rho, trig=trig)
    assert_close(got[:, idx], ref, TOL[trig], f"half forward 512^3 {trig}")


def test_adjoint_of_half_fhd():
    """<F rho, D> = <rho, F^H D> with both sides on the half-split engine."""
    from tests.gpu_util import gpu_fhd
    p = inputs.random_problem(517, M=3000, L=16)
    d = dev_problem(p)
    rho = _images(518, 1, p.N)
    Frho = _forward(p, rho, d, trig="accurate")[0].astype(np.complex128)
    FHd = gpu_fhd(p, d, trig="accurate", engine="mfma16")[0].astype(np.complex128)
    lhs = np.vdot(Frho, p.D[0].astype(np.complex128))
    rhs = np.vdot(rho[0].astype(np.complex128), FHd)
    scale = np.linalg.norm(Frho) * np.linalg.norm(p.D[0])
    assert abs(lhs - rhs) <= TOL["accurate"] * scale, (lhs, rhs)


def test_deterministic():
    p = inputs.random_problem(519, M=2500, L=16)
    d = dev_problem(p)
    rho = _images(520, 1, p.N)
    a = _forward(p, rho, d, trig="hw")
    b = _forward(p, rho, d, trig="hw")
    assert np.array_equal(a.view(np.uint32), b.view(np.uint32))
