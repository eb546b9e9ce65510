"""GPU parity of the forward operator F rho (fhd_forward, through the C ABI)
against the double-precision oracle, plus its adjointness with fhd_compute.

Grids whose rows hold whole voxel groups (32 or 64 voxels) run the
matrix-core path; non-grid coordinates and displaced voxels take the direct
kernel for their groups.  Sizes span several waves of 32 samples, several
32-group chunks and summation tiles, with ragged samples and groups.
"""
import numpy as np
import pytest
import torch

from non_cartesian_mri_amd import inputs
from tests.gpu_util import TOL, assert_close, dev_problem, require_gpu

pytestmark = pytest.mark.gpu

TRIGS = ["accurate", "hw"]
GROUPS = [32, 64, 128]   # 128: the four-group engine (16x16x4, K = four groups)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _images(seed, B, N):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.stack([inputs.complex_normal(rng, N) for _ in range(B)]).reshape(B, N)


def gpu_forward(p, rho, d=None, **opts) -> np.ndarray:
    from non_cartesian_mri_amd import fhd_forward
    d = d or dev_problem(p)
    r = torch.from_numpy(np.ascontiguousarray(rho)).to("cuda:0")
    out = fhd_forward(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], r, **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(rho.shape[0], p.M)


@pytest.fixture(scope="module")
def fwd_grid(oracle_mod):
    # 30,000 of the 32^3 voxels (a partial last group and wave of groups), 1001 samples
    p = inputs.random_problem(401, M=1001, L=32, N=30000)
    rho = _images(402, 1, p.N)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    return p, dev_problem(p), rho, ref


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("sum_", ["blocked", "plain"])
@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("G", GROUPS)
def test_forward_grid(fwd_grid, trig, sum_, splits, G):
    p, d, rho, ref = fwd_grid
    got = gpu_forward(p, rho, d, trig=trig, sum=sum_, tile=64, sample_splits=splits, voxels_per_lane=G)
    assert_close(got, ref, TOL[trig], f"forward grid {trig}/{sum_}/splits={splits}/G={G}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("B", [2, 3, 16, 19])
@pytest.mark.parametrize("G", GROUPS)
def test_forward_batched(oracle_mod, trig, B, G):
    """Passes of 16/8/4/2/1 images: groups of G * (vectors in the pass) / 16 ... voxels."""
    p = inputs.random_problem(403, M=650, L=16)
    rho = _images(404, B, p.N)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    assert_close(gpu_forward(p, rho, trig=trig, voxels_per_lane=G, tile=64), ref, TOL[trig],
                 f"forward batched {trig}/B={B}/G={G}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("splits", [1, 3])
def test_forward_irregular_voxels(oracle_mod, trig, splits):
    """Non-grid voxel centres: every group goes through the direct kernel."""
    p = inputs.random_problem(405, M=777, N=3001, L=40, coords="random")
    rho = _images(406, 2, p.N)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    assert_close(gpu_forward(p, rho, trig=trig, sample_splits=splits), ref, TOL[trig],
                 f"forward irregular {trig}/splits={splits}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("G", GROUPS)
def test_forward_mixed_groups(oracle_mod, trig, splits, G):
    """A 32^3 grid with three displaced voxels: their groups are evaluated
    directly and added after the matrix-core rows are reduced."""
    p = inputs.random_problem(407, M=600, L=32)
    x = p.x.copy()
    x[[100, 5000, 32767]] += np.float32(0.25)
    p.x = x
    rho = _images(408, 1, p.N)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    assert_close(gpu_forward(p, rho, trig=trig, sample_splits=splits, voxels_per_lane=G), ref,
                 TOL[trig], f"forward mixed {trig}/splits={splits}/G={G}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("N", [1, 3, 33, 65, 1000])
def test_forward_tiny_and_ragged_voxel_counts(oracle_mod, trig, N):
    p = inputs.random_problem(409, M=321, L=16, N=N)
    rho = _images(410, 1, N)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    assert_close(gpu_forward(p, rho, trig=trig), ref, TOL[trig], f"forward N={N} {trig}")


@pytest.mark.parametrize("M", [1, 31, 32, 33, 65, 4099])
def test_forward_sample_count_tails(oracle_mod, M):
    p = inputs.random_problem(411, M=M, L=8)
    rho = _images(412, 2, p.N)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    for trig in TRIGS:
        assert_close(gpu_forward(p, rho, trig=trig), ref, TOL[trig], f"forward M={M} {trig}")


def test_forward_empty_sets():
    from non_cartesian_mri_amd import fhd_forward
    p = inputs.random_problem(413, M=50, L=4)
    d = dev_problem(p)
    e = torch.empty(0, dtype=torch.float32, device="cuda:0")
    er = torch.empty((2, 0), dtype=torch.complex64, device="cuda:0")
    out = torch.full((2, p.M), 7.0 + 7.0j, dtype=torch.complex64, device="cuda:0")
    got = fhd_forward(d["kx"], d["ky"], d["kz"], e, e, e, d["phi"], er, out=out)
    torch.cuda.synchronize()
    assert np.all(got.cpu().numpy() == 0)  # empty voxel set: zero data
    ek = torch.empty(0, dtype=torch.float32, device="cuda:0")
    ep = torch.empty(0, dtype=torch.complex64, device="cuda:0")
    r = torch.from_numpy(_images(414, 1, p.N)[0]).to("cuda:0")
    assert fhd_forward(ek, ek, ek, d["x"], d["y"], d["z"], ep, r).numel() == 0


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("G", GROUPS)
def test_forward_closed_forms(trig, G):
    """k = 0: phi * sum(rho); k on an axis at a quarter turn with a one-voxel
    image at integer c: phi * rho * (-i)^(j c)."""
    p = inputs.random_problem(415, M=5, L=16)
    rho = _images(416, 1, p.N)
    p.kx, p.ky, p.kz = (np.zeros(p.M, np.float32) for _ in range(3))
    got = gpu_forward(p, rho, trig=trig, voxels_per_lane=G)[0]
    want = p.phi.astype(np.complex128) * np.sum(rho[0].astype(np.complex128))
    assert np.max(np.abs(got - want)) <= 2e-6 * np.max(np.abs(want))
    for axis in range(3):
        kv = [np.zeros(p.M, np.float32) for _ in range(3)]
        kv[axis] = (np.arange(p.M) / 4.0).astype(np.float32)
        p.kx, p.ky, p.kz = kv
        img = np.zeros((1, p.N), np.complex64)
        n = 3 * 16 * 16 + 2 * 16 + 11   # voxel (ix, iy, iz) = (11, 2, 3)
        img[0, n] = 0.5 - 1.5j
        c = int((p.x, p.y, p.z)[axis][n])
        got = gpu_forward(p, img, trig=trig, voxels_per_lane=G)[0]
        want = np.array([p.phi[j].astype(np.complex128) * (0.5 - 1.5j) * (-1j) ** (j * c) for j in range(p.M)])
        assert np.max(np.abs(got - want)) <= 1e-6 * np.max(np.abs(want)), (axis, G)


@pytest.mark.parametrize("trig", TRIGS)
def test_forward_is_the_adjoint_of_fhd(trig):
    """<F rho, d> = <rho, F^H d> with both sides computed on the GPU."""
    from tests.gpu_util import gpu_fhd
    p = inputs.random_problem(417, M=3000, L=32)
    d = dev_problem(p)
    rho = _images(418, 1, p.N)
    Frho = gpu_forward(p, rho, d, trig=trig)[0].astype(np.complex128)
    FHd = gpu_fhd(p, d, trig=trig)[0].astype(np.complex128)
    lhs = np.vdot(Frho, p.D[0].astype(np.complex128))
    rhs = np.vdot(rho[0].astype(np.complex128), FHd)
    scale = np.linalg.norm(Frho) * np.linalg.norm(p.D[0])
    assert abs(lhs - rhs) <= TOL[trig] * scale, (lhs, rhs)


@pytest.mark.parametrize("trig", TRIGS)
def test_forward_deterministic_and_stages(trig):
    from non_cartesian_mri_amd import fhd_forward, fhd_workspace_bytes
    p = inputs.random_problem(419, M=999, L=32)
    d = dev_problem(p)
    rho = _images(420, 3, p.N)
    a = gpu_forward(p, rho, d, trig=trig, sample_splits=2)
    assert np.array_equal(a, gpu_forward(p, rho, d, trig=trig, sample_splits=2))
    # pack / gather+reduce in separate calls on one workspace give the same result
    nb = fhd_workspace_bytes(p.M, p.N, 3, op="forward", trig=trig, sample_splits=2)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    r = torch.from_numpy(rho).to("cuda:0")
    out = torch.empty((3, p.M), dtype=torch.complex64, device="cuda:0")
    args = (d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], r)
    for st in ("mu", "gather+reduce"):
        fhd_forward(*args, trig=trig, stages=st, workspace=ws, out=out, sample_splits=2)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), a)


def test_forward_side_stream(oracle_mod):
    from non_cartesian_mri_amd import fhd_forward
    p = inputs.random_problem(421, M=400, L=16)
    d = dev_problem(p)
    rho = _images(422, 1, p.N)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    r = torch.from_numpy(rho[0]).to("cuda:0")
    with torch.cuda.stream(s):
        out = fhd_forward(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], r)
    s.synchronize()
    assert_close(out.cpu().numpy().reshape(1, -1), ref, TOL["accurate"], "forward side stream")


@pytest.mark.parametrize("trig", TRIGS)
def test_forward_full_size_sampled(oracle_mod, trig):
    """128^3 voxels x 262,144 stack-of-spirals samples in the benchmark's launch
    configuration; the oracle evaluates 256 seeded samples."""
    p = inputs.make_config("fhd_128cube_262144_spirals")
    rho = _images(423, 1, p.N)
    idx = inputs.subset_indices(p.M, 256, p.seed)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho, idx=idx)
    print(f"[oracle] forward 128^3 x 256 samples: {oracle_mod.last.seconds:.1f}s", flush=True)
    got = gpu_forward(p, rho, trig=trig)
    assert_close(got[:, idx], ref, TOL[trig], f"forward 128^3 {trig}")


@pytest.mark.parametrize("trig", TRIGS)
def test_forward_512cubed_sampled(oracle_mod, trig):
    """512^3 voxels (134M) x 262,144 spiral samples: 16 seeded samples against the oracle."""
    p = inputs.make_config("fhd_512cube_262144_spirals")
    rho = _images(424, 1, p.N)
    idx = inputs.subset_indices(p.M, 16, p.seed)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho, idx=idx)
    print(f"[oracle] forward 512^3 x 16 samples: {oracle_mod.last.seconds:.1f}s", flush=True)
    got = gpu_forward(p, rho, trig=trig)
    assert_close(got[:, idx], ref, TOL[trig], f"forward 512^3 {trig}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("B", [1, 3])
def test_forward_four_group_row_block_and_folded_tiles(oracle_mod, fwd_grid, trig, splits, B):
    """Four-group engine (groups of 128): a tile that spans the launch row
    takes the kernel without running totals; shorter tiles fold into totals.
    One vector, and three (passes of two and one: each half of the G block
    then holds whole vectors)."""
    p, d, rho1, ref1 = fwd_grid
    if B == 1:
        rho, ref = rho1, ref1
    else:
        rho = _images(403, B, p.N)
        ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    for tile in (32, 1 << 20):
        got = gpu_forward(p, rho, d, trig=trig, tile=tile, sample_splits=splits, voxels_per_lane=128)
        assert_close(got, ref, TOL[trig], f"forward G=128 {trig} B={B} rows={splits} tile={tile}")
