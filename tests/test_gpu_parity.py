"""GPU parity: the HIP path (through the C ABI) against the double-precision oracle.

Small problems are compared exhaustively; they span several workgroups,
several summation tiles and ragged tails in both the voxel and the sample
dimension.  Every trig path, summation mode and voxel-group size is covered,
for F^H D, batched F^H D and Q, on grid (factored phase) and non-grid (direct
phase) voxel sets, on both engines: the VALU kernels (selected here by an
explicit voxels_per_lane or Kahan summation) and the matrix-core kernels (the
default; their factored path needs groups of 32 / vectors voxels that line up
with the grid rows, other waves take the direct kernel).
"""
import numpy as np
import pytest
import torch

from non_cartesian_mri_amd import inputs
from tests.gpu_util import TOL, assert_close, dev_problem, gpu_fhd, gpu_q, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


TRIGS = ["accurate", "hw"]
SUMS = ["blocked", "kahan", "plain"]
VS = [1, 2, 4, 8, 16]


@pytest.fixture(scope="module")
def small_grid(oracle_mod):
    # 18^3 = 5832 voxels: not a multiple of 64*V; M = 1001 with 128-sample tiles
    p = inputs.random_problem(201, M=1001, L=18)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    qref = oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi)
    return p, dev_problem(p), ref, qref


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("sum_", SUMS)
@pytest.mark.parametrize("V", VS)
def test_fhd_small_grid(small_grid, trig, sum_, V):
    p, d, ref, _ = small_grid
    got = gpu_fhd(p, d, trig=trig, sum=sum_, voxels_per_lane=V, tile=128)
    assert_close(got, ref, TOL[trig], f"fhd grid {trig}/{sum_}/V={V}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("sum_", SUMS)
@pytest.mark.parametrize("V", VS)
def test_q_small_grid(small_grid, trig, sum_, V):
    p, d, _, qref = small_grid
    got = gpu_q(p, d, trig=trig, sum=sum_, voxels_per_lane=V, tile=128)
    assert_close(got, qref, TOL[trig], f"q grid {trig}/{sum_}/V={V}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("V", [1, 4, 8, 16])
def test_irregular_voxels(oracle_mod, trig, V):
    """Non-grid voxel centres: every wave takes the direct-phase path."""
    p = inputs.random_problem(202, M=777, N=3001, L=40, coords="random")
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    assert_close(gpu_fhd(p, trig=trig, voxels_per_lane=V), ref, TOL[trig], f"fhd irregular {trig}/V={V}")
    qref = oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi)
    assert_close(gpu_q(p, trig=trig, voxels_per_lane=V), qref, TOL[trig], f"q irregular {trig}/V={V}")


@pytest.mark.parametrize("trig", TRIGS)
def test_mixed_regular_and_irregular_waves(oracle_mod, trig):
    """A grid with a few displaced voxels: only the waves holding them go direct."""
    p = inputs.random_problem(203, M=600, L=24)
    x = p.x.copy()
    x[[100, 5000, 13823]] += np.float32(0.25)
    p.x = x
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    assert_close(gpu_fhd(p, trig=trig, voxels_per_lane=8), ref, TOL[trig], f"fhd mixed {trig}")
    qref = oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi)
    assert_close(gpu_q(p, trig=trig, voxels_per_lane=8), qref, TOL[trig], f"q mixed {trig}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("B", [2, 3, 5, 16, 19])
def test_batched(oracle_mod, trig, B):
    p = inputs.random_problem(204, M=513, L=10, B=B)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    assert_close(gpu_fhd(p, trig=trig), ref, TOL[trig], f"fhd batched {trig}/B={B}")


@pytest.mark.parametrize("trig", TRIGS)
def test_batch_rows_equal_single_calls_bitwise(trig):
    """VALU engine: row b of a batched call equals a single call on D[b] (same
    per-sample arithmetic: one voxel per lane in both), and permuting the data
    vectors of a batch permutes its output rows bit for bit (the vectors share
    one phase, sine and cosine per sample and keep their own sums)."""
    p = inputs.random_problem(205, M=300, L=8, B=16)
    d = dev_problem(p)
    full = gpu_fhd(p, d, trig=trig, engine="valu")
    for b in (0, 7, 15):
        q = inputs.Problem(p.name, "fhd", p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D[b:b + 1], p.seed)
        one = gpu_fhd(q, trig=trig, voxels_per_lane=1)
        assert np.array_equal(one[0], full[b])
    perm = np.random.Generator(np.random.PCG64(2051)).permutation(p.B)
    q = inputs.Problem(p.name, "fhd", p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, np.ascontiguousarray(p.D[perm]), p.seed)
    assert np.array_equal(gpu_fhd(q, trig=trig, engine="valu"), full[perm])


@pytest.mark.parametrize("trig", TRIGS)
def test_deterministic(trig):
    p = inputs.random_problem(206, M=2000, L=20)
    d = dev_problem(p)
    a = gpu_fhd(p, d, trig=trig)
    b = gpu_fhd(p, d, trig=trig)
    assert np.array_equal(a, b)
    qa, qb = gpu_q(p, d, trig=trig), gpu_q(p, d, trig=trig)
    assert np.array_equal(qa, qb)


@pytest.mark.parametrize("B,splits", [(1, 3), (3, 1), (3, 2)])
def test_split_stages_equal_one_call(B, splits):
    """mu / gather / reduce in separate calls give the one-call result bitwise
    (multi-pass batches with sample splits run gather and reduce together)."""
    from non_cartesian_mri_amd import fhd_compute, fhd_workspace_bytes
    p = inputs.random_problem(207, M=999, L=12, B=B)
    d = dev_problem(p)
    nb = fhd_workspace_bytes(p.M, p.N, p.B, sample_splits=splits)
    ws = torch.empty(nb, dtype=torch.uint8, device="cuda:0")
    args = (d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], d["D"])
    out = torch.empty((p.B, p.N), dtype=torch.complex64, device="cuda:0")
    steps = ["mu", "gather", "reduce"] if (B == 1 or splits == 1) else ["mu", "gather+reduce"]
    for st in steps:
        fhd_compute(*args, stages=st, workspace=ws, out=out, sample_splits=splits)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), gpu_fhd(p, d, sample_splits=splits))


def test_non_default_stream(oracle_mod):
    p = inputs.random_problem(208, M=400, L=10)
    d = dev_problem(p)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    from non_cartesian_mri_amd import fhd_compute
    with torch.cuda.stream(s):
        out = fhd_compute(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], d["D"])
    s.synchronize()
    assert_close(out.cpu().numpy().reshape(1, -1), ref, TOL["accurate"], "fhd side stream")


# ------------------------------ edge cases ---------------------------------
@pytest.mark.parametrize("trig", TRIGS)
def test_empty_sample_set_gives_zeros(trig):
    p = inputs.random_problem(209, M=0, L=6, B=2)
    got = gpu_fhd(p, trig=trig)
    assert got.shape == (2, 216) and np.all(got == 0)
    assert np.all(gpu_q(p, trig=trig) == 0)


def test_empty_voxel_set():
    from non_cartesian_mri_amd import fhd_compute, q_compute
    p = inputs.random_problem(210, M=50, L=4)
    d = dev_problem(p)
    e = torch.empty(0, dtype=torch.float32, device="cuda:0")
    out = fhd_compute(d["kx"], d["ky"], d["kz"], e, e, e, d["phi"], d["D"])
    assert out.numel() == 0
    assert q_compute(d["kx"], d["ky"], d["kz"], e, e, e, d["phi"]).numel() == 0


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("N", [1, 3, 5, 17])
def test_tiny_voxel_counts(oracle_mod, trig, N):
    """N below the group size: the group size shrinks; lanes past N stay idle."""
    p = inputs.random_problem(211, M=321, L=4, N=N)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    assert_close(gpu_fhd(p, trig=trig, voxels_per_lane=16), ref, TOL[trig], f"fhd N={N} {trig}")
    qref = oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi)
    assert_close(gpu_q(p, trig=trig, voxels_per_lane=16), qref, TOL[trig], f"q N={N} {trig}")


@pytest.mark.parametrize("trig", TRIGS)
def test_single_sample_at_k0(trig):
    """M=1, k=0: every voxel gets Mu = conj(phi) D (to within fp32 rounding of the packing)."""
    p = inputs.random_problem(212, M=1, L=8)
    p.kx, p.ky, p.kz = (np.zeros(1, np.float32) for _ in range(3))
    mu = np.conj(p.phi[0].astype(np.complex128)) * p.D[0, 0].astype(np.complex128)
    for V in (1, 8):
        got = gpu_fhd(p, trig=trig, voxels_per_lane=V)[0]
        assert np.max(np.abs(got - mu)) <= 2.5e-7 * abs(mu)
        assert np.all(got == got[0])
    w = abs(complex(p.phi[0])) ** 2
    gq = gpu_q(p, trig=trig)
    assert np.max(np.abs(gq - w)) <= 1.5e-7 * w


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("axis,k,base", [(0, 0.25, 1j), (1, 0.5, -1.0), (2, -0.25, -1j)])
def test_single_sample_plane_wave(trig, axis, k, base):
    """One sample on an axis with k.x a multiple of a quarter turn: base**x."""
    p = inputs.random_problem(213, M=1, L=8)
    kv = [np.zeros(1, np.float32) for _ in range(3)]
    kv[axis][0] = k
    p.kx, p.ky, p.kz = kv
    mu = np.conj(p.phi[0].astype(np.complex128)) * p.D[0, 0].astype(np.complex128)
    coord = (p.x, p.y, p.z)[axis].astype(np.int64)
    want = np.array([mu * base ** int(c) for c in coord])
    for V in (1, 4, 16):
        got = gpu_fhd(p, trig=trig, voxels_per_lane=V)[0]
        assert np.max(np.abs(got - want)) <= 1e-6 * abs(mu), (V, np.max(np.abs(got - want)))


@pytest.mark.parametrize("M", [3, 4, 5, 127, 128, 129, 4099])
def test_sample_count_tails(oracle_mod, M):
    """Sample counts around the unroll step and the tile size (tile=128)."""
    p = inputs.random_problem(214, M=M, L=9)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    for trig in TRIGS:
        assert_close(gpu_fhd(p, trig=trig, tile=128), ref, TOL[trig], f"fhd M={M} {trig}")


def test_voxel_at_origin_sums_mu():
    p = inputs.random_problem(215, M=5000, L=8)
    got = gpu_fhd(p)[0]
    o = np.nonzero((p.x == 0) & (p.y == 0) & (p.z == 0))[0][0]
    want = np.sum(np.conj(p.phi.astype(np.complex128)) * p.D[0].astype(np.complex128))
    assert abs(got[o] - want) <= 1e-5 * np.sqrt(np.sum(np.abs(p.phi.astype(np.complex128) * p.D[0]) ** 2))


def test_permutation_invariance_within_tolerance():
    p = inputs.random_problem(216, M=3000, L=12)
    a = gpu_fhd(p)
    perm = np.random.Generator(np.random.PCG64(5)).permutation(p.M)
    q = inputs.Problem(p.name, "fhd", p.kx[perm], p.ky[perm], p.kz[perm], p.x, p.y, p.z,
                       p.phi[perm], p.D[:, perm], p.seed)
    b = gpu_fhd(q)
    assert np.linalg.norm(a - b) <= 1e-5 * np.linalg.norm(a)


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("sum_", ["blocked", "kahan"])
@pytest.mark.parametrize("V", [1, 16])
@pytest.mark.parametrize("splits", [1, 2, 5])
def test_sample_splits(small_grid, trig, sum_, V, splits):
    """Samples split across launch rows (partial sums + fixed-order reduction);
    1001 samples pad to 1004, so 5 rows get 204, 204, 204, 204 and 188."""
    p, d, ref, qref = small_grid
    got = gpu_fhd(p, d, trig=trig, sum=sum_, voxels_per_lane=V, tile=64, sample_splits=splits)
    assert_close(got, ref, TOL[trig], f"fhd splits={splits} {trig}/{sum_}/V={V}")
    gq = gpu_q(p, d, trig=trig, sum=sum_, voxels_per_lane=V, tile=64, sample_splits=splits)
    assert_close(gq, qref, TOL[trig], f"q splits={splits} {trig}/{sum_}/V={V}")
    again = gpu_fhd(p, d, trig=trig, sum=sum_, voxels_per_lane=V, tile=64, sample_splits=splits)
    assert np.array_equal(got, again)


@pytest.mark.parametrize("splits", [1, 3])
def test_batched_sample_splits(oracle_mod, splits):
    """Batch passes of 16 and 2 vectors share one partial-sum buffer."""
    p = inputs.random_problem(217, M=900, L=9, B=18)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    assert_close(gpu_fhd(p, trig="hw", sample_splits=splits), ref, TOL["hw"], f"batched splits={splits}")


# ------------------------- matrix-core engine ------------------------------
# Grids whose rows hold whole groups of 32 / vectors voxels run the factored
# MFMA path; 30000 of the 32^3 voxels leave a partial last wave and group.
@pytest.fixture(scope="module")
def mfma_grid(oracle_mod):
    p = inputs.random_problem(301, M=1001, L=32, N=30000)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    qref = oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi)
    return p, dev_problem(p), ref, qref


# MFMA group sizes of single-vector passes: T = 2, 4 (two samples per
# 32x32x2 MFMA) and 8 (four samples per 16x16x4 MFMA)
GROUPS = [32, 64, 128]


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("sum_", ["blocked", "plain"])
@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("G", GROUPS)
def test_mfma_grid(mfma_grid, trig, sum_, splits, G):
    p, d, ref, qref = mfma_grid
    opts = dict(trig=trig, sum=sum_, tile=128, sample_splits=splits, engine="mfma", voxels_per_lane=G)
    assert_close(gpu_fhd(p, d, **opts), ref, TOL[trig], f"mfma fhd {trig}/{sum_}/splits={splits}/G={G}")
    assert_close(gpu_q(p, d, **opts), qref, TOL[trig], f"mfma q {trig}/{sum_}/splits={splits}/G={G}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("B", [2, 4, 8, 16, 19])
@pytest.mark.parametrize("G", GROUPS)
def test_mfma_batched_grid(oracle_mod, trig, B, G):
    """Batch passes of 16/8/4/2/1 vectors: groups of G/16 ... G voxels, each a
    whole number of the 16-voxel rows or a divisor of them."""
    p = inputs.random_problem(302, M=700, L=16, B=B)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    assert_close(gpu_fhd(p, trig=trig, engine="mfma", tile=96, voxels_per_lane=G), ref, TOL[trig],
                 f"mfma batched {trig}/B={B}/G={G}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("splits", [1, 4])
@pytest.mark.parametrize("G", GROUPS)
def test_mfma_irregular_voxels(oracle_mod, trig, splits, G):
    """Non-grid voxel centres: every wave runs the direct kernel (partial row 0
    carries its totals, the other rows zeros)."""
    p = inputs.random_problem(303, M=777, N=3001, L=40, coords="random", B=3)
    opts = dict(trig=trig, engine="mfma", sample_splits=splits, voxels_per_lane=G)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    assert_close(gpu_fhd(p, **opts), ref, TOL[trig], f"mfma fhd irregular {trig}/splits={splits}/G={G}")
    qref = oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi)
    assert_close(gpu_q(p, **opts), qref, TOL[trig], f"mfma q irregular {trig}/splits={splits}/G={G}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("splits", [1, 3])
@pytest.mark.parametrize("G", GROUPS)
def test_mfma_mixed_regular_and_irregular_waves(oracle_mod, trig, splits, G):
    """A 32^3 grid with displaced voxels in three waves: those go direct, the
    others through the matrix cores, and both write the same partial rows."""
    p = inputs.random_problem(304, M=600, L=32)
    x = p.x.copy()
    x[[100, 5000, 32767]] += np.float32(0.25)
    p.x = x
    opts = dict(trig=trig, engine="mfma", sample_splits=splits, voxels_per_lane=G)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    assert_close(gpu_fhd(p, **opts), ref, TOL[trig], f"mfma fhd mixed {trig}/splits={splits}/G={G}")
    qref = oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi)
    assert_close(gpu_q(p, **opts), qref, TOL[trig], f"mfma q mixed {trig}/splits={splits}/G={G}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("N", [1, 3, 31, 33, 65, 1000])
@pytest.mark.parametrize("G", GROUPS)
def test_mfma_tiny_and_ragged_voxel_counts(oracle_mod, trig, N, G):
    """Fewer voxels than one group (unused columns are never written) and
    partial groups and waves."""
    p = inputs.random_problem(305, M=321, L=16, N=N)
    opts = dict(trig=trig, engine="mfma", voxels_per_lane=G)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    assert_close(gpu_fhd(p, **opts), ref, TOL[trig], f"mfma fhd N={N} {trig}/G={G}")
    qref = oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi)
    assert_close(gpu_q(p, **opts), qref, TOL[trig], f"mfma q N={N} {trig}/G={G}")


@pytest.mark.parametrize("M", [1, 31, 32, 33, 63, 65, 4099])
@pytest.mark.parametrize("G", GROUPS)
def test_mfma_sample_count_tails(oracle_mod, M, G):
    """Sample counts around the 32-sample chunk and the 64-sample tile."""
    p = inputs.random_problem(306, M=M, L=8)
    ref = oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)
    for trig in TRIGS:
        assert_close(gpu_fhd(p, trig=trig, engine="mfma", tile=64, voxels_per_lane=G), ref, TOL[trig],
                     f"mfma fhd M={M} {trig}/G={G}")


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("G", GROUPS)
def test_mfma_plane_waves_and_k0(trig, G):
    """One sample at k = 0 gives Mu everywhere; on an axis at a quarter-turn k
    the result is Mu * base**x (factored path on the 16^3 grid)."""
    p = inputs.random_problem(307, M=1, L=16)
    mu = np.conj(p.phi[0].astype(np.complex128)) * p.D[0, 0].astype(np.complex128)
    p.kx, p.ky, p.kz = (np.zeros(1, np.float32) for _ in range(3))
    got = gpu_fhd(p, trig=trig, engine="mfma", voxels_per_lane=G)[0]
    assert np.max(np.abs(got - mu)) <= 2.5e-7 * abs(mu)
    assert np.all(got == got[0])
    for axis, k, base in ((0, 0.25, 1j), (1, 0.5, -1.0), (2, -0.25, -1j)):
        kv = [np.zeros(1, np.float32) for _ in range(3)]
        kv[axis][0] = k
        p.kx, p.ky, p.kz = kv
        coord = (p.x, p.y, p.z)[axis].astype(np.int64)
        want = np.array([mu * base ** int(c) for c in coord])
        got = gpu_fhd(p, trig=trig, engine="mfma", voxels_per_lane=G)[0]
        assert np.max(np.abs(got - want)) <= 1e-6 * abs(mu), (axis, np.max(np.abs(got - want)))


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("G", GROUPS)
def test_mfma_deterministic_and_engines_agree(trig, G):
    p = inputs.random_problem(308, M=2000, L=32, B=2)
    d = dev_problem(p)
    a = gpu_fhd(p, d, trig=trig, engine="mfma", voxels_per_lane=G)
    assert np.array_equal(a, gpu_fhd(p, d, trig=trig, engine="mfma", voxels_per_lane=G))
    v = gpu_fhd(p, d, trig=trig, engine="valu")
    assert np.linalg.norm(a - v) <= TOL[trig] * np.linalg.norm(v)


@pytest.mark.parametrize("trig", TRIGS)
@pytest.mark.parametrize("splits", [1, 3])
def test_mfma4_row_block_and_folded_tiles(mfma_grid, trig, splits):
    """Four-sample engine: a tile as long as the launch row takes the kernel
    without running totals (each row one summation block); shorter tiles fold
    into totals.  Both match the oracle, F^H D and Q."""
    p, d, ref, qref = mfma_grid
    base = dict(trig=trig, engine="mfma", voxels_per_lane=128, sample_splits=splits)
    for tile in (64, 8192):   # 8192 >= every row of the 1001 samples
        assert_close(gpu_fhd(p, d, tile=tile, **base), ref, TOL[trig], f"fhd {trig} rows={splits} tile={tile}")
        assert_close(gpu_q(p, d, tile=tile, **base), qref, TOL[trig], f"q {trig} rows={splits} tile={tile}")


def test_kahan_folds_hold_a_coherent_sum(oracle_mod):
    """Q at x = 0 is the coherent sum sum_m |phi_m|^2 (its closed form).  With
    2^22 samples summed on one lane (VALU engine, one launch row, tiles of 64
    samples) a single running fp32 sum drifts far past the 1e-5 bar; blocked
    summation folds 65,536 tile sums in plain fp32; Kahan-compensated folds
    keep the total within 1e-6 and below the blocked error.  The other voxels
    (incoherent sums) are checked against the oracle."""
    from non_cartesian_mri_amd import q_compute
    M = 1 << 22
    rng = np.random.Generator(np.random.PCG64(1000))
    kx, ky, kz = inputs.uniform_k(M, rng)
    phi = inputs.complex_normal(rng, M)
    x = np.array([0.0, 1.0, -3.0, 7.0], np.float32)
    y = np.array([0.0, 2.0, 1.0, -5.0], np.float32)
    z = np.array([0.0, -1.0, 5.0, 2.0], np.float32)
    exact = float(np.sum(np.abs(phi.astype(np.complex128)) ** 2))
    ref = oracle_mod.q(kx, ky, kz, x, y, z, phi)
    assert abs(ref[0] - exact) <= 1e-12 * exact
    t = [torch.from_numpy(a).to("cuda:0") for a in (kx, ky, kz, x, y, z, phi)]
    err = {}
    for sum_ in ("plain", "blocked", "kahan"):
        got = q_compute(*t, trig="accurate", sum=sum_, engine="valu", voxels_per_lane=1,
                        sample_splits=1, tile=64)
        torch.cuda.synchronize()
        got = got.cpu().numpy()
        err[sum_] = abs(complex(got[0]) - exact) / exact
        print(f"[kahan] Q(0) of 2^22 samples, {sum_}: rel err {err[sum_]:.3e}", flush=True)
        if sum_ == "kahan":
            assert_close(got, ref, TOL["accurate"], "Q kahan 2^22 samples")
    assert err["plain"] > 1e-5
    assert err["kahan"] < 1e-6
    assert err["kahan"] < err["blocked"]


def test_row_block_sum_of_a_coherent_sum(oracle_mod):
    """The matrix-core engine's HW path sums a whole launch row as one block
    (no tile folds); the longest rows the planner makes are the 512^3
    adjoint's 131,072 samples.  Q(0) = sum |phi|^2 over two such rows on a 32^3
    grid stays within the accurate path's bar, and the grid matches the
    oracle within the HW bar."""
    from non_cartesian_mri_amd import fhd_describe_plan, q_compute
    M = 262144
    rng = np.random.Generator(np.random.PCG64(2000))
    kx, ky, kz = inputs.uniform_k(M, rng)
    phi = inputs.complex_normal(rng, M)
    x, y, z = inputs.voxel_grid(32)
    opts = dict(trig="hw", engine="mfma", voxels_per_lane=128, sample_splits=2)
    plan = fhd_describe_plan(M, x.size, 1, is_q=True, **opts)
    assert plan["tile"] == 131072 and plan["sample_splits"] == 2
    t = [torch.from_numpy(a).to("cuda:0") for a in (kx, ky, kz, x, y, z, phi)]
    got = q_compute(*t, **opts)
    torch.cuda.synchronize()
    got = got.cpu().numpy()
    o = int(np.nonzero((x == 0) & (y == 0) & (z == 0))[0][0])
    exact = float(np.sum(np.abs(phi.astype(np.complex128)) ** 2))
    e0 = abs(complex(got[o]) - exact) / exact
    print(f"[row-block] Q(0), two rows of 131,072 samples: rel err {e0:.3e}", flush=True)
    assert e0 <= TOL["accurate"]
    idx = inputs.subset_indices(x.size, 2048, 2001)
    ref = oracle_mod.q(kx, ky, kz, x, y, z, phi, idx=idx)
    assert_close(got[idx], ref, TOL["hw"], "Q row-block hw 32^3")
