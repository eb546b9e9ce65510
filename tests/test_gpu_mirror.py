"""GPU parity of the mirror-pair gather (four-sample matrix-core engine, both
trig paths; launch rows summed in blocks of the plan's tile, at most 16,384
samples on the HW path) against the double-precision oracle.

The pairing rests on e^{-i2 pi k.x} = conj e^{i2 pi k.x} for real k and x (the
phase of PMPP ch. 17 Eq. 17.1): a voxel group whose reference voxel (column
V / 2) is the negated reference of another group gets its sums from the same
phase and factors.  The tests use box grids x fastest, rows of 128 voxels
along x from -64 to 63, and y / z ranges chosen so that some rows have a
mirror row (-y, -z), one row is its own mirror (y = z = 0) and some have none;
they check
  - the outputs against the oracle and against the same call with pairing off;
  - the pair plan the device wrote (read back from the caller's workspace):
    the number of pairs and of groups summed alone equals the count from the
    coordinates;
  - batched passes (groups of 64, 32 and 8 voxels: several groups per row,
    each mirrored onto another segment of the mirror row), Q, ragged voxel
    counts (a partial last group, a last group without its reference voxel),
    a displaced voxel, a grid without mirrors (half-integer coordinates),
    plain sums, fixed and device-chosen launch rows, separate stages, sample
    count tails and bitwise repeatability.
"""
import dataclasses

import numpy as np
import pytest
import torch

from non_cartesian_mri_amd import inputs
from tests.gpu_util import TOL, assert_close, dev_problem, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _box(xs, ys, zs):
    """Voxel centres of the box xs x ys x zs, x fastest."""
    X, Y, Z = np.meshgrid(np.asarray(xs, np.float32), np.asarray(ys, np.float32), np.asarray(zs, np.float32),
                          indexing="ij")
    return tuple(np.ascontiguousarray(a.transpose(2, 1, 0).ravel()) for a in (X, Y, Z))


def _problem(seed, M, xs, ys, zs, B=1, N=None, kind="fhd"):
    p = inputs.random_problem(seed, M=M, N=8, coords="random", L=8, B=B, kind=kind)
    x, y, z = _box(xs, ys, zs)
    if N is not None:
        x, y, z = x[:N], y[:N], z[:N]
    return dataclasses.replace(p, x=x, y=y, z=z)


def _run(p, d, ws=None, **opts):
    from non_cartesian_mri_amd import fhd_compute, q_compute
    opts.setdefault("engine", "mfma")
    opts.setdefault("voxels_per_lane", 128)
    opts.setdefault("trig", "hw")
    if p.kind == "q":
        out = q_compute(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], workspace=ws, **opts)
    else:
        out = fhd_compute(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], d["D"], workspace=ws, **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(-1, p.x.size)


def _plan_header(p, d, **opts):
    """Runs with a caller workspace and returns the pair plan's header."""
    from non_cartesian_mri_amd.fhd import fhd_describe_plan, fhd_workspace_bytes
    o = dict(engine="mfma", voxels_per_lane=128, trig="hw")
    o.update(opts)
    B = 1 if p.kind == "q" else p.D.shape[0]
    info = fhd_describe_plan(p.kx.size, p.x.size, B, p.kind == "q", **o)
    assert info["mirror_pairs"] == 1
    nbytes = fhd_workspace_bytes(p.kx.size, p.x.size, B, p.kind == "q", **o)
    V = info["voxels_per_lane"]
    G = -(-p.x.size // V)
    pair_bytes = ((64 + 8 * G + 15) // 16 * 16 + 16 * G + 255) // 256 * 256
    ws = torch.zeros(nbytes, dtype=torch.uint8, device="cuda:0")
    out = _run(p, d, ws, **opts)
    head = ws[nbytes - pair_bytes:nbytes - pair_bytes + 64].view(torch.int32).cpu().numpy()
    return out, head


def _oracle(oracle_mod, p):
    if p.kind == "q":
        return oracle_mod.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi)
    return oracle_mod.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D)


XS = np.arange(-64, 64)


def _expected_pairs(ys, zs, segs=1):
    """(pairs, alone) among the groups of the box's rows (y, z), `segs` groups per
    row: segment q of a row mirrors segment segs - 1 - q of row (-y, -z), so the
    row y = z = 0 pairs its own segments when it has more than one."""
    rows = {(y, z) for y in ys for z in zs}
    pairs = sum(1 for (y, z) in rows if (-y, -z) in rows and (y, z) != (-y, -z)) // 2 * segs
    if (0, 0) in rows:
        pairs += segs // 2
    return pairs, len(rows) * segs - 2 * pairs


@pytest.mark.parametrize("trig", ["hw", "accurate"])
@pytest.mark.parametrize("kind", ["fhd", "q"])
def test_pairs_on_an_asymmetric_box(oracle_mod, kind, trig):
    """y from -5 to 4, z from -3 to 3: 31 mirror pairs, the 7 rows at y = -5 and
    the row y = z = 0 alone; 70 groups in 5 waves (the last one partial)."""
    ys, zs = np.arange(-5, 5), np.arange(-3, 4)
    p = _problem(901, 1500, XS, ys, zs, kind=kind)
    d = dev_problem(p)
    ref = _oracle(oracle_mod, p)
    got, head = _plan_header(p, d, trig=trig)
    pairs, alone = _expected_pairs(ys, zs)
    assert (pairs, alone) == (31, 8)
    assert head[1] == pairs and head[0] == pairs + alone, head[:8]
    assert_close(got, ref, TOL[trig], f"mirror pairs {kind} {trig}")
    off = _run(p, d, mirror_pairs=False, trig=trig)
    assert_close(off, ref, TOL[trig], f"pairing off {kind} {trig}")
    # same phases up to the conjugation: the two paths agree far below the HW bar
    assert np.linalg.norm(got - off) <= 1e-5 * np.linalg.norm(off)


@pytest.mark.parametrize("trig", ["hw", "accurate"])
@pytest.mark.parametrize("B", [2, 4, 16, 19])
def test_pairs_in_batched_passes(oracle_mod, B, trig):
    """Passes of 16/4/2/1 vectors: groups of 8, 32, 64 and 128 voxels, 16 to 1
    groups per row, each mirrored onto the mirror row's opposite segment."""
    ys, zs = np.arange(-3, 3), np.arange(-2, 3)
    p = _problem(902 + B, 700, XS, ys, zs, B=B)
    d = dev_problem(p)
    ref = _oracle(oracle_mod, p)
    assert_close(_run(p, d, trig=trig), ref, TOL[trig], f"mirror pairs batched B={B} {trig}")


def test_pair_counts_with_several_groups_per_row(oracle_mod):
    """Two vectors: groups of 64 voxels, two per row; segment q of row (y, z)
    mirrors segment 1 - q of row (-y, -z)."""
    ys, zs = np.arange(-2, 3), np.arange(-2, 2)
    p = _problem(903, 600, XS, ys, zs, B=2)
    d = dev_problem(p)
    got, head = _plan_header(p, d)
    pairs, alone = _expected_pairs(ys, zs, segs=2)
    assert head[1] == pairs and head[0] == pairs + alone, head[:8]
    assert_close(got, _oracle(oracle_mod, p), TOL["hw"], "mirror pairs, two groups per row")


@pytest.mark.parametrize("trig", ["hw", "accurate"])
@pytest.mark.parametrize("N", [70 * 128 - 50, 70 * 128 - 70, 69 * 128 + 1])
def test_ragged_voxel_counts(oracle_mod, N, trig):
    """A partial last group that holds its reference voxel (summed alone), and
    last groups without it (their wave goes to the direct kernel)."""
    p = _problem(904, 900, XS, np.arange(-5, 5), np.arange(-3, 4), N=N)
    d = dev_problem(p)
    assert_close(_run(p, d, trig=trig), _oracle(oracle_mod, p), TOL[trig], f"mirror pairs N={N} {trig}")


def test_displaced_voxel_and_no_mirrors(oracle_mod):
    """One displaced voxel sends its wave to the direct kernel; a grid of
    half-integer coordinates has no mirror reference at all (every group alone)."""
    p = _problem(905, 800, XS, np.arange(-4, 4), np.arange(-2, 3))
    x = p.x.copy()
    x[5 * 128 + 17] += 0.25
    p = dataclasses.replace(p, x=x)
    d = dev_problem(p)
    assert_close(_run(p, d), _oracle(oracle_mod, p), TOL["hw"], "displaced voxel")
    q = _problem(906, 800, XS + 0.5, np.arange(-4, 4) + 0.5, np.arange(-2, 2) + 0.5)
    dq = dev_problem(q)
    got, head = _plan_header(q, dq)
    assert head[1] == 0 and head[0] == q.x.size // 128, head[:8]
    assert_close(got, _oracle(oracle_mod, q), TOL["hw"], "no mirrors")


@pytest.mark.parametrize("opts", [dict(sum="plain"), dict(sample_splits=3), dict(sample_splits=1),
                                  dict(sample_splits=7), dict(tile=96), dict(tile=96, sample_splits=2),
                                  dict(trig="accurate", sum="plain"), dict(trig="accurate", tile=2048),
                                  dict(trig="accurate", sample_splits=3)])
def test_row_choices(oracle_mod, opts):
    """Plain sums (one block per row), fixed and device-chosen rows, blocks
    shorter than a row (tile) on both trig paths."""
    p = _problem(907, 2100, XS, np.arange(-3, 4), np.arange(-3, 3))
    d = dev_problem(p)
    trig = opts.get("trig", "hw")
    assert_close(_run(p, d, **opts), _oracle(oracle_mod, p), TOL[trig], f"mirror pairs {opts}")


@pytest.mark.parametrize("M", [0, 1, 3, 33, 4099])
def test_sample_count_tails(oracle_mod, M):
    p = _problem(908, max(M, 1), XS, np.arange(-2, 3), np.arange(-2, 2))
    if M == 0:
        p = dataclasses.replace(p, kx=p.kx[:0], ky=p.ky[:0], kz=p.kz[:0], phi=p.phi[:0], D=p.D[:, :0])
        got = _run(p, dev_problem(p))
        assert not np.any(got)
        return
    assert_close(_run(p, dev_problem(p)), _oracle(oracle_mod, p), TOL["hw"], f"mirror pairs M={M}")


def test_stages_and_repeats_are_bitwise_equal():
    """The stages run in separate calls (one caller workspace) and two runs in a
    row give the one-call result bit for bit."""
    from non_cartesian_mri_amd import fhd_compute
    from non_cartesian_mri_amd.fhd import fhd_workspace_bytes
    p = _problem(909, 3000, XS, np.arange(-4, 4), np.arange(-3, 4), B=3)
    d = dev_problem(p)
    o = dict(engine="mfma", voxels_per_lane=128, trig="hw")
    nbytes = fhd_workspace_bytes(p.kx.size, p.x.size, 3, False, **o)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda:0")
    one = _run(p, d, ws)
    again = _run(p, d, ws)
    assert np.array_equal(one, again)
    out = torch.empty((3, p.x.size), dtype=torch.complex64, device="cuda:0")
    for st in ("mu", "gather+reduce"):
        fhd_compute(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], d["D"], stages=st,
                    workspace=ws, out=out, **o)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), one)
    p1 = dataclasses.replace(p, D=p.D[:1])
    d1 = dev_problem(p1)
    n1 = fhd_workspace_bytes(p.kx.size, p.x.size, 1, False, **o)
    ws1 = torch.empty(n1, dtype=torch.uint8, device="cuda:0")
    whole = _run(p1, d1, ws1)
    out1 = torch.empty((1, p.x.size), dtype=torch.complex64, device="cuda:0")
    for st in ("mu", "gather", "reduce"):
        fhd_compute(d1["kx"], d1["ky"], d1["kz"], d1["x"], d1["y"], d1["z"], d1["phi"], d1["D"], stages=st,
                    workspace=ws1, out=out1, **o)
    torch.cuda.synchronize()
    assert np.array_equal(out1.cpu().numpy(), whole)


# ------------------------- forward operator F rho ---------------------------
def _fwd(p, rho, **opts):
    from non_cartesian_mri_amd import fhd_forward
    d = dev_problem(p)
    opts.setdefault("engine", "mfma")
    opts.setdefault("voxels_per_lane", 128)
    r = torch.from_numpy(np.ascontiguousarray(rho)).to("cuda:0")
    out = fhd_forward(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], r, **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(rho.shape[0], -1)


def _rho(seed, B, N):
    rng = np.random.Generator(np.random.PCG64(seed))
    return np.stack([inputs.complex_normal(rng, N) for _ in range(B)])


@pytest.mark.parametrize("trig", ["hw", "accurate"])
@pytest.mark.parametrize("B", [1, 2, 16, 19])
def test_forward_pairs(oracle_mod, trig, B):
    """F rho with the sum over voxel groups run over mirror pairs (one phase
    and four products per pair: c (rho_g + rho_h) - i s (rho_g - rho_h)),
    against the oracle, on the asymmetric box (pairs, a self-mirrored row and
    rows alone) and against the same call with pairing off."""
    p = _problem(910 + B, 900, XS, np.arange(-5, 5), np.arange(-3, 4), B=B)
    rho = _rho(911 + B, B, p.x.size)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    got = _fwd(p, rho, trig=trig)
    assert_close(got, ref, TOL[trig], f"forward pairs B={B} {trig}")
    off = _fwd(p, rho, trig=trig, mirror_pairs=False)
    assert_close(off, ref, TOL[trig], f"forward pairing off B={B} {trig}")


@pytest.mark.parametrize("trig", ["hw", "accurate"])
@pytest.mark.parametrize("case", ["ragged", "short", "displaced", "no_mirrors", "rows3", "plain", "tile64"])
def test_forward_pair_cases(oracle_mod, trig, case):
    """A partial last group with its reference, a last wave without (direct
    path), a displaced voxel (its wave direct), a grid without mirrors (every
    group alone), explicit rows, a plain sum and short blocks."""
    ys, zs, opts, N = np.arange(-5, 5), np.arange(-3, 4), {}, None
    xs = XS
    if case == "ragged":
        N = 70 * 128 - 50
    elif case == "short":
        N = 69 * 128 + 1
    elif case == "no_mirrors":
        xs, ys, zs = XS + 0.5, np.arange(-4, 4) + 0.5, np.arange(-2, 2) + 0.5
    elif case == "rows3":
        opts = dict(sample_splits=3)
    elif case == "plain":
        opts = dict(sum="plain")
    elif case == "tile64":
        opts = dict(tile=64)
    p = _problem(920, 700, xs, ys, zs, N=N)
    if case == "displaced":
        x = p.x.copy()
        x[3 * 128 + 5] += 0.25
        p = dataclasses.replace(p, x=x)
    rho = _rho(921, 1, p.x.size)
    ref = oracle_mod.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho)
    assert_close(_fwd(p, rho, trig=trig, **opts), ref, TOL[trig], f"forward pairs {case} {trig}")


def test_forward_pairs_adjoint_and_repeat():
    """<F rho, d> = <rho, F^H d> between the paired forward and the paired
    adjoint, and two forward runs agree bit for bit."""
    from non_cartesian_mri_amd import fhd_compute
    p = _problem(930, 1100, XS, np.arange(-4, 4), np.arange(-3, 3))
    rho = _rho(931, 1, p.x.size)
    d = dev_problem(p)
    a1 = _fwd(p, rho, trig="accurate")
    a2 = _fwd(p, rho, trig="accurate")
    assert np.array_equal(a1, a2)
    fh = fhd_compute(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], d["D"], trig="accurate",
                     engine="mfma", voxels_per_lane=128)
    torch.cuda.synchronize()
    fh = fh.cpu().numpy().ravel().astype(np.complex128)
    # the adjoint pairs phi against D: F^H D = sum_m conj(phi) D e^{+}, F rho = phi sum rho e^{-}
    lhs = np.vdot(a1.ravel().astype(np.complex128), p.D[0].astype(np.complex128))
    rhs = np.vdot(rho.ravel().astype(np.complex128), fh)
    assert abs(lhs - rhs) <= 1e-5 * abs(lhs)
