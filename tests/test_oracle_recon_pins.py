"""Pins of the reconstruction oracle (oracle/recon.py), CPU.

  function          pinned by
  ----------------  ------------------------------------------------------------
  toeplitz_apply    an explicit dense F^H F built from F[m,n] = phi_m e^{-i2pi k.x};
                    Hermitian; <p, F^H F p> = ||F p||^2 with the pinned forward oracle
  normal_direct     equals toeplitz_apply (+ lam laplacian) on small grids (the
                    Q-difference route, in double); equals the compiled adjoint
                    oracle applied to the compiled forward oracle's F p; one
                    sample gives a plane wave times the image's projection
  laplacian         constant images -> 0; a single voxel -> degree at the voxel,
                    -1 at each neighbour; symmetric and positive semidefinite;
                    an explicit sparse matrix of the neighbour graph
  cg                reaches numpy.linalg.solve on a small Hermitian positive definite
                    system; its first step is the steepest-descent step; successive
                    residuals are orthogonal
Status: all pinned.
"""
import numpy as np

from oracle import recon


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _cn(rng, n):
    return (rng.standard_normal(n) + 1j * rng.standard_normal(n)).astype(np.complex64)


def _problem(seed, M, nx, ny, nz):
    rng = _rng(seed)
    kx, ky, kz = ((rng.random(M) - 0.5).astype(np.float32) for _ in range(3))
    phi = _cn(rng, M)
    x, y, z = recon.grid_coords(nx, ny, nz)
    return rng, kx, ky, kz, phi, x, y, z


def _F(kx, ky, kz, phi, x, y, z):
    K = np.stack([kx, ky, kz], 1).astype(np.float64)
    X = np.stack([x, y, z], 1).astype(np.float64)
    return phi.astype(np.complex128)[:, None] * np.exp(-2j * np.pi * (K @ X.T))


def test_toeplitz_apply_is_FhF(oracle_mod):
    nx, ny, nz = 4, 3, 5
    rng, kx, ky, kz, phi, x, y, z = _problem(31, 60, nx, ny, nz)
    F = _F(kx, ky, kz, phi, x, y, z)
    A = F.conj().T @ F
    p = _cn(rng, nx * ny * nz).astype(np.complex128)
    qd = recon.q_differences(kx, ky, kz, phi, nx, ny, nz)
    got = recon.toeplitz_apply(qd, p, nx, ny, nz)
    assert np.max(np.abs(got - A @ p)) <= 1e-11 * np.max(np.abs(A @ p))
    # Hermitian: <u, A v> = <A u, v>
    u = _cn(rng, p.size).astype(np.complex128)
    assert abs(np.vdot(u, recon.toeplitz_apply(qd, p, nx, ny, nz)) -
               np.vdot(recon.toeplitz_apply(qd, u, nx, ny, nz), p)) <= 1e-9 * np.linalg.norm(A) * np.linalg.norm(u) * np.linalg.norm(p)


def test_toeplitz_quadratic_form_is_forward_norm(oracle_mod):
    nx, ny, nz = 3, 4, 3
    rng, kx, ky, kz, phi, x, y, z = _problem(32, 45, nx, ny, nz)
    p = _cn(rng, nx * ny * nz)
    qd = recon.q_differences(kx, ky, kz, phi, nx, ny, nz)
    quad = np.vdot(p.astype(np.complex128), recon.toeplitz_apply(qd, p, nx, ny, nz))
    Fp = oracle_mod.forward(kx, ky, kz, x, y, z, phi, p)[0]
    assert abs(quad.imag) <= 1e-9 * abs(quad.real)
    assert abs(quad.real - np.vdot(Fp, Fp).real) <= 1e-10 * abs(quad.real)


def test_laplacian_closed_forms():
    nx, ny, nz = 5, 4, 3
    ones = np.ones(nx * ny * nz, np.complex128)
    assert np.max(np.abs(recon.laplacian(ones, nx, ny, nz))) == 0
    # one voxel in the interior: 6 at the voxel, -1 at its six neighbours
    p = np.zeros((nz, ny, nx), np.complex128)
    p[1, 2, 3] = 1.0
    out = recon.laplacian(p.ravel(), nx, ny, nz).reshape(nz, ny, nx)
    want = np.zeros_like(p)
    want[1, 2, 3] = 6
    for dz, dy, dx in ((1, 0, 0), (-1, 0, 0), (0, 1, 0), (0, -1, 0), (0, 0, 1), (0, 0, -1)):
        want[1 + dz, 2 + dy, 3 + dx] = -1
    assert np.array_equal(out, want)
    # a corner voxel has 3 neighbours
    p = np.zeros((nz, ny, nx), np.complex128)
    p[0, 0, 0] = 1.0
    out = recon.laplacian(p.ravel(), nx, ny, nz).reshape(nz, ny, nx)
    assert out[0, 0, 0] == 3 and out[1, 0, 0] == -1 and out[0, 1, 0] == -1 and out[0, 0, 1] == -1
    assert np.sum(out != 0) == 4


def test_laplacian_is_the_neighbour_graph_matrix():
    nx, ny, nz = 4, 3, 2
    n = nx * ny * nz
    L = np.zeros((n, n))
    idx = lambda x, y, z: (z * ny + y) * nx + x
    for z in range(nz):
        for y in range(ny):
            for x in range(nx):
                for dx, dy, dz in ((1, 0, 0), (0, 1, 0), (0, 0, 1)):
                    if x + dx < nx and y + dy < ny and z + dz < nz:
                        a, b = idx(x, y, z), idx(x + dx, y + dy, z + dz)
                        L[a, a] += 1; L[b, b] += 1; L[a, b] -= 1; L[b, a] -= 1
    rng = _rng(33)
    p = _cn(rng, n).astype(np.complex128)
    assert np.max(np.abs(recon.laplacian(p, nx, ny, nz) - L @ p)) <= 1e-13
    assert np.allclose(L, L.T) and np.min(np.linalg.eigvalsh(L)) > -1e-12


def test_cg_solves_a_small_system():
    rng = _rng(34)
    n = 12
    G = rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))
    A = G.conj().T @ G + 0.5 * np.eye(n)
    b = rng.standard_normal(n) + 1j * rng.standard_normal(n)
    x, hist = recon.cg(lambda v: A @ v, b, np.zeros(n), 3 * n)
    assert np.max(np.abs(x - np.linalg.solve(A, b))) <= 1e-9 * np.max(np.abs(np.linalg.solve(A, b)))
    assert hist[-1] <= 1e-18 * hist[0]


def test_cg_first_step_and_orthogonal_residuals():
    rng = _rng(35)
    n = 10
    G = rng.standard_normal((n, n)) + 1j * rng.standard_normal((n, n))
    A = G.conj().T @ G + np.eye(n)
    b = rng.standard_normal(n) + 1j * rng.standard_normal(n)
    x1, _ = recon.cg(lambda v: A @ v, b, np.zeros(n), 1)
    alpha = np.vdot(b, b).real / np.vdot(b, A @ b).real   # steepest descent from 0
    assert np.max(np.abs(x1 - alpha * b)) <= 1e-13 * np.max(np.abs(x1))
    rs = []
    x = np.zeros(n, np.complex128)
    for k in range(4):
        xk, _ = recon.cg(lambda v: A @ v, b, np.zeros(n), k)
        rs.append(b - A @ xk)
    for i in range(4):
        for j in range(i):
            assert abs(np.vdot(rs[i], rs[j])) <= 1e-9 * np.linalg.norm(rs[i]) * np.linalg.norm(rs[j]) + 1e-12


def test_normal_direct_equals_toeplitz_route(oracle_mod):
    for seed, M, (nx, ny, nz), lam in ((41, 1, (5, 4, 3), 0.0), (42, 3, (4, 6, 2), 0.0), (43, 50, (3, 4, 5), 0.7)):
        rng, kx, ky, kz, phi, x, y, z = _problem(seed, M, nx, ny, nz)
        p = _cn(rng, nx * ny * nz)
        qd = recon.q_differences(kx, ky, kz, phi, nx, ny, nz)
        want = recon.toeplitz_apply(qd, p, nx, ny, nz) + lam * recon.laplacian(p, nx, ny, nz)
        got = recon.normal_direct(kx, ky, kz, phi, p, nx, ny, nz, lam)
        assert np.max(np.abs(got - want)) <= 1e-11 * np.max(np.abs(want)), (seed, M)


def test_normal_direct_equals_forward_then_adjoint(oracle_mod):
    nx, ny, nz = 6, 5, 4
    rng, kx, ky, kz, phi, x, y, z = _problem(44, 3, nx, ny, nz)
    p = _cn(rng, nx * ny * nz)
    d = oracle_mod.forward(kx, ky, kz, x, y, z, phi, p)[0]
    # the compiled adjoint takes float32 data: F p rounded once to complex64
    want = oracle_mod.fhd(kx, ky, kz, x, y, z, phi, d.astype(np.complex64))[0]
    got = recon.normal_direct(kx, ky, kz, phi, p, nx, ny, nz)
    assert np.max(np.abs(got - want)) <= 1e-6 * np.max(np.abs(want))


def test_normal_direct_one_sample_is_a_plane_wave(oracle_mod):
    """M = 1: F^H F p = |phi|^2 e^{+i2pi k.x_n} sum_n' e^{-i2pi k.x_n'} p[n'], so
    every output has the same modulus and neighbouring voxels along x differ
    by the phase factor e^{i 2 pi kx}."""
    nx, ny, nz = 8, 3, 2
    rng, kx, ky, kz, phi, x, y, z = _problem(45, 1, nx, ny, nz)
    p = _cn(rng, nx * ny * nz)
    got = recon.normal_direct(kx, ky, kz, phi, p, nx, ny, nz).reshape(nz, ny, nx)
    mod = np.abs(got)
    assert np.max(np.abs(mod - mod.flat[0])) <= 1e-12 * mod.flat[0]
    ratio = got[:, :, 1:] / got[:, :, :-1]
    assert np.max(np.abs(ratio - np.exp(2j * np.pi * float(kx[0])))) <= 1e-12
    # |F^H F p| = |phi|^2 |(F p) / phi|
    d = oracle_mod.forward(kx, ky, kz, x, y, z, phi, p)[0, 0]
    assert abs(mod.flat[0] - abs(complex(phi[0])) * abs(d)) <= 1e-12 * mod.flat[0]
