"""Oracle for the iterative reconstruction step -- TEST INFRASTRUCTURE.

PMPP ch. 17 "Iterative MRI reconstruction", section 17.2: the image rho is
found by solving (F^H F + lambda W^H W) rho = F^H D iteratively (conjugate
gradient, Fig. 17.3); F^H F is applied through Q, which is computed once per
trajectory; W is a regulariser.  The pages' W^H W holds an anatomical prior
that needs patient data; here W is the stand-in of first differences along
each axis of the voxel grid, so W^H W is the 6-neighbour graph Laplacian.

Plain double-precision steps, small grids only (the Toeplitz product is an
O(N^2) sum):
  toeplitz_apply() -- (F^H F p)[n] = sum_n' Q(x_n - x_n') p[n'] on a unit grid,
                      Q from oracle.q at every coordinate difference
  normal_direct()  -- F^H F p (+ lam W^H W p) by the definition F^H (F p), one
                      sample at a time: O(M N), so any grid size for a few samples
  laplacian()      -- (W^H W p)[n] = sum over grid neighbours n' of p[n] - p[n']
  cg()             -- textbook conjugate gradient, fixed iteration count
Only the tests may use this module; it shares nothing with the HIP library.
"""
from __future__ import annotations

import numpy as np


def grid_coords(nx: int, ny: int, nz: int):
    """Voxel coordinates of an nx x ny x nz unit grid, x fastest, origin at the centre."""
    iz, iy, ix = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")
    return ((ix - nx // 2).ravel().astype(np.float32), (iy - ny // 2).ravel().astype(np.float32),
            (iz - nz // 2).ravel().astype(np.float32))


def q_differences(kx, ky, kz, phi, nx: int, ny: int, nz: int) -> np.ndarray:
    """Q at every coordinate difference d in (-n, n) per axis: complex128 [2nz-1, 2ny-1, 2nx-1]."""
    import oracle
    dz, dy, dx = np.meshgrid(np.arange(-(nz - 1), nz), np.arange(-(ny - 1), ny),
                             np.arange(-(nx - 1), nx), indexing="ij")
    q = oracle.q(kx, ky, kz, dx.ravel().astype(np.float32), dy.ravel().astype(np.float32),
                 dz.ravel().astype(np.float32), phi)
    return q.reshape(2 * nz - 1, 2 * ny - 1, 2 * nx - 1)


def toeplitz_apply(qd: np.ndarray, p: np.ndarray, nx: int, ny: int, nz: int) -> np.ndarray:
    """(F^H F p)[n] = sum_n' Q(x_n - x_n') p[n'], by the plain double sum over all pairs."""
    p = np.asarray(p, np.complex128).reshape(nz, ny, nx)
    out = np.zeros((nz, ny, nx), np.complex128)
    for z in range(nz):
        for y in range(ny):
            for x in range(nx):
                # Q at (x - x', y - y', z - z') for every (x', y', z')
                sub = qd[z + nz - 1 - np.arange(nz)][:, y + ny - 1 - np.arange(ny)][:, :, x + nx - 1 - np.arange(nx)]
                out[z, y, x] = np.sum(sub * p)
    return out.ravel()


def normal_direct(kx, ky, kz, phi, p: np.ndarray, nx: int, ny: int, nz: int, lam: float = 0.0) -> np.ndarray:
    """F^H F p + lam W^H W p on the unit grid of grid_coords, from the definition
    of F (F[m][n] = phi_m exp(-i 2 pi k_m . x_n)): for each sample m in turn,
    (F p)[m] = phi_m sum_n exp(-i 2 pi k_m . x_n) p[n], then
    conj(phi_m) exp(+i 2 pi k_m . x_n) (F p)[m] is added at every voxel n.  All
    in double from the float32 inputs; complex128 [N]."""
    x, y, z = (a.astype(np.float64) for a in grid_coords(nx, ny, nz))
    pv = np.asarray(p, np.complex128).ravel()
    out = np.zeros(pv.size, np.complex128)
    ph = np.asarray(phi, np.complex64).astype(np.complex128)
    for m in range(len(kx)):
        theta = 2.0 * np.pi * (float(kx[m]) * x + float(ky[m]) * y + float(kz[m]) * z)
        e = np.exp(1j * theta)                    # exp(+i 2 pi k_m . x_n)
        fp = ph[m] * np.sum(np.conj(e) * pv)      # (F p)[m]
        out += np.conj(ph[m]) * fp * e
        del theta, e
    if lam:
        out += lam * laplacian(pv, nx, ny, nz)
    return out


def laplacian(p: np.ndarray, nx: int, ny: int, nz: int) -> np.ndarray:
    """(W^H W p)[n] = sum of p[n] - p[n'] over the (up to 6) grid neighbours n'."""
    p = np.asarray(p, np.complex128).reshape(nz, ny, nx)
    out = np.zeros_like(p)
    for axis in range(3):
        d = np.diff(p, axis=axis)          # p[i+1] - p[i] along the axis
        lo = [slice(None)] * 3
        hi = [slice(None)] * 3
        lo[axis] = slice(0, -1)
        hi[axis] = slice(1, None)
        out[tuple(lo)] -= d                # p[i] - p[i+1]
        out[tuple(hi)] += d                # p[i+1] - p[i]
    return out.ravel()


def cg(apply_a, b: np.ndarray, x0: np.ndarray, iters: int):
    """Conjugate gradient for a Hermitian positive definite operator.

    r = b - A x, p = r; each iteration: alpha = <r, r> / <p, A p>,
    x += alpha p, r -= alpha A p, beta = <r_new, r_new> / <r, r>, p = r + beta p.
    Returns (x, residual norms squared <r_i, r_i> for i = 0..iters).
    """
    x = np.array(x0, np.complex128)
    r = np.asarray(b, np.complex128) - apply_a(x)
    p = r.copy()
    rs = float(np.vdot(r, r).real)
    hist = [rs]
    for _ in range(iters):
        ap = apply_a(p)
        alpha = rs / float(np.vdot(p, ap).real)
        x = x + alpha * p
        r = r - alpha * ap
        rs_new = float(np.vdot(r, r).real)
        p = r + (rs_new / rs) * p
        rs = rs_new
        hist.append(rs)
    return x, np.array(hist)
