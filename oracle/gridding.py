"""Oracle for the gridding + inverse-FFT baseline -- TEST INFRASTRUCTURE.

PMPP ch. 17 "Iterative MRI reconstruction", section 17.1 (Fig. 17.1B): in
gridding, each k-space sample is convolved with a gridding mask and
accumulated onto a uniform Cartesian grid, and the image is then obtained
with an (inverse) FFT; section 17.3 step 3 (Fig. 17.19) compares a simple
bilinear-interpolation gridding/iFFT image with the iterative one.

Reading taken: the 3-D form of bilinear interpolation (trilinear weights on
the 8 lattice points around a sample) onto the image's own k-lattice, with
the sample value Mu = conj(phi) D of F^H D, so that the gridded image
approximates F^H D.  For an n-point axis with voxel coordinates
x_i = i - n//2 the lattice is kappa_j = (j - n//2) / n cycles per voxel,
j = 0..n-1; the lattice is periodic with period 1 (exp(i 2 pi kappa x) with
integer x does not change when kappa moves by 1), so the 8 neighbours wrap
around.  The image is the plain sum over the lattice:

    image[i] = sum_j G[j] exp(+i 2 pi kappa_j . x_i)

Only the tests may use this module; it shares nothing with the HIP library.
"""
from __future__ import annotations

import math

import numpy as np


def lattice(n: int) -> np.ndarray:
    """k-lattice of an n-point axis: (j - n//2) / n, j = 0..n-1 (float64)."""
    return (np.arange(n) - n // 2) / float(n)


def positions(n: int) -> np.ndarray:
    """Voxel coordinates of an n-point axis: i - n//2 (float64)."""
    return (np.arange(n) - n // 2).astype(np.float64)


def grid_samples(kx, ky, kz, phi, D, nx: int, ny: int, nz: int) -> np.ndarray:
    """G[jz, jy, jx] = sum_m Mu_m w_m(j): trilinear weights, periodic lattice (complex128)."""
    mu = np.conj(np.asarray(phi, np.complex128)) * np.asarray(D, np.complex128)
    G = np.zeros((nz, ny, nx), np.complex128)
    cells, fracs = [], []
    for k, n in ((kx, nx), (ky, ny), (kz, nz)):
        # lattice units: u = k n + n//2, so that u = j on the lattice point kappa_j
        u = np.asarray(k, np.float64) * n + n // 2
        j0 = np.floor(u)
        cells.append(j0.astype(np.int64))
        fracs.append(u - j0)
    (jx, jy, jz), (fx, fy, fz) = cells, fracs
    for dz in (0, 1):
        wz = fz if dz else 1.0 - fz
        for dy in (0, 1):
            wy = fy if dy else 1.0 - fy
            for dx in (0, 1):
                wx = fx if dx else 1.0 - fx
                np.add.at(G, ((jz + dz) % nz, (jy + dy) % ny, (jx + dx) % nx), mu * (wx * wy * wz))
    return G


def lattice_image(G: np.ndarray) -> np.ndarray:
    """image[iz, iy, ix] = sum_j G[j] exp(+i 2 pi kappa_j . x_i), by explicit separable sums."""
    nz, ny, nx = G.shape
    E = [np.exp(2j * math.pi * np.outer(positions(n), lattice(n))) for n in (nx, ny, nz)]
    # sum over jx, then jy, then jz (each a plain matrix-vector sum along one axis)
    t = np.einsum("zyj,xj->zyx", G, E[0])
    t = np.einsum("zjx,yj->zyx", t, E[1])
    return np.einsum("jyx,zj->zyx", t, E[2])


def lattice_image_at(G: np.ndarray, idx) -> np.ndarray:
    """The same sum as lattice_image at the voxels idx only (flat indices, x
    fastest): over jx (once per distinct voxel x index), then jy, then jz."""
    nz, ny, nx = G.shape
    idx = np.asarray(idx, np.int64)
    ix, iy, iz = idx % nx, (idx // nx) % ny, idx // (nx * ny)
    ux, inv = np.unique(ix, return_inverse=True)
    ex = np.exp(2j * math.pi * np.outer(positions(nx)[ux], lattice(nx)))   # [distinct x, nx]
    ey = np.exp(2j * math.pi * np.outer(positions(ny)[iy], lattice(ny)))   # [count, ny]
    ez = np.exp(2j * math.pi * np.outer(positions(nz)[iz], lattice(nz)))
    t = (G.reshape(nz * ny, nx) @ ex.T).reshape(nz, ny, ux.size)       # sum over jx
    out = np.empty(idx.size, np.complex128)
    for c0 in range(0, idx.size, 256):
        c = slice(c0, min(c0 + 256, idx.size))
        u = np.einsum("zyc,cy->zc", t[:, :, inv[c]], ey[c])              # then jy
        out[c] = np.einsum("zc,cz->c", u, ez[c])                         # then jz
    return out


def gridding(kx, ky, kz, phi, D, nx: int, ny: int, nz: int) -> np.ndarray:
    """Gridded image, complex128 [nz * ny * nx] (x fastest)."""
    return lattice_image(grid_samples(kx, ky, kz, phi, D, nx, ny, nz)).ravel()


def grid_coords(nx: int, ny: int, nz: int):
    """Voxel coordinates of the gridding image (float32, x fastest), as fhd() takes them."""
    iz, iy, ix = np.meshgrid(positions(nz), positions(ny), positions(nx), indexing="ij")
    return ix.ravel().astype(np.float32), iy.ravel().astype(np.float32), iz.ravel().astype(np.float32)
