"""Pins of the gridding oracle (oracle/gridding.py), CPU.

  function        pinned by
  --------------  ------------------------------------------------------------
  grid_samples    hand-computed trilinear weights of one off-lattice sample;
                  periodic wrap at the lattice edge; partition of unity
                  (sum G = sum Mu); a sample on a lattice point lands there only
  lattice_image   a single lattice value -> the plane wave exp(i 2 pi kappa.x);
                  pure-Python triple-loop brute force on tiny grids
  lattice_image_at  equals lattice_image at the chosen voxels
  gridding        on a Cartesian trajectory (every sample on a lattice point)
                  it equals F^H D from the pinned oracle exactly (rounding)
Status: all pinned.
"""
import math

import numpy as np
import pytest

from oracle import gridding as G_


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _cn(rng, n):
    return (rng.standard_normal(n) + 1j * rng.standard_normal(n)).astype(np.complex64)


def test_trilinear_weights_by_hand():
    nx, ny, nz = 8, 4, 8
    # lattice units u = k n + n//2 = (3.25, 1.5, 6.75)
    kx = np.array([(3.25 - 4) / 8], np.float32)
    ky = np.array([(1.5 - 2) / 4], np.float32)
    kz = np.array([(6.75 - 4) / 8], np.float32)
    phi = np.array([1.0], np.complex64)
    D = np.array([2.0 - 1.0j], np.complex64)
    g = G_.grid_samples(kx, ky, kz, phi, D, nx, ny, nz)
    want = np.zeros((nz, ny, nx), np.complex128)
    for z, wz in ((6, 0.25), (7, 0.75)):
        for y, wy in ((1, 0.5), (2, 0.5)):
            for x, wx in ((3, 0.75), (4, 0.25)):
                want[z, y, x] = (2.0 - 1.0j) * wx * wy * wz
    assert np.array_equal(g, want)


def test_wrap_at_the_lattice_edge():
    n = 8
    # u = 7.75 in x: floor 7, fraction 0.75 -> 0.25 to cell 7 and 0.75 to
    # cell 8, which is cell 0 (periodic)
    kx = np.array([(7.75 - 4) / 8], np.float32)
    zero = np.array([0.0], np.float32)
    g = G_.grid_samples(kx, zero, zero, np.ones(1, np.complex64), np.ones(1, np.complex64), n, n, n)
    assert g[4, 4, 7] == 0.25 and g[4, 4, 0] == 0.75
    assert np.count_nonzero(g) == 2
    # a negative coordinate below the first lattice point wraps to the top
    kx = np.array([(-0.5 - 4) / 8], np.float32)            # u = -0.5
    g = G_.grid_samples(kx, zero, zero, np.ones(1, np.complex64), np.ones(1, np.complex64), n, n, n)
    assert g[4, 4, 7] == 0.5 and g[4, 4, 0] == 0.5


def test_partition_of_unity_and_on_lattice_samples():
    rng = _rng(41)
    M = 500
    k = (rng.random((3, M)) - 0.5).astype(np.float32)
    phi, D = _cn(rng, M), _cn(rng, M)
    g = G_.grid_samples(k[0], k[1], k[2], phi, D, 8, 16, 4)
    mu = np.conj(phi.astype(np.complex128)) * D
    assert abs(g.sum() - mu.sum()) <= 1e-12 * np.abs(mu).sum()
    # on a lattice point: all of the value in that one cell
    g = G_.grid_samples(np.array([2 / 8], np.float32), np.array([-3 / 16], np.float32),
                        np.array([1 / 4], np.float32), phi[:1], D[:1], 8, 16, 4)
    assert np.count_nonzero(g) == 1 and g[3, 5, 6] == mu[0]


def test_single_lattice_value_is_a_plane_wave():
    nx, ny, nz = 4, 8, 2
    g = np.zeros((nz, ny, nx), np.complex128)
    g[1, 6, 3] = 1.5 - 0.5j
    img = G_.lattice_image(g)
    kap = (G_.lattice(nx)[3], G_.lattice(ny)[6], G_.lattice(nz)[1])
    z, y, x = np.meshgrid(G_.positions(nz), G_.positions(ny), G_.positions(nx), indexing="ij")
    want = (1.5 - 0.5j) * np.exp(2j * math.pi * (kap[0] * x + kap[1] * y + kap[2] * z))
    assert np.max(np.abs(img - want)) <= 1e-13


@pytest.mark.parametrize("shape", [(3, 2, 4), (2, 2, 2), (5, 1, 3)])
def test_lattice_image_brute_force(shape):
    nz, ny, nx = shape
    rng = _rng(42)
    g = rng.standard_normal(shape) + 1j * rng.standard_normal(shape)
    img = G_.lattice_image(g)
    for iz in range(nz):
        for iy in range(ny):
            for ix in range(nx):
                acc = 0j
                for jz in range(nz):
                    for jy in range(ny):
                        for jx in range(nx):
                            ph = ((jx - nx // 2) / nx * (ix - nx // 2) + (jy - ny // 2) / ny * (iy - ny // 2)
                                  + (jz - nz // 2) / nz * (iz - nz // 2))
                            acc += g[jz, jy, jx] * complex(math.cos(2 * math.pi * ph), math.sin(2 * math.pi * ph))
                assert abs(img[iz, iy, ix] - acc) <= 1e-12 * max(1.0, abs(acc))


def test_cartesian_trajectory_equals_fhd(oracle_mod):
    """Every sample on a lattice point: gridding is exact, so it equals F^H D."""
    nx, ny, nz = 8, 4, 8
    rng = _rng(43)
    jz, jy, jx = np.meshgrid(np.arange(nz), np.arange(ny), np.arange(nx), indexing="ij")
    kx = G_.lattice(nx)[jx.ravel()].astype(np.float32)
    ky = G_.lattice(ny)[jy.ravel()].astype(np.float32)
    kz = G_.lattice(nz)[jz.ravel()].astype(np.float32)
    M = kx.size
    phi, D = _cn(rng, M), _cn(rng, M)
    x, y, z = G_.grid_coords(nx, ny, nz)
    ref = oracle_mod.fhd(kx, ky, kz, x, y, z, phi, D[None, :])[0]
    got = G_.gridding(kx, ky, kz, phi, D, nx, ny, nz)
    assert np.max(np.abs(got - ref)) <= 1e-11 * np.max(np.abs(ref))


def test_lattice_image_at_matches_the_full_sum():
    rng = _rng(44)
    g = rng.standard_normal((4, 8, 2)) + 1j * rng.standard_normal((4, 8, 2))
    full = G_.lattice_image(g).ravel()
    idx = np.array([0, 5, 17, 63, 40])
    assert np.max(np.abs(G_.lattice_image_at(g, idx) - full[idx])) <= 1e-12 * np.max(np.abs(full))
