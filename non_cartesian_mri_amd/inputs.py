"""Seeded synthetic inputs for the F^H D / Q computation.

This module only *generates data*: voxel grids, k-space trajectories, complex
sample weights and scan data, and an analytic 3-D ellipsoid phantom.  It holds
none of the reconstruction arithmetic (no Mu, no gather sum), so both the HIP
path and the CPU oracle can be fed from it without sharing any of the method.

Conventions (chosen here, the pages fix none of them):

* k is in cycles/voxel and voxel coordinates are in voxel units, so the phase
  of a (sample, voxel) pair is k.x revolutions (Eq. 17.1 of "Iterative MRI
  reconstruction", PMPP ch. 17, section 17.1: exp(i 2 pi k_j . r)).
* voxel n = (iz*L + iy)*L + ix (x fastest), coordinate c_i = (i - L/2)*step.
* RNG: numpy Generator(PCG64(seed)); a complex N(0,1) vector draws its real
  block, then its imaginary block; draw order is trajectory (if random), phi,
  then D[0..B-1].  Everything is generated in float64 and cast to float32; the
  float32 arrays are what both sides consume.

Workload shapes follow the pages' moderate-resolution case (128^3 voxels,
hundreds of thousands of samples on spiral / radial trajectories, single
precision data; ch. 17 sections 17.2 and 17.3).  The pages name no dataset.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "voxel_grid", "uniform_k", "radial_k", "stack_of_spirals_k",
    "complex_normal", "subset_indices", "PHANTOM", "phantom_image",
    "phantom_kspace", "phantom_slices", "Problem", "make_config", "CONFIGS",
]


def _rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def voxel_grid(L: int, step: float = 1.0) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """Cartesian voxel centres of an L^3 grid, x fastest, c_i = (i - L/2)*step."""
    c = ((np.arange(L, dtype=np.float64) - L // 2) * step).astype(np.float32)
    shape = (L, L, L)
    return (np.broadcast_to(c[None, None, :], shape).ravel(), np.broadcast_to(c[None, :, None], shape).ravel(),
            np.broadcast_to(c[:, None, None], shape).ravel())


def uniform_k(M: int, rng: np.random.Generator) -> tuple[np.ndarray, np.ndarray, np.ndarray]:
    """M samples uniform in [-0.5, 0.5)^3 cycles/voxel (kx block, ky, kz)."""
    k = rng.random((3, M)) - 0.5
    return tuple(k[i].astype(np.float32) for i in range(3))


def fibonacci_directions(n: int) -> np.ndarray:
    """n unit vectors on a Fibonacci sphere: z_s = 1-(2s+1)/n, azimuth s*pi*(3-sqrt5)."""
    s = np.arange(n, dtype=np.float64)
    zs = 1.0 - (2.0 * s + 1.0) / n
    az = s * math.pi * (3.0 - math.sqrt(5.0))
    rho = np.sqrt(np.maximum(0.0, 1.0 - zs * zs))
    return np.stack([rho * np.cos(az), rho * np.sin(az), zs], axis=1)


def radial_k(n_spokes: int, n_points: int = 256, M: int | None = None):
    """Centre-out 3-D radial spokes; radii 0.5*j/(n_points-1); m = spoke*n_points + j.

    If M is given the spoke-major list is truncated to its first M samples.
    """
    u = fibonacci_directions(n_spokes)
    r = 0.5 * np.arange(n_points, dtype=np.float64) / (n_points - 1)
    k = (u[:, None, :] * r[None, :, None]).reshape(-1, 3)
    if M is not None:
        if M > k.shape[0]:
            raise ValueError("M larger than n_spokes*n_points")
        k = k[:M]
    return tuple(k[:, i].astype(np.float32) for i in range(3))


def stack_of_spirals_k(n_planes: int = 64, n_points: int = 4096, turns: int = 64):
    """Stack of Archimedean spirals inside the ball |k| <= 0.5.

    Plane p sits at kz_p = -0.5 + (p+0.5)/n_planes with radius
    R_p = sqrt(0.25 - kz_p^2); point j has tau = j/n_points, r = R_p*tau,
    angle 2*pi*turns*tau; m = p*n_points + j.
    """
    p = np.arange(n_planes, dtype=np.float64)
    kz_p = -0.5 + (p + 0.5) / n_planes
    R_p = np.sqrt(0.25 - kz_p ** 2)
    tau = np.arange(n_points, dtype=np.float64) / n_points
    r = R_p[:, None] * tau[None, :]
    th = 2.0 * math.pi * turns * tau
    kx = (r * np.cos(th)[None, :]).ravel()
    ky = (r * np.sin(th)[None, :]).ravel()
    kz = np.repeat(kz_p, n_points)
    return kx.astype(np.float32), ky.astype(np.float32), kz.astype(np.float32)


def complex_normal(rng: np.random.Generator, n: int) -> np.ndarray:
    """complex64[n] with N(0,1) real and imaginary parts (real block drawn first)."""
    re = rng.standard_normal(n)
    im = rng.standard_normal(n)
    return (re + 1j * im).astype(np.complex64)


def subset_indices(N: int, count: int, seed: int) -> np.ndarray:
    """Sorted seeded subset of voxel indices used where the oracle cannot do all N."""
    if count >= N:
        return np.arange(N, dtype=np.int64)
    rng = _rng(seed + 1000)
    return np.sort(rng.choice(N, count, replace=False)).astype(np.int64)


# ---------------------------------------------------------------------------
# Phantom: six uniform ellipsoids (our own parameters, voxel units).  Each row:
# centre (3), semi-axes (a, b, c), rotation about z in degrees, density.
PHANTOM = (
    ((0.0, 0.0, 0.0), (40.0, 44.0, 38.0), 0.0, 1.0),
    ((0.0, 0.0, 0.0), (36.0, 40.0, 34.0), 0.0, -0.6),
    ((-12.0, 8.0, 0.0), (8.0, 14.0, 10.0), 25.0, 0.35),
    ((13.0, -6.0, 6.0), (10.0, 6.0, 12.0), -20.0, 0.25),
    ((0.0, 18.0, -10.0), (5.0, 5.0, 5.0), 0.0, 0.5),
    ((4.0, -22.0, 12.0), (3.0, 7.0, 3.0), 40.0, 0.45),
)


def scaled_phantom(f: float, phantom=PHANTOM):
    """The phantom with centres and semi-axes multiplied by f (for smaller grids)."""
    return tuple((tuple(f * c for c in centre), tuple(f * a for a in axes), psi, rho)
                 for centre, axes, psi, rho in phantom)


def _rot_z(deg: float) -> np.ndarray:
    a = math.radians(deg)
    c, s = math.cos(a), math.sin(a)
    return np.array([[c, -s, 0.0], [s, c, 0.0], [0.0, 0.0, 1.0]])


def phantom_image(x, y, z, phantom=PHANTOM) -> np.ndarray:
    """Ideal image I0 at the given voxel centres (float64)."""
    p = np.stack([np.asarray(x, np.float64), np.asarray(y, np.float64),
                  np.asarray(z, np.float64)], axis=1)
    img = np.zeros(p.shape[0])
    for centre, axes, psi, rho in phantom:
        R = _rot_z(psi)
        u = (p - np.asarray(centre)) @ R  # = R^T (x - c) per row
        u = u / np.asarray(axes)
        img += rho * (np.sum(u * u, axis=1) <= 1.0)
    return img


def _ball_ft(kappa: np.ndarray) -> np.ndarray:
    """Fourier transform of the unit-ball indicator at radial frequency kappa.

    (sin 2 pi k - 2 pi k cos 2 pi k) / (2 pi^2 k^3), with a two-term series
    below kappa = 1e-3 where the closed form cancels catastrophically.
    """
    kappa = np.asarray(kappa, np.float64)
    out = np.empty_like(kappa)
    small = kappa < 1e-3
    a = 2.0 * math.pi * kappa[~small]
    out[~small] = (np.sin(a) - a * np.cos(a)) / (2.0 * math.pi ** 2 * kappa[~small] ** 3)
    a2 = (2.0 * math.pi * kappa[small]) ** 2
    out[small] = (4.0 * math.pi / 3.0) * (1.0 - a2 / 10.0)
    return out


def phantom_kspace(kx, ky, kz, phantom=PHANTOM) -> np.ndarray:
    """Continuous Fourier transform of the phantom, sum_e rho_e abc e^{-i2pi k.c_e} J(|A R^T k|).

    This is the synthetic "scan" of the ideal image (forward model with
    exp(-i 2 pi k.x)); complex128.
    """
    k = np.stack([np.asarray(kx, np.float64), np.asarray(ky, np.float64),
                  np.asarray(kz, np.float64)], axis=1)
    out = np.zeros(k.shape[0], np.complex128)
    for centre, axes, psi, rho in phantom:
        R = _rot_z(psi)
        kk = (k @ R) * np.asarray(axes)  # rows: A R^T k
        kappa = np.sqrt(np.sum(kk * kk, axis=1))
        vol = axes[0] * axes[1] * axes[2]
        shift = np.exp(-2j * math.pi * (k @ np.asarray(centre)))
        out += rho * vol * shift * _ball_ft(kappa)
    return out


def phantom_slices(L: int) -> np.ndarray:
    """Indices of the three central orthogonal slices (x=0, y=0, z=0) of an L^3 grid."""
    i = np.arange(L)
    c = L // 2
    iz, iy, ix = np.meshgrid(i, i, i, indexing="ij")
    mask = (ix == c) | (iy == c) | (iz == c)
    return np.nonzero(mask.ravel())[0].astype(np.int64)


# ---------------------------------------------------------------------------
@dataclass
class Problem:
    """One F^H D (or Q) problem instance: float32 arrays as both sides consume them."""
    name: str
    kind: str                      # "fhd" or "q"
    kx: np.ndarray
    ky: np.ndarray
    kz: np.ndarray
    x: np.ndarray
    y: np.ndarray
    z: np.ndarray
    phi: np.ndarray                # complex64 [M]
    D: np.ndarray | None           # complex64 [B, M] (fhd) or None (q)
    seed: int
    L: int = 0
    extra: dict = field(default_factory=dict)

    @property
    def M(self) -> int:
        return int(self.kx.shape[0])

    @property
    def N(self) -> int:
        return int(self.x.shape[0])

    @property
    def B(self) -> int:
        return 1 if self.D is None else int(self.D.shape[0])

    @property
    def pairs(self) -> int:
        return self.M * self.N * self.B


CONFIGS = {
    "fhd_32cube_2048_uniform": "FhD 32^3 voxels, M=2048 uniform-random k, complex N(0,1) phi and D",
    "fhd_64cube_65536_radial": "FhD 64^3 voxels, M=65,536 on 256 Fibonacci spokes x 256 points",
    "fhd_128cube_262144_spirals": "FhD 128^3 voxels, M=262,144 on 64 kz planes x 4096-point spirals",
    "fhd_512cube_262144_spirals": "FhD 512^3 voxels (N beyond 128^3), the same 262,144-sample spiral stack",
    "fhd_128cube_262144_spirals_jittered": "FhD at 2,097,152 off-grid points (each 128^3 voxel centre displaced by "
                                           "a seeded uniform offset in [-0.25, 0.25)^3), the 128^3 workload's "
                                           "samples, phi and D",
    "q_128cube_halfstep_1048576_uniform": "Q on a 2x-oversampled 128^3 grid (step 0.5), M=1,048,576 uniform-random k",
    "q_128cube_unitstep_1048576_uniform": "Q on a 128^3 grid with step 1 (coords -64..63), M=1,048,576 uniform-random k",
    "fhd16_96cube_500001_radial": "FhD x16 D vectors, 96^3 voxels, M=500,001 radial (odd tail)",
    "phantom_96cube_500001_radial": "FhD of the analytic ellipsoid phantom, 96^3 voxels, M=500,001 radial, phi=|k|^2",
}


def make_config(name: str) -> Problem:
    """Build one of the named workloads (see CONFIGS)."""
    if name == "fhd_32cube_2048_uniform":
        rng = _rng(101)
        kx, ky, kz = uniform_k(2048, rng)
        x, y, z = voxel_grid(32)
        phi = complex_normal(rng, 2048)
        D = complex_normal(rng, 2048)[None, :]
        return Problem(name, "fhd", kx, ky, kz, x, y, z, phi, D, 101, 32)
    if name == "fhd_64cube_65536_radial":
        rng = _rng(102)
        kx, ky, kz = radial_k(256, 256)
        x, y, z = voxel_grid(64)
        M = kx.shape[0]
        phi = complex_normal(rng, M)
        D = complex_normal(rng, M)[None, :]
        return Problem(name, "fhd", kx, ky, kz, x, y, z, phi, D, 102, 64)
    if name == "fhd_128cube_262144_spirals":
        rng = _rng(103)
        kx, ky, kz = stack_of_spirals_k(64, 4096, 64)
        x, y, z = voxel_grid(128)
        M = kx.shape[0]
        phi = complex_normal(rng, M)
        D = complex_normal(rng, M)[None, :]
        return Problem(name, "fhd", kx, ky, kz, x, y, z, phi, D, 103, 128)
    if name == "fhd_128cube_262144_spirals_jittered":
        p = make_config("fhd_128cube_262144_spirals")
        j = _rng(107).random((3, p.N)) - 0.5
        x, y, z = ((c.astype(np.float64) + 0.5 * j[i]).astype(np.float32) for i, c in enumerate((p.x, p.y, p.z)))
        return Problem(name, "fhd", p.kx, p.ky, p.kz, x, y, z, p.phi, p.D, 103, 128, extra={"jitter": 0.25})
    if name == "fhd_512cube_262144_spirals":
        rng = _rng(106)
        kx, ky, kz = stack_of_spirals_k(64, 4096, 64)
        x, y, z = voxel_grid(512)
        M = kx.shape[0]
        phi = complex_normal(rng, M)
        D = complex_normal(rng, M)[None, :]
        return Problem(name, "fhd", kx, ky, kz, x, y, z, phi, D, 106, 512)
    if name in ("q_128cube_halfstep_1048576_uniform", "q_128cube_unitstep_1048576_uniform"):
        rng = _rng(104)
        kx, ky, kz = uniform_k(1 << 20, rng)
        x, y, z = voxel_grid(128, 0.5 if name == "q_128cube_halfstep_1048576_uniform" else 1.0)
        phi = complex_normal(rng, 1 << 20)
        return Problem(name, "q", kx, ky, kz, x, y, z, phi, None, 104, 128,
                       extra={"step": 0.5 if name == "q_128cube_halfstep_1048576_uniform" else 1.0})
    if name == "fhd16_96cube_500001_radial":
        rng = _rng(105)
        kx, ky, kz = radial_k(1954, 256, 500_001)
        x, y, z = voxel_grid(96)
        M = kx.shape[0]
        phi = complex_normal(rng, M)
        D = np.stack([complex_normal(rng, M) for _ in range(16)])
        return Problem(name, "fhd", kx, ky, kz, x, y, z, phi, D, 105, 96)
    if name == "phantom_96cube_500001_radial":
        kx, ky, kz = radial_k(1954, 256, 500_001)
        x, y, z = voxel_grid(96)
        k2 = (kx.astype(np.float64) ** 2 + ky.astype(np.float64) ** 2
              + kz.astype(np.float64) ** 2)
        phi = k2.astype(np.complex64)
        D = phantom_kspace(kx, ky, kz).astype(np.complex64)[None, :]
        return Problem(name, "fhd", kx, ky, kz, x, y, z, phi, D, 105, 96,
                       extra={"slices": phantom_slices(96)})
    raise KeyError(f"unknown config {name!r}; known: {sorted(CONFIGS)}")


def random_problem(seed: int, M: int, N: int | None = None, B: int = 1,
                   L: int | None = None, kind: str = "fhd",
                   coords: str = "grid", kmax: float = 0.5) -> Problem:
    """Small seeded problem for parity and edge-case tests.

    coords="grid" uses an L^3 Cartesian grid (N = L^3); coords="random" draws
    N voxel centres uniform in [-L/2, L/2)^3 (an irregular set).
    """
    rng = _rng(seed)
    k = (rng.random((3, M)) - 0.5) * (2.0 * kmax)
    kx, ky, kz = (k[i].astype(np.float32) for i in range(3))
    if coords == "grid":
        if L is None:
            raise ValueError("grid coords need L")
        x, y, z = voxel_grid(L)
    elif coords == "random":
        if N is None or L is None:
            raise ValueError("random coords need N and L")
        c = (rng.random((3, N)) - 0.5) * L
        x, y, z = (c[i].astype(np.float32) for i in range(3))
    else:
        raise ValueError(coords)
    if N is not None and coords == "grid":
        x, y, z = x[:N], y[:N], z[:N]
    phi = complex_normal(rng, M)
    D = None if kind == "q" else np.stack([complex_normal(rng, M) for _ in range(B)]).reshape(B, M)
    return Problem(f"rand{seed}", kind, kx, ky, kz, x, y, z, phi, D, seed, L or 0)
