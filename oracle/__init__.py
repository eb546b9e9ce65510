"""CPU oracle for F^H D and Q -- TEST INFRASTRUCTURE, not part of the product.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may
import this package.  It wraps ``oracle.c`` (a plain double-precision triple
loop, OpenMP over voxels) with ctypes and adds the image-quality metric used
by the phantom round trip.  It never imports or calls the HIP library.

Function map to the pages (PMPP ch. 17 "Iterative MRI reconstruction"):
  fhd()       -- F^H D, section 17.2 (Fig. 17.3) and section 17.3 (Figs. 17.4/17.6)
  q()         -- Q, section 17.2 (same core computation with |phi|^2 weights)
  forward()   -- F rho, the forward model whose conjugate transpose fhd() applies
                 (section 17.2; the "inverse process" of section 17.3 step 3)
  psnr_db()   -- PSNR = 20 log10(max(I0) / sqrt(MSE)), section 17.3 step 3 (Fig. 17.18)
Submodules: recon (Toeplitz F^H F, regulariser, CG; section 17.2) and
gridding (trilinear gridding onto the k-lattice + lattice inverse DFT, the
baseline of section 17.1 / Fig. 17.19).
  ls_scale()  -- least-squares intensity scale; the pages leave the scaling of
                 the reconstructed image open, so it is fitted (see the header
                 of psnr_db).
Parity status of each function is recorded in the module docstring of
tests/test_oracle_pins.py (all pinned).
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import time

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (-O2 -fopenmp, no fast-math)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + f".tmp{os.getpid()}"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
                               "-fno-fast-math", "-ffp-contract=off", _SRC, "-o", tmp, "-lm"])
        os.replace(tmp, _LIB)
    return _LIB


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        lib = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i64, i32 = ctypes.c_int64, ctypes.c_int32
        lib.oracle_fhd.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i32, P, i64, P, P]
        lib.oracle_fhd.restype = ctypes.c_int
        lib.oracle_q.argtypes = [P, P, P, P, P, P, P, i64, i64, P, i64, P, P]
        lib.oracle_q.restype = ctypes.c_int
        lib.oracle_forward.argtypes = [P, P, P, P, P, P, P, P, i64, i64, i32, P, i64, P, P]
        lib.oracle_forward.restype = ctypes.c_int
        _lib = lib
    return _lib


def _f32(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.float32:
        raise TypeError(f"oracle expects float32 arrays, got {a.dtype}")
    return a


def _c64(a) -> np.ndarray:
    a = np.ascontiguousarray(a)
    if a.dtype != np.complex64:
        raise TypeError(f"oracle expects complex64 arrays, got {a.dtype}")
    return a


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


class Timing:
    """Wall time and OpenMP thread count of the last oracle call."""
    seconds: float = 0.0
    threads: int = 0


last = Timing()


def fhd(kx, ky, kz, x, y, z, phi, D, idx=None) -> np.ndarray:
    """F^H D in double: complex128 [B, nidx] (D may be [M] or [B, M])."""
    kx, ky, kz, x, y, z = (_f32(a) for a in (kx, ky, kz, x, y, z))
    phi = _c64(phi)
    D = _c64(D)
    if D.ndim == 1:
        D = D[None, :]
    B, M = D.shape
    N = x.shape[0]
    if not (kx.shape == ky.shape == kz.shape == (M,) and phi.shape == (M,)):
        raise ValueError("k, phi and D must all have M samples")
    if not (y.shape == z.shape == (N,)):
        raise ValueError("x, y, z must have N voxels")
    if idx is None:
        nidx = N
        idx_arr = None
    else:
        idx_arr = np.ascontiguousarray(idx, dtype=np.int64)
        if idx_arr.size and (idx_arr.min() < 0 or idx_arr.max() >= N):
            raise IndexError("voxel subset out of range")
        nidx = idx_arr.shape[0]
    out = np.zeros((B, nidx, 2), np.float64)
    th = ctypes.c_int32(0)
    t0 = time.perf_counter()
    rc = _load().oracle_fhd(_ptr(kx), _ptr(ky), _ptr(kz), _ptr(x), _ptr(y), _ptr(z),
                            _ptr(phi), _ptr(D), M, N, B, _ptr(idx_arr), nidx,
                            _ptr(out), ctypes.byref(th))
    last.seconds = time.perf_counter() - t0
    last.threads = th.value
    if rc != 0:
        raise RuntimeError(f"oracle_fhd failed with code {rc}")
    return out[..., 0] + 1j * out[..., 1]


def q(kx, ky, kz, x, y, z, phi, idx=None) -> np.ndarray:
    """Q in double: complex128 [nidx]."""
    kx, ky, kz, x, y, z = (_f32(a) for a in (kx, ky, kz, x, y, z))
    phi = _c64(phi)
    M = kx.shape[0]
    N = x.shape[0]
    if not (ky.shape == kz.shape == phi.shape == (M,)):
        raise ValueError("k and phi must have M samples")
    if not (y.shape == z.shape == (N,)):
        raise ValueError("x, y, z must have N voxels")
    if idx is None:
        nidx, idx_arr = N, None
    else:
        idx_arr = np.ascontiguousarray(idx, dtype=np.int64)
        if idx_arr.size and (idx_arr.min() < 0 or idx_arr.max() >= N):
            raise IndexError("voxel subset out of range")
        nidx = idx_arr.shape[0]
    out = np.zeros((nidx, 2), np.float64)
    th = ctypes.c_int32(0)
    t0 = time.perf_counter()
    rc = _load().oracle_q(_ptr(kx), _ptr(ky), _ptr(kz), _ptr(x), _ptr(y), _ptr(z),
                          _ptr(phi), M, N, _ptr(idx_arr), nidx, _ptr(out), ctypes.byref(th))
    last.seconds = time.perf_counter() - t0
    last.threads = th.value
    if rc != 0:
        raise RuntimeError(f"oracle_q failed with code {rc}")
    return out[:, 0] + 1j * out[:, 1]


def forward(kx, ky, kz, x, y, z, phi, rho, idx=None) -> np.ndarray:
    """F rho in double: complex128 [B, nidx] over samples (rho may be [N] or [B, N])."""
    kx, ky, kz, x, y, z = (_f32(a) for a in (kx, ky, kz, x, y, z))
    phi = _c64(phi)
    rho = _c64(rho)
    if rho.ndim == 1:
        rho = rho[None, :]
    B, N = rho.shape
    M = kx.shape[0]
    if not (ky.shape == kz.shape == phi.shape == (M,)):
        raise ValueError("k and phi must have M samples")
    if not (x.shape == y.shape == z.shape == (N,)):
        raise ValueError("x, y, z and rho must have N voxels")
    if idx is None:
        nidx, idx_arr = M, None
    else:
        idx_arr = np.ascontiguousarray(idx, dtype=np.int64)
        if idx_arr.size and (idx_arr.min() < 0 or idx_arr.max() >= M):
            raise IndexError("sample subset out of range")
        nidx = idx_arr.shape[0]
    out = np.zeros((B, nidx, 2), np.float64)
    th = ctypes.c_int32(0)
    t0 = time.perf_counter()
    rc = _load().oracle_forward(_ptr(kx), _ptr(ky), _ptr(kz), _ptr(x), _ptr(y), _ptr(z),
                                _ptr(phi), _ptr(rho), M, N, B, _ptr(idx_arr), nidx,
                                _ptr(out), ctypes.byref(th))
    last.seconds = time.perf_counter() - t0
    last.threads = th.value
    if rc != 0:
        raise RuntimeError(f"oracle_forward failed with code {rc}")
    return out[..., 0] + 1j * out[..., 1]


def rel_l2(test, ref) -> float:
    """||test - ref||_2 / ||ref||_2 over every element (complex, promoted to double)."""
    test = np.asarray(test, np.complex128)
    ref = np.asarray(ref, np.complex128)
    den = np.linalg.norm(ref.ravel())
    num = np.linalg.norm((test - ref).ravel())
    return float(num / den) if den > 0 else float(num)


def ls_scale(ideal, recon) -> float:
    """alpha minimising ||ideal - alpha*|recon|||^2 (real ideal, magnitude image)."""
    ideal = np.asarray(ideal, np.float64)
    mag = np.abs(np.asarray(recon))
    return float(np.dot(ideal, mag) / np.dot(mag, mag))


def psnr_db(ideal, recon, alpha: float | None = None) -> float:
    """PSNR = 20 log10(max(I0)/sqrt(MSE)) of the scaled magnitude image (Fig. 17.18).

    The pages define PSNR against the ideal image I0 but not how the
    reconstruction's intensity is scaled; here |recon| is scaled by alpha
    (least squares against I0 when not given) before the MSE is taken.
    """
    ideal = np.asarray(ideal, np.float64)
    mag = np.abs(np.asarray(recon))
    if alpha is None:
        alpha = ls_scale(ideal, recon)
    mse = np.mean((ideal - alpha * mag) ** 2)
    return float(20.0 * np.log10(np.max(ideal) / np.sqrt(mse)))
