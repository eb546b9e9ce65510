"""Helpers shared by the GPU parity tests (device transfer, comparisons)."""
from __future__ import annotations

import numpy as np
import torch

# Parity bars: relative L2 error against the double-precision oracle.
TOL = {"accurate": 1e-5, "hw": 2e-3}
# Per-element bar, relative to the RMS magnitude of the oracle's outputs: an
# element-wise error of ~6 standard deviations of the L2 bar.
ELEM_FACTOR = 6.0


def require_gpu():
    import pytest
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    from non_cartesian_mri_amd import _lib
    _lib.load()  # raises if the HIP library was not built


def dev_problem(p, device="cuda:0"):
    d = {k: torch.from_numpy(np.ascontiguousarray(getattr(p, k))).to(device)
         for k in ("kx", "ky", "kz", "x", "y", "z", "phi")}
    d["D"] = None if p.D is None else torch.from_numpy(np.ascontiguousarray(p.D)).to(device)
    return d


def gpu_fhd(p, d=None, **opts) -> np.ndarray:
    from non_cartesian_mri_amd import fhd_compute
    d = d or dev_problem(p)
    out = fhd_compute(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], d["D"], **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy().reshape(p.B, p.N)


def gpu_q(p, d=None, **opts) -> np.ndarray:
    from non_cartesian_mri_amd import q_compute
    d = d or dev_problem(p)
    out = q_compute(d["kx"], d["ky"], d["kz"], d["x"], d["y"], d["z"], d["phi"], **opts)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def assert_close(test, ref, tol, what=""):
    """Relative-L2 bar plus a per-element bar scaled by the oracle's RMS."""
    test = np.asarray(test, np.complex128).ravel()
    ref = np.asarray(ref, np.complex128).ravel()
    assert test.shape == ref.shape, (test.shape, ref.shape)
    assert np.all(np.isfinite(test)), f"{what}: non-finite output"
    nref = np.linalg.norm(ref)
    err = np.abs(test - ref)
    rel = float(np.linalg.norm(err) / nref) if nref > 0 else float(np.linalg.norm(err))
    rms = nref / np.sqrt(max(ref.size, 1))
    worst = float(err.max() / rms) if rms > 0 and ref.size else float(err.max(initial=0.0))
    print(f"[parity] {what}: rel_l2={rel:.3e} max_elem/rms={worst:.3e} (tol {tol:g})", flush=True)
    assert rel <= tol, f"{what}: rel_l2 {rel:.3e} > {tol:g}"
    assert worst <= ELEM_FACTOR * tol, f"{what}: element error {worst:.3e} > {ELEM_FACTOR * tol:g}"
    return rel
