"""gfx950 (MI355X) F^H D / Q for iterative non-Cartesian MRI reconstruction.

Public entry points (thin wrappers over the C ABI in include/fhd.h):
  fhd_compute(kx, ky, kz, x, y, z, phi, D, ...) -> complex64 [N] or [B, N]
  fhd_compute_noalloc(...)                      -> as fhd_compute, workspace in the library's fixed array
  q_compute(kx, ky, kz, x, y, z, phi, ...)      -> complex64 [N]
  fhd_forward(kx, ky, kz, x, y, z, phi, rho, ...) -> complex64 [M] or [B, M]
  fhd_workspace_bytes(M, N, batch, is_q, ..., op=...), fhd_describe_plan(...)
  fhd_toeplitz_kernel(kx, ky, kz, phi, (nz, ny, nx), ...) -> complex64 [2nz, 2ny, 2nx]
  fhd_normal_apply(Qhat, p, lam, ...)           -> F^H F p + lam W^H W p
  fhd_cg_solve(Qhat, b, iters, lam, ...)        -> conjugate-gradient image
  fhd_gridding(kx, ky, kz, phi, D, (nz, ny, nx)) -> gridding/iFFT baseline image

The HIP library is loaded on first use; a missing library raises instead of
falling back to any CPU path.  ``inputs`` holds the seeded synthetic data
generators (trajectories, voxel grids, phantom).
"""
from . import inputs  # noqa: F401

__all__ = ["fhd_compute", "fhd_compute_noalloc", "q_compute", "fhd_forward", "fhd_workspace_bytes", "fhd_describe_plan",
           "fhd_toeplitz_kernel", "fhd_normal_apply", "fhd_cg_solve", "fhd_toeplitz_bytes",
           "fhd_cg_workspace_bytes", "fhd_gridding", "inputs", "library_path"]


def __getattr__(name):
    if name in __all__ and name not in ("inputs", "library_path"):
        from . import fhd
        return getattr(fhd, name)
    if name == "library_path":
        from . import _lib
        return _lib.LIB_PATH
    raise AttributeError(name)
