"""ctypes loader for libncmri_fhd.so (the C ABI declared in include/fhd.h).

The library is built in-tree by ``python -m non_cartesian_mri_amd.build``.  If
it is missing, loading raises: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libncmri_fhd.so")

# fhd_status
FHD_OK = 0
FHD_ERR_INVALID_ARGUMENT = 1
FHD_ERR_WORKSPACE = 2
FHD_ERR_HIP = 3
FHD_ERR_UNSUPPORTED_DEVICE = 4
FHD_ERR_INTERNAL = 5
# fhd_trig
FHD_TRIG_ACCURATE = 0
FHD_TRIG_HW = 1
# fhd_sum
FHD_SUM_BLOCKED = 0
FHD_SUM_KAHAN = 1
FHD_SUM_PLAIN = 2
# stages
FHD_OP_FHD = 0
FHD_OP_Q = 1
FHD_OP_FORWARD = 2

FHD_ENGINE_AUTO = 0
FHD_ENGINE_VALU = 1
FHD_ENGINE_MFMA = 2
FHD_ENGINE_MFMA16 = 3

FHD_STAGE_MU = 1
FHD_STAGE_GATHER = 2
FHD_STAGE_REDUCE = 4
FHD_STAGE_ALL = 7

FHD_FLAG_NO_MIRROR_PAIRS = 1

# size of the device array behind fhd_compute_noalloc (FHD_NOALLOC_SCRATCH_BYTES)
NOALLOC_SCRATCH_BYTES = 512 << 20

# every symbol the header declares
EXPORTED = ("fhd_default_opts", "fhd_workspace_bytes", "fhd_compute", "fhd_compute_noalloc", "q_compute",
            "fhd_forward", "fhd_toeplitz_bytes", "fhd_toeplitz_kernel", "fhd_cg_workspace_bytes",
            "fhd_normal_apply", "fhd_cg_solve", "fhd_gridding", "fhd_describe_plan", "fhd_status_string",
            "fhd_last_error", "fhd_version")


class FhdOpts(ctypes.Structure):
    _fields_ = [
        ("trig", ctypes.c_int32),
        ("sum", ctypes.c_int32),
        ("voxels_per_lane", ctypes.c_int32),
        ("tile", ctypes.c_int32),
        ("stages", ctypes.c_int32),
        ("sample_splits", ctypes.c_int32),
        ("engine", ctypes.c_int32),
        ("flags", ctypes.c_int32),
        ("workspace", ctypes.c_void_p),
        ("workspace_bytes", ctypes.c_size_t),
    ]


class FhdPlanInfo(ctypes.Structure):
    _fields_ = [
        ("voxels_per_lane", ctypes.c_int32),
        ("tile", ctypes.c_int32),
        ("passes", ctypes.c_int32),
        ("record_dwords", ctypes.c_int32),
        ("padded_samples", ctypes.c_int64),
        ("workspace_bytes", ctypes.c_size_t),
        ("sample_splits", ctypes.c_int32),
        ("engine", ctypes.c_int32),
        ("mirror_pairs", ctypes.c_int32),
        ("max_sample_splits", ctypes.c_int32),
    ]


class FhdError(RuntimeError):
    def __init__(self, status: int, detail: str):
        self.status = status
        super().__init__(f"{status_string(status)}: {detail}")


_lib = None


def load() -> ctypes.CDLL:
    """Load the HIP library once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(
            f"{LIB_PATH} is missing: build it with `python -m non_cartesian_mri_amd.build` "
            "(or __graft_entry__.build()); there is no CPU fallback")
    # torch's HIP runtime is loaded first, so the library binds to that same
    # runtime (by soname) instead of bringing in a second copy from the system
    import torch  # noqa: F401
    lib = ctypes.CDLL(LIB_PATH)
    P, i64, i32, sz = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_size_t
    lib.fhd_default_opts.argtypes = [ctypes.POINTER(FhdOpts)]
    lib.fhd_default_opts.restype = None
    lib.fhd_workspace_bytes.argtypes = [i64, i64, i32, i32, ctypes.POINTER(FhdOpts)]
    lib.fhd_workspace_bytes.restype = sz
    lib.fhd_compute.argtypes = [P, P, P, P, P, P, P, P, P, i64, i64, i32, ctypes.POINTER(FhdOpts), P]
    lib.fhd_compute.restype = ctypes.c_int
    lib.fhd_compute_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, i64, i64, i32, ctypes.POINTER(FhdOpts), P]
    lib.fhd_compute_noalloc.restype = ctypes.c_int
    lib.q_compute.argtypes = [P, P, P, P, P, P, P, P, i64, i64, ctypes.POINTER(FhdOpts), P]
    lib.q_compute.restype = ctypes.c_int
    lib.fhd_forward.argtypes = [P, P, P, P, P, P, P, P, P, i64, i64, i32, ctypes.POINTER(FhdOpts), P]
    lib.fhd_forward.restype = ctypes.c_int
    lib.fhd_toeplitz_bytes.argtypes = [i32, i32, i32]
    lib.fhd_toeplitz_bytes.restype = sz
    lib.fhd_toeplitz_kernel.argtypes = [P, P, P, P, i64, i32, i32, i32, P, ctypes.POINTER(FhdOpts), P]
    lib.fhd_toeplitz_kernel.restype = ctypes.c_int
    lib.fhd_cg_workspace_bytes.argtypes = [i32, i32, i32]
    lib.fhd_cg_workspace_bytes.restype = sz
    lib.fhd_normal_apply.argtypes = [P, i32, i32, i32, ctypes.c_float, P, P, P, sz, P]
    lib.fhd_normal_apply.restype = ctypes.c_int
    lib.fhd_cg_solve.argtypes = [P, i32, i32, i32, ctypes.c_float, P, P, i32, P, P, sz, P]
    lib.fhd_cg_solve.restype = ctypes.c_int
    lib.fhd_gridding.argtypes = [P, P, P, P, P, i64, i32, i32, i32, P, P]
    lib.fhd_gridding.restype = ctypes.c_int
    lib.fhd_describe_plan.argtypes = [i64, i64, i32, i32, ctypes.POINTER(FhdOpts), ctypes.POINTER(FhdPlanInfo)]
    lib.fhd_describe_plan.restype = ctypes.c_int
    lib.fhd_status_string.argtypes = [ctypes.c_int]
    lib.fhd_status_string.restype = ctypes.c_char_p
    lib.fhd_last_error.argtypes = []
    lib.fhd_last_error.restype = ctypes.c_char_p
    lib.fhd_version.argtypes = []
    lib.fhd_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().fhd_status_string(status).decode()


def last_error() -> str:
    return load().fhd_last_error().decode()


def check(status: int) -> None:
    if status != FHD_OK:
        raise FhdError(status, last_error())
