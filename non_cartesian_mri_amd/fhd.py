"""Python binding of the F^H D / Q library: argument marshalling only.

torch provides device memory and the stream; every step of the computation
runs in the HIP kernels behind the C ABI (include/fhd.h).  Names match the C
entry points: fhd_compute, fhd_compute_noalloc, q_compute, fhd_forward,
fhd_workspace_bytes, and the
reconstruction calls fhd_toeplitz_kernel, fhd_normal_apply, fhd_cg_solve.
"""
from __future__ import annotations

import ctypes

import torch

from . import _lib

_TRIG = {"accurate": _lib.FHD_TRIG_ACCURATE, "hw": _lib.FHD_TRIG_HW}
_SUM = {"blocked": _lib.FHD_SUM_BLOCKED, "kahan": _lib.FHD_SUM_KAHAN, "plain": _lib.FHD_SUM_PLAIN}
_ENGINE = {"auto": _lib.FHD_ENGINE_AUTO, "valu": _lib.FHD_ENGINE_VALU, "mfma": _lib.FHD_ENGINE_MFMA,
           "mfma16": _lib.FHD_ENGINE_MFMA16}
_STAGES = {"all": _lib.FHD_STAGE_ALL, "mu": _lib.FHD_STAGE_MU, "gather": _lib.FHD_STAGE_GATHER,
           "reduce": _lib.FHD_STAGE_REDUCE,
           "gather+reduce": _lib.FHD_STAGE_GATHER | _lib.FHD_STAGE_REDUCE}


def make_opts(trig="accurate", sum="blocked", voxels_per_lane=0, tile=0, stages="all",
              workspace: torch.Tensor | None = None, sample_splits=0, engine="auto",
              mirror_pairs=True) -> _lib.FhdOpts:
    o = _lib.FhdOpts()
    _lib.load().fhd_default_opts(ctypes.byref(o))
    o.trig = _TRIG[trig] if isinstance(trig, str) else int(trig)
    o.sum = _SUM[sum] if isinstance(sum, str) else int(sum)
    o.voxels_per_lane = int(voxels_per_lane)
    o.tile = int(tile)
    o.stages = _STAGES[stages] if isinstance(stages, str) else int(stages)
    o.sample_splits = int(sample_splits)
    o.engine = _ENGINE[engine] if isinstance(engine, str) else int(engine)
    o.flags = 0 if mirror_pairs else _lib.FHD_FLAG_NO_MIRROR_PAIRS
    if workspace is not None:
        o.workspace = workspace.data_ptr()
        o.workspace_bytes = workspace.numel() * workspace.element_size()
    return o


_OPS = {"fhd": _lib.FHD_OP_FHD, "q": _lib.FHD_OP_Q, "forward": _lib.FHD_OP_FORWARD}


def _op_code(is_q, op) -> int:
    if op is None:
        return _lib.FHD_OP_Q if is_q else _lib.FHD_OP_FHD
    return _OPS[op] if isinstance(op, str) else int(op)


def fhd_workspace_bytes(M: int, N: int, batch: int = 1, is_q: bool = False, op=None, **opts) -> int:
    """Workspace bytes of fhd_compute (default), q_compute (is_q) or op="forward"."""
    o = make_opts(**opts)
    return int(_lib.load().fhd_workspace_bytes(int(M), int(N), int(batch), _op_code(is_q, op),
                                               ctypes.byref(o)))


def fhd_describe_plan(M: int, N: int, batch: int = 1, is_q: bool = False, op=None, **opts) -> dict:
    """The launch plan (group size, tile, passes, record size, workspace) for these sizes."""
    o = make_opts(**opts)
    info = _lib.FhdPlanInfo()
    _lib.check(_lib.load().fhd_describe_plan(int(M), int(N), int(batch), _op_code(is_q, op),
                                             ctypes.byref(o), ctypes.byref(info)))
    return {k: getattr(info, k) for k, _ in _lib.FhdPlanInfo._fields_}


def resolved_voxels_per_lane(M: int, N: int, batch: int = 1, is_q: bool = False, **opts) -> int:
    return fhd_describe_plan(M, N, batch, is_q, **opts)["voxels_per_lane"]


def _dev_f32(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != torch.float32 or not t.is_contiguous() or t.dim() != 1:
        raise TypeError(f"{name} must be a contiguous 1-D float32 tensor")
    return t


def _dev_c64(t: torch.Tensor, name: str) -> torch.Tensor:
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != torch.complex64 or not t.is_contiguous():
        raise TypeError(f"{name} must be a contiguous complex64 tensor")
    return t


def _stream_ptr(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


def fhd_compute(kx, ky, kz, x, y, z, phi, D, *, trig="accurate", sum="blocked",
                voxels_per_lane=0, tile=0, stages="all", out=None, workspace=None,
                stream=None, sample_splits=0, engine="auto", mirror_pairs=True) -> torch.Tensor:
    """F^H D on the GPU.  D is complex64 [M] or [B, M]; returns complex64 [N] or [B, N].

    The work is enqueued on `stream` (default: torch's current stream).
    """
    for n, t in (("kx", kx), ("ky", ky), ("kz", kz), ("x", x), ("y", y), ("z", z)):
        _dev_f32(t, n)
    _dev_c64(phi, "phi")
    _dev_c64(D, "D")
    M, N = kx.numel(), x.numel()
    if not (ky.numel() == kz.numel() == phi.numel() == M) or not (y.numel() == z.numel() == N):
        raise ValueError("inconsistent sizes")
    squeeze = D.dim() == 1
    D2 = D.reshape(1, -1) if squeeze else D
    if D2.dim() != 2 or D2.shape[1] != M:
        raise ValueError("D must be [M] or [B, M]")
    B = D2.shape[0]
    if out is None:
        out = torch.empty((B, N), dtype=torch.complex64, device=x.device)
    else:
        _dev_c64(out, "out")
        if out.numel() != B * N:
            raise ValueError("out must hold B*N complex values")
    if workspace is None:
        nbytes = fhd_workspace_bytes(M, N, B, False, trig=trig, sum=sum,
                                     voxels_per_lane=voxels_per_lane, tile=tile,
                                     sample_splits=sample_splits, engine=engine,
                                     mirror_pairs=mirror_pairs)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    o = make_opts(trig, sum, voxels_per_lane, tile, stages, workspace, sample_splits, engine, mirror_pairs)
    st = _lib.load().fhd_compute(kx.data_ptr(), ky.data_ptr(), kz.data_ptr(), x.data_ptr(),
                                 y.data_ptr(), z.data_ptr(), phi.data_ptr(), D2.data_ptr(),
                                 out.data_ptr(), M, N, B, ctypes.byref(o), _stream_ptr(stream))
    _lib.check(st)
    return out.reshape(N) if squeeze else out.reshape(B, N)


def fhd_compute_noalloc(kx, ky, kz, x, y, z, phi, D, *, trig="accurate", sum="blocked",
                        voxels_per_lane=0, tile=0, out=None, stream=None, sample_splits=0,
                        engine="auto", mirror_pairs=True) -> torch.Tensor:
    """F^H D through the allocation-free entry point: the library's fixed device
    array is the workspace (no device allocation by the library).  Same
    arguments as fhd_compute without workspace and stages; pass `out` to keep
    the call itself free of allocations."""
    for n, t in (("kx", kx), ("ky", ky), ("kz", kz), ("x", x), ("y", y), ("z", z)):
        _dev_f32(t, n)
    _dev_c64(phi, "phi")
    _dev_c64(D, "D")
    M, N = kx.numel(), x.numel()
    if not (ky.numel() == kz.numel() == phi.numel() == M) or not (y.numel() == z.numel() == N):
        raise ValueError("inconsistent sizes")
    squeeze = D.dim() == 1
    D2 = D.reshape(1, -1) if squeeze else D
    if D2.dim() != 2 or D2.shape[1] != M:
        raise ValueError("D must be [M] or [B, M]")
    B = D2.shape[0]
    if out is None:
        out = torch.empty((B, N), dtype=torch.complex64, device=x.device)
    else:
        _dev_c64(out, "out")
        if out.numel() != B * N:
            raise ValueError("out must hold B*N complex values")
    o = make_opts(trig, sum, voxels_per_lane, tile, "all", None, sample_splits, engine, mirror_pairs)
    st = _lib.load().fhd_compute_noalloc(kx.data_ptr(), ky.data_ptr(), kz.data_ptr(), x.data_ptr(),
                                         y.data_ptr(), z.data_ptr(), phi.data_ptr(), D2.data_ptr(),
                                         out.data_ptr(), M, N, B, ctypes.byref(o), _stream_ptr(stream))
    _lib.check(st)
    return out.reshape(N) if squeeze else out.reshape(B, N)


def q_compute(kx, ky, kz, x, y, z, phi, *, trig="accurate", sum="blocked",
              voxels_per_lane=0, tile=0, stages="all", out=None, workspace=None,
              stream=None, sample_splits=0, engine="auto", mirror_pairs=True) -> torch.Tensor:
    """Q on the GPU: complex64 [N]."""
    for n, t in (("kx", kx), ("ky", ky), ("kz", kz), ("x", x), ("y", y), ("z", z)):
        _dev_f32(t, n)
    _dev_c64(phi, "phi")
    M, N = kx.numel(), x.numel()
    if not (ky.numel() == kz.numel() == phi.numel() == M) or not (y.numel() == z.numel() == N):
        raise ValueError("inconsistent sizes")
    if out is None:
        out = torch.empty(N, dtype=torch.complex64, device=x.device)
    else:
        _dev_c64(out, "out")
        if out.numel() != N:
            raise ValueError("out must hold N complex values")
    if workspace is None:
        nbytes = fhd_workspace_bytes(M, N, 1, True, trig=trig, sum=sum,
                                     voxels_per_lane=voxels_per_lane, tile=tile,
                                     sample_splits=sample_splits, engine=engine,
                                     mirror_pairs=mirror_pairs)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=x.device)
    o = make_opts(trig, sum, voxels_per_lane, tile, stages, workspace, sample_splits, engine, mirror_pairs)
    st = _lib.load().q_compute(kx.data_ptr(), ky.data_ptr(), kz.data_ptr(), x.data_ptr(),
                               y.data_ptr(), z.data_ptr(), phi.data_ptr(), out.data_ptr(),
                               M, N, ctypes.byref(o), _stream_ptr(stream))
    _lib.check(st)
    return out


def fhd_forward(kx, ky, kz, x, y, z, phi, rho, *, trig="accurate", sum="blocked",
                voxels_per_lane=0, tile=0, stages="all", out=None, workspace=None,
                stream=None, sample_splits=0, engine="auto", mirror_pairs=True) -> torch.Tensor:
    """F rho on the GPU: rho complex64 [N] or [B, N]; returns complex64 [M] or [B, M].

    D[b][m] = phi[m] sum_n rho[b][n] exp(-i 2 pi k_m . x_n), the adjoint of
    fhd_compute.  The work is enqueued on `stream` (default: torch's current stream).
    """
    for n, t in (("kx", kx), ("ky", ky), ("kz", kz), ("x", x), ("y", y), ("z", z)):
        _dev_f32(t, n)
    _dev_c64(phi, "phi")
    _dev_c64(rho, "rho")
    M, N = kx.numel(), x.numel()
    if not (ky.numel() == kz.numel() == phi.numel() == M) or not (y.numel() == z.numel() == N):
        raise ValueError("inconsistent sizes")
    squeeze = rho.dim() == 1
    R2 = rho.reshape(1, -1) if squeeze else rho
    if R2.dim() != 2 or R2.shape[1] != N:
        raise ValueError("rho must be [N] or [B, N]")
    B = R2.shape[0]
    if out is None:
        out = torch.empty((B, M), dtype=torch.complex64, device=kx.device)
    else:
        _dev_c64(out, "out")
        if out.numel() != B * M:
            raise ValueError("out must hold B*M complex values")
    if workspace is None:
        nbytes = fhd_workspace_bytes(M, N, B, op="forward", trig=trig, sum=sum,
                                     voxels_per_lane=voxels_per_lane, tile=tile,
                                     sample_splits=sample_splits, engine=engine,
                                     mirror_pairs=mirror_pairs)
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=kx.device)
    o = make_opts(trig, sum, voxels_per_lane, tile, stages, workspace, sample_splits, engine, mirror_pairs)
    st = _lib.load().fhd_forward(kx.data_ptr(), ky.data_ptr(), kz.data_ptr(), x.data_ptr(),
                                 y.data_ptr(), z.data_ptr(), phi.data_ptr(), R2.data_ptr(),
                                 out.data_ptr(), M, N, B, ctypes.byref(o), _stream_ptr(stream))
    _lib.check(st)
    return out.reshape(M) if squeeze else out.reshape(B, M)


def fhd_toeplitz_bytes(nx: int, ny: int, nz: int) -> int:
    return int(_lib.load().fhd_toeplitz_bytes(int(nx), int(ny), int(nz)))


def fhd_cg_workspace_bytes(nx: int, ny: int, nz: int) -> int:
    return int(_lib.load().fhd_cg_workspace_bytes(int(nx), int(ny), int(nz)))


def _grid(shape) -> tuple[int, int, int]:
    nz, ny, nx = (int(v) for v in shape)
    return nx, ny, nz


def toeplitz_lengths(shape) -> tuple[int, int, int]:
    """Transform lengths (pz, py, px) of an image grid (nz, ny, nx): powers of two >= 2n."""
    out = []
    for n in shape:
        p = 2
        while p < 2 * int(n):
            p *= 2
        out.append(p)
    return tuple(out)


def fhd_toeplitz_kernel(kx, ky, kz, phi, shape, *, trig="accurate", sum="blocked",
                        voxels_per_lane=0, tile=0, sample_splits=0, engine="auto",
                        out=None, stream=None, mirror_pairs=True) -> torch.Tensor:
    """Qhat for an image grid of `shape` = (nz, ny, nx): pz * py * px float32 values,
    returned as a [pz, py, px] tensor whose storage order is the library's
    (blocks of min(32, px py) consecutive (ky, kx) columns, kz-major within a
    block: see fhd_toeplitz_kernel in include/fhd.h).

    The (real) DFT of Q embedded in the padded grid of coordinate differences,
    divided by px py pz, so that fhd_normal_apply applies F^H F as a cyclic
    convolution.
    """
    for n, t in (("kx", kx), ("ky", ky), ("kz", kz)):
        _dev_f32(t, n)
    _dev_c64(phi, "phi")
    M = kx.numel()
    if not (ky.numel() == kz.numel() == phi.numel() == M):
        raise ValueError("inconsistent sizes")
    nx, ny, nz = _grid(shape)
    plen = toeplitz_lengths((nz, ny, nx))
    if out is None:
        out = torch.empty(plen, dtype=torch.float32, device=kx.device)
    else:
        if not isinstance(out, torch.Tensor) or not out.is_cuda or out.dtype != torch.float32 \
                or not out.is_contiguous():
            raise TypeError("out must be a contiguous float32 CUDA tensor")
        if out.numel() != plen[0] * plen[1] * plen[2]:
            raise ValueError("out must hold pz * py * px floats")
    o = make_opts(trig, sum, voxels_per_lane, tile, "all", None, sample_splits, engine, mirror_pairs)
    st = _lib.load().fhd_toeplitz_kernel(kx.data_ptr(), ky.data_ptr(), kz.data_ptr(), phi.data_ptr(),
                                         M, nx, ny, nz, out.data_ptr(), ctypes.byref(o),
                                         _stream_ptr(stream))
    _lib.check(st)
    return out


def _check_qhat(Qhat, nx, ny, nz):
    if not isinstance(Qhat, torch.Tensor) or not Qhat.is_cuda or Qhat.dtype != torch.float32 \
            or not Qhat.is_contiguous():
        raise TypeError("Qhat must be the contiguous float32 CUDA tensor of fhd_toeplitz_kernel")
    pz, py, px = toeplitz_lengths((nz, ny, nx))
    if Qhat.numel() != pz * py * px:
        raise ValueError("Qhat does not match the image grid")


def _cg_workspace(workspace, nx, ny, nz, device):
    if workspace is None:
        nbytes = fhd_cg_workspace_bytes(nx, ny, nz)
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def fhd_normal_apply(Qhat, p, lam=0.0, *, out=None, workspace=None, stream=None) -> torch.Tensor:
    """F^H F p + lam W^H W p for an image p of shape (nz, ny, nx) (complex64)."""
    _dev_c64(p, "p")
    if p.dim() != 3:
        raise ValueError("p must be [nz, ny, nx]")
    nx, ny, nz = _grid(p.shape)
    _check_qhat(Qhat, nx, ny, nz)
    if out is None:
        out = torch.empty_like(p)
    else:
        _dev_c64(out, "out")
        if out.numel() != p.numel():
            raise ValueError("out must match p")
    workspace, nbytes = _cg_workspace(workspace, nx, ny, nz, p.device)
    st = _lib.load().fhd_normal_apply(Qhat.data_ptr(), nx, ny, nz, float(lam), p.data_ptr(),
                                      out.data_ptr(), workspace.data_ptr(), nbytes, _stream_ptr(stream))
    _lib.check(st)
    return out


def fhd_cg_solve(Qhat, b, iters, lam=0.0, *, x0=None, out=None, resid=False, workspace=None,
                 stream=None):
    """`iters` CG iterations on (F^H F + lam W^H W) x = b, b of shape (nz, ny, nx).

    Starts from x0 (default zeros; never modified), or, when `out` is given,
    from the image in `out`, which is then updated in place.  Returns x, or
    (x, r) with r the float64 device tensor of <r, r> before and after each
    iteration.
    """
    _dev_c64(b, "b")
    if b.dim() != 3:
        raise ValueError("b must be [nz, ny, nx]")
    nx, ny, nz = _grid(b.shape)
    _check_qhat(Qhat, nx, ny, nz)
    if out is not None:
        if x0 is not None:
            raise ValueError("give x0 or out, not both")
        _dev_c64(out, "out")
        if out.shape != b.shape:
            raise ValueError("out must match b")
        x = out
    elif x0 is None:
        x = torch.zeros_like(b)
    else:
        _dev_c64(x0, "x0")
        if x0.shape != b.shape:
            raise ValueError("x0 must match b")
        x = x0.clone()
    r = torch.empty(int(iters) + 1, dtype=torch.float64, device=b.device) if resid else None
    workspace, nbytes = _cg_workspace(workspace, nx, ny, nz, b.device)
    st = _lib.load().fhd_cg_solve(Qhat.data_ptr(), nx, ny, nz, float(lam), b.data_ptr(), x.data_ptr(),
                                  int(iters), r.data_ptr() if r is not None else None,
                                  workspace.data_ptr(), nbytes, _stream_ptr(stream))
    _lib.check(st)
    return (x, r) if resid else x


def fhd_gridding(kx, ky, kz, phi, D, shape, *, out=None, stream=None) -> torch.Tensor:
    """Gridding reconstruction on a grid of `shape` = (nz, ny, nx) (powers of two):
    complex64 [nz, ny, nx] at voxel coordinates i - n/2 per axis."""
    for n, t in (("kx", kx), ("ky", ky), ("kz", kz)):
        _dev_f32(t, n)
    _dev_c64(phi, "phi")
    _dev_c64(D, "D")
    M = kx.numel()
    if not (ky.numel() == kz.numel() == phi.numel() == D.numel() == M):
        raise ValueError("inconsistent sizes")
    nx, ny, nz = _grid(shape)
    if out is None:
        out = torch.empty((nz, ny, nx), dtype=torch.complex64, device=kx.device)
    else:
        _dev_c64(out, "out")
        if out.numel() != nx * ny * nz:
            raise ValueError("out must hold nx ny nz complex values")
    st = _lib.load().fhd_gridding(kx.data_ptr(), ky.data_ptr(), kz.data_ptr(), phi.data_ptr(), D.data_ptr(), M,
                                  nx, ny, nz, out.data_ptr(), _stream_ptr(stream))
    _lib.check(st)
    return out
