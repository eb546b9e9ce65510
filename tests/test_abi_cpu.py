"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments before touching the device."""
import ctypes
import os
import re

import pytest

from non_cartesian_mri_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fhd.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.LIB_PATH):
        from non_cartesian_mri_amd.build import build_library
        build_library()
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    text = re.sub(r"^\s*#.*$", "", text, flags=re.M)   # preprocessor lines
    names = re.findall(r"\b([A-Za-z_]\w*)\s*\([^;{]*\)\s*;", text)
    return sorted(set(n for n in names if n not in ("sizeof",)))


def test_header_declarations_match_binding():
    assert sorted(_lib.EXPORTED) == _declared_functions()


def test_every_declared_symbol_is_exported(lib):
    for name in _declared_functions():
        assert hasattr(lib, name), name


def test_noalloc_scratch_size_matches_header():
    text = open(HEADER).read()
    m = re.search(r"#define FHD_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", text)
    assert m and int(m.group(1)) << int(m.group(2)) == _lib.NOALLOC_SCRATCH_BYTES


def test_opts_struct_layout(lib):
    # 8 int32 + pointer + size_t on LP64
    assert ctypes.sizeof(_lib.FhdOpts) == 48
    assert _lib.FhdOpts.workspace.offset == 32
    o = _lib.FhdOpts()
    o.trig = 77
    o.engine = 5
    lib.fhd_default_opts(ctypes.byref(o))
    assert (o.trig, o.sum, o.voxels_per_lane, o.tile, o.stages, o.sample_splits) == (0, 0, 0, 0, 7, 0)
    assert (o.engine, o.flags) == (_lib.FHD_ENGINE_AUTO, 0)
    assert o.workspace is None and o.workspace_bytes == 0
    assert ctypes.sizeof(_lib.FhdPlanInfo) == 48


def test_status_strings_and_version(lib):
    assert lib.fhd_status_string(0) == b"FHD_OK"
    assert lib.fhd_status_string(1) == b"FHD_ERR_INVALID_ARGUMENT"
    assert lib.fhd_status_string(2) == b"FHD_ERR_WORKSPACE"
    assert lib.fhd_status_string(99) == b"FHD_UNKNOWN_STATUS"
    assert b"gfx950" in lib.fhd_version()


def _opts(**kw):
    o = _lib.FhdOpts()
    _lib.load().fhd_default_opts(ctypes.byref(o))
    for k, v in kw.items():
        setattr(o, k, v)
    return o


# Fake, never dereferenced device addresses: every case below must be rejected
# by argument checks that run before any HIP call.
A = 1 << 40


def _fhd(lib, M=16, N=8, batch=1, opts=None, **ptrs):
    p = dict(kx=A, ky=A + 0x1000, kz=A + 0x2000, x=A + 0x3000, y=A + 0x4000, z=A + 0x5000,
             phi=A + 0x6000, D=A + 0x8000, out=A + 0x100000)
    p.update(ptrs)
    return lib.fhd_compute(p["kx"], p["ky"], p["kz"], p["x"], p["y"], p["z"], p["phi"], p["D"],
                           p["out"], M, N, batch, None if opts is None else ctypes.byref(opts), None)


@pytest.mark.parametrize("kw,err", [
    (dict(M=-1), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(N=-5), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(batch=0), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(batch=513), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(M=1 << 31), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(kx=None), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(D=None), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(out=None), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(x=None), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(out=A + 0x3000), _lib.FHD_ERR_INVALID_ARGUMENT),    # output aliases x
    (dict(out=A + 0x8000 + 64), _lib.FHD_ERR_INVALID_ARGUMENT),  # output inside D
])
def test_fhd_argument_errors(lib, kw, err):
    assert _fhd(lib, **kw) == err
    assert lib.fhd_last_error() != b""


def test_stage_combinations(lib):
    big = _opts(workspace=A + 0x10000000, workspace_bytes=1 << 30)
    # mu + reduce without the gather between them
    big.stages = _lib.FHD_STAGE_MU | _lib.FHD_STAGE_REDUCE
    assert _fhd(lib, opts=big) == _lib.FHD_ERR_INVALID_ARGUMENT
    # batch of 5 = two passes sharing one partial buffer: gather and reduce must run together
    for st in (_lib.FHD_STAGE_GATHER, _lib.FHD_STAGE_REDUCE, _lib.FHD_STAGE_MU | _lib.FHD_STAGE_GATHER):
        o = _opts(workspace=A + 0x10000000, workspace_bytes=1 << 30, stages=st, sample_splits=2)
        assert _fhd(lib, M=4096, batch=5, opts=o) == _lib.FHD_ERR_INVALID_ARGUMENT
        assert b"same call" in lib.fhd_last_error()


@pytest.mark.parametrize("field,value", [
    ("trig", 2), ("trig", -1), ("sum", 3), ("voxels_per_lane", 3), ("voxels_per_lane", 48),
    ("voxels_per_lane", 256),
    ("tile", -4), ("stages", 8), ("sample_splits", -1), ("sample_splits", 1025),
    ("engine", 4), ("engine", -1), ("flags", 2), ("flags", -1),
])
def test_bad_options(lib, field, value):
    assert _fhd(lib, opts=_opts(**{field: value})) == _lib.FHD_ERR_INVALID_ARGUMENT


def test_engine_option_conflicts(lib):
    E = _lib.FHD_ERR_INVALID_ARGUMENT
    # the matrix-core engine sums blocked or plain, and its group size is fixed
    assert _fhd(lib, opts=_opts(engine=_lib.FHD_ENGINE_MFMA, sum=_lib.FHD_SUM_KAHAN)) == E
    assert b"Kahan" in lib.fhd_last_error()
    assert _fhd(lib, opts=_opts(engine=_lib.FHD_ENGINE_MFMA, voxels_per_lane=4)) == E
    assert b"MFMA group sizes" in lib.fhd_last_error()
    assert _fhd(lib, opts=_opts(engine=_lib.FHD_ENGINE_VALU, voxels_per_lane=32)) == E
    assert b"VALU group sizes" in lib.fhd_last_error()
    # the half-split engine: blocked or plain sums, groups of 128 voxels, F^H D and Q only
    assert _fhd(lib, opts=_opts(engine=_lib.FHD_ENGINE_MFMA16, sum=_lib.FHD_SUM_KAHAN)) == E
    assert b"half-split" in lib.fhd_last_error()
    assert _fhd(lib, opts=_opts(engine=_lib.FHD_ENGINE_MFMA16, voxels_per_lane=64)) == E
    assert b"groups of 128" in lib.fhd_last_error()


def test_workspace_errors(lib):
    need = lib.fhd_workspace_bytes(16, 8, 1, 0, None)
    assert need > 0
    small = _opts(workspace=A + 0x200000, workspace_bytes=need - 1)
    assert _fhd(lib, opts=small) == _lib.FHD_ERR_WORKSPACE
    # a single stage needs a caller workspace
    assert _fhd(lib, opts=_opts(stages=_lib.FHD_STAGE_MU)) == _lib.FHD_ERR_WORKSPACE
    assert _fhd(lib, opts=_opts(stages=_lib.FHD_STAGE_REDUCE)) == _lib.FHD_ERR_WORKSPACE
    # misaligned workspace (records are read as 16-byte vectors)
    assert _fhd(lib, opts=_opts(workspace=A + 0x200008, workspace_bytes=need)) == _lib.FHD_ERR_INVALID_ARGUMENT
    assert b"aligned" in lib.fhd_last_error()
    # workspace overlapping an input or the output
    assert _fhd(lib, opts=_opts(workspace=A + 0x6000, workspace_bytes=need)) == _lib.FHD_ERR_INVALID_ARGUMENT
    assert _fhd(lib, opts=_opts(workspace=A + 0x100000, workspace_bytes=need)) == _lib.FHD_ERR_INVALID_ARGUMENT


def _noalloc(lib, M=16, N=8, batch=1, opts=None, **ptrs):
    p = dict(kx=A, ky=A + 0x1000, kz=A + 0x2000, x=A + 0x3000, y=A + 0x4000, z=A + 0x5000,
             phi=A + 0x6000, D=A + 0x8000, out=A + 0x100000)
    p.update(ptrs)
    return lib.fhd_compute_noalloc(p["kx"], p["ky"], p["kz"], p["x"], p["y"], p["z"], p["phi"], p["D"],
                                   p["out"], M, N, batch, None if opts is None else ctypes.byref(opts), None)


def test_noalloc_argument_errors(lib):
    """fhd_compute_noalloc checks its arguments as fhd_compute does, refuses a
    caller workspace or a partial stage mask, and refuses a plan larger than
    its fixed array -- all before any device call."""
    E = _lib.FHD_ERR_INVALID_ARGUMENT
    assert _noalloc(lib, M=-1) == E
    assert _noalloc(lib, kx=None) == E
    assert _noalloc(lib, out=A + 0x3000) == E
    assert _noalloc(lib, opts=_opts(trig=7)) == E
    assert _noalloc(lib, opts=_opts(workspace=A + 0x200000, workspace_bytes=1 << 20)) == E
    assert b"workspace must be NULL" in lib.fhd_last_error()
    assert _noalloc(lib, opts=_opts(stages=_lib.FHD_STAGE_MU)) == E
    assert b"all stages" in lib.fhd_last_error()
    # 2^22 samples on the four-sample engine: 6.4 GB of factor records even with one row
    big = dict(M=1 << 22, N=1 << 21, D=A + 0x40000000, out=A + 0x80000000,
               x=A + 0x10000000, y=A + 0x18000000, z=A + 0x20000000, phi=A + 0x30000000)
    assert _noalloc(lib, **big) == _lib.FHD_ERR_WORKSPACE
    assert b"at most 536870912" in lib.fhd_last_error()
    assert _noalloc(lib, opts=_opts(sample_splits=1, engine=_lib.FHD_ENGINE_MFMA), **big) == _lib.FHD_ERR_WORKSPACE
    # N == 0 is a no-op before any device call, as for fhd_compute
    assert _noalloc(lib, N=0, x=None, y=None, z=None, out=None) == _lib.FHD_OK


def test_empty_voxel_set_is_a_noop(lib):
    # N == 0 returns before any device call
    assert _fhd(lib, N=0, x=None, y=None, z=None, out=None) == _lib.FHD_OK
    assert lib.q_compute(A, A + 0x1000, A + 0x2000, None, None, None, A + 0x6000, None, 16, 0,
                         None, None) == _lib.FHD_OK


def test_q_argument_errors(lib):
    E = _lib.FHD_ERR_INVALID_ARGUMENT
    assert lib.q_compute(None, A, A, A + 0x3000, A + 0x4000, A + 0x5000, A + 0x6000, A + 0x100000, 4, 4, None, None) == E
    assert lib.q_compute(A, A, A, A + 0x3000, A + 0x4000, A + 0x5000, A + 0x6000, A + 0x3000, 4, 4, None, None) == E
    assert lib.q_compute(A, A, A, A + 0x3000, A + 0x4000, A + 0x5000, A + 0x6000, A + 0x100000, -4, 4, None, None) == E


def test_workspace_bytes(lib):
    # records: mpad * stride dwords, 256-byte aligned per pass
    def ws(M, N, batch=1, is_q=0, **kw):
        kw.setdefault("sample_splits", 1)
        kw.setdefault("engine", _lib.FHD_ENGINE_VALU)
        return lib.fhd_workspace_bytes(M, N, batch, is_q, ctypes.byref(_opts(**kw)))
    assert ws(-1, 4) == 0
    assert ws(4, 4, batch=0) == 0
    assert ws(0, 100) == 0
    # HW trig, V=1, one vector: 3 header + 3 weights -> 8 dwords (padded to 4)
    assert ws(1000, 1, trig=1, voxels_per_lane=1) == (1000 * 8 * 4 + 255) // 256 * 256
    # accurate trig, V=8: 6 + 24 = 30 -> 32 dwords
    assert ws(1001, 4096, voxels_per_lane=8) == (1004 * 32 * 4 + 255) // 256 * 256
    # Q, HW, V=4: 3 + 1 + 9 = 13 -> 16 dwords
    assert ws(8, 64, is_q=1, trig=1, voxels_per_lane=4) == 8 * 16 * 4 // 256 * 256 + 256 * (8 * 16 * 4 % 256 > 0)
    # batch 5 = passes of 4 and 1 vectors, V forced to 1 (HW): strides 3+12->16 and 3+3->8
    assert ws(100, 50, batch=5, trig=1) == (100 * 16 * 4 + 255) // 256 * 256 + (100 * 8 * 4 + 255) // 256 * 256
    # 3 sample splits add one [3][4][50] complex partial buffer shared by the passes
    assert ws(1000, 50, batch=5, trig=1, sample_splits=3) == ((1000 * 16 * 4 + 255) // 256 * 256 + (1000 * 8 * 4 + 255) // 256 * 256
                                                             + (3 * 4 * 50 * 8 + 255) // 256 * 256)


def test_workspace_bytes_mfma(lib):
    # per pass: header [mpad][4 or 8] floats (256-aligned) + factors [mpad][48 T] floats (three per complex column; T = 2 on 16^3),
    # mpad = M rounded up to the 32-sample chunk
    def ws(M, N, batch=1, is_q=0, **kw):
        kw.setdefault("sample_splits", 1)
        kw.setdefault("engine", _lib.FHD_ENGINE_MFMA)
        return lib.fhd_workspace_bytes(M, N, batch, is_q, ctypes.byref(_opts(**kw)))
    a256 = lambda b: (b + 255) // 256 * 256
    # plus one int32 regularity flag per gather wave (groups of V = 16 T / BC, 32 groups
    # per wave for T = 2, 4 and 16 for T = 8): 16^3 with T = 2 -> 4 waves, one 256-byte block
    fl = a256(4 * 4)
    assert ws(1000, 4096, trig=1) == a256(1024 * 16) + 1024 * 384 + fl
    assert ws(1000, 4096) == a256(1024 * 32) + 1024 * 384 + fl       # accurate: 8 header floats
    assert ws(1000, 4096, is_q=1, trig=1) == a256(1024 * 16) + 1024 * 384 + fl
    assert ws(33, 4096, trig=1) == a256(64 * 16) + 64 * 384 + fl
    # batch 5: passes of 4 and 1 vectors, same record size; 3 splits add [3][4][N] partials;
    # the passes share the flags (one wave each here)
    one = a256(1024 * 16) + 1024 * 384
    assert ws(1000, 50, batch=5, trig=1) == 2 * one + a256(4)
    assert ws(1000, 50, batch=5, trig=1, sample_splits=3) == 2 * one + a256(3 * 4 * 50 * 8) + a256(4)
    # the default engine is the matrix-core one
    assert lib.fhd_workspace_bytes(1000, 4096, 1, 0, ctypes.byref(_opts(trig=1, sample_splits=1))) == ws(1000, 4096, trig=1)
    assert lib.fhd_workspace_bytes(1000, 4096, 1, 0, ctypes.byref(_opts(trig=1, sample_splits=1, sum=1))) == \
        ws(1000, 4096, trig=1, engine=_lib.FHD_ENGINE_VALU, sum=1)


def test_describe_plan_valu(lib):
    from non_cartesian_mri_amd.fhd import fhd_describe_plan as plan

    def fhd_describe_plan(*a, **kw):
        kw.setdefault("engine", "valu")
        r = plan(*a, **kw)
        assert r["engine"] == _lib.FHD_ENGINE_VALU
        return r
    # the 128^3 benchmark shape: 16 voxels per lane on both trig paths
    hw = fhd_describe_plan(262144, 128 ** 3, trig="hw")
    acc = fhd_describe_plan(262144, 128 ** 3, trig="accurate")
    assert hw["voxels_per_lane"] == 16 and acc["voxels_per_lane"] == 16
    assert hw["record_dwords"] == 52 and acc["record_dwords"] == 56
    assert hw["workspace_bytes"] == lib.fhd_workspace_bytes(262144, 128 ** 3, 1, 0, ctypes.byref(_opts(trig=1, engine=1)))
    assert hw["padded_samples"] == 262144 and hw["passes"] == 1
    # 262,144 samples -> 16 rows of 16384 samples
    assert hw["sample_splits"] == 16
    assert hw["workspace_bytes"] == 262144 * 52 * 4 + 16 * 128 ** 3 * 8
    # small voxel sets are filled by splitting the samples (>= 256 samples per split)
    assert fhd_describe_plan(65536, 64 ** 3, trig="hw")["sample_splits"] == 48
    tiny = fhd_describe_plan(2048, 32 ** 3, trig="hw")
    assert tiny["voxels_per_lane"] == 1 and tiny["sample_splits"] == 8
    assert fhd_describe_plan(1000, 5, trig="hw")["sample_splits"] == 3
    # batched: 31 rows of 16384 samples wanted, partial sums capped at 2 GiB -> 18
    assert fhd_describe_plan(500001, 96 ** 3, batch=16)["sample_splits"] == 18
    # short sample lists with plenty of voxels: one row
    assert fhd_describe_plan(4096, 256 ** 3)["sample_splits"] == 1
    # explicit and plain-sum choices
    assert fhd_describe_plan(262144, 128 ** 3, sample_splits=5)["sample_splits"] == 5
    assert fhd_describe_plan(262144, 128 ** 3, sum="plain")["sample_splits"] == 1
    assert fhd_describe_plan(10, 4096, sample_splits=7)["sample_splits"] == 3  # no empty rows (12 padded samples)
    assert fhd_describe_plan(0, 4096)["sample_splits"] == 1
    # tiny N shrinks the group; batches force one voxel per lane and split into passes
    assert fhd_describe_plan(1000, 5, trig="hw")["voxels_per_lane"] == 1  # cannot fill the GPU anyway
    assert fhd_describe_plan(1000, 5, trig="hw", voxels_per_lane=1)["voxels_per_lane"] == 1
    b = fhd_describe_plan(500001, 96 ** 3, batch=19)
    assert b["voxels_per_lane"] == 1 and b["passes"] == 3 and b["padded_samples"] == 500004
    assert fhd_describe_plan(1000, 100, sum="plain")["tile"] == 1000
    info = _lib.FhdPlanInfo()
    assert lib.fhd_describe_plan(-1, 4, 1, 0, None, ctypes.byref(info)) == _lib.FHD_ERR_INVALID_ARGUMENT
    assert lib.fhd_describe_plan(4, 4, 1, 0, None, None) == _lib.FHD_ERR_INVALID_ARGUMENT


def test_describe_plan_half_split(lib):
    from non_cartesian_mri_amd.fhd import fhd_describe_plan, fhd_workspace_bytes
    # groups of 128 / vectors voxels; the HW path sums each launch row as one
    # block (tile = the row), the accurate path folds tiles of ~sqrt(M);
    # records: header + 1536 bytes of fp16 factor parts + Mu of each vector in fp32
    for trig, hf in (("hw", 4), ("accurate", 8)):
        p = fhd_describe_plan(262144, 128 ** 3, engine="mfma16", trig=trig)
        assert p["engine"] == _lib.FHD_ENGINE_MFMA16 and p["voxels_per_lane"] == 128
        assert p["record_dwords"] == hf + 384 + 2
        assert p["padded_samples"] == 262144
        assert p["tile"] == (262144 // p["sample_splits"] if trig == "hw" else 512)
    b = fhd_describe_plan(500001, 96 ** 3, 16, engine="mfma16")
    assert b["voxels_per_lane"] == 8 and b["passes"] == 1 and b["padded_samples"] == 500032
    assert fhd_describe_plan(1000, 100, engine="mfma16", sum="plain")["sample_splits"] == 1
    # workspace: headers, factor parts, Mu, the scale pair, partial sums, flags
    assert fhd_workspace_bytes(262144, 128 ** 3, engine="mfma16", trig="accurate") == p["workspace_bytes"] > 0
    # the forward operator: groups of 128 / vectors voxels; fp16 parts of the
    # packed image (gpad x 1536 bytes), the gather's headers (gpad x 16) and the
    # scale beside the fp32 workspace
    f = fhd_describe_plan(262144, 128 ** 3, op="forward", engine="mfma16", trig="hw")
    f32 = fhd_describe_plan(262144, 128 ** 3, op="forward", engine="mfma", trig="hw", mirror_pairs=False)
    assert f["engine"] == _lib.FHD_ENGINE_MFMA16 and f["voxels_per_lane"] == 128
    assert f["workspace_bytes"] - f32["workspace_bytes"] == 16384 * 1536 + 16384 * 16 + 1280
    # one launch row of all 16,384 groups: HW sums it as one block, accurate folds ~sqrt(G)
    assert f["sample_splits"] == 1 and f["tile"] == 16384
    assert fhd_describe_plan(262144, 128 ** 3, op="forward", engine="mfma16", trig="accurate")["tile"] == 128
    # rows beyond 256 MB of packed groups fold tiles, as on the fp32 engine (512^3: 1.6 GB)
    assert fhd_describe_plan(262144, 512 ** 3, op="forward", engine="mfma16", trig="hw")["tile"] == 4096
    with pytest.raises(Exception):
        fhd_describe_plan(1000, 4096, op="forward", engine="mfma16", voxels_per_lane=64)
    with pytest.raises(Exception):
        fhd_describe_plan(1000, 4096, op="forward", engine="valu")


def test_describe_plan_mfma(lib):
    from non_cartesian_mri_amd.fhd import fhd_describe_plan
    # the 128^3 benchmark shape: a cube whose edge is a multiple of 128 -> T = 8
    # units of 16 complex columns per group phase, groups of 128 voxels (one
    # row), the four-sample engine
    hw = fhd_describe_plan(262144, 128 ** 3, trig="hw")
    acc = fhd_describe_plan(262144, 128 ** 3, trig="accurate")
    assert hw["engine"] == acc["engine"] == _lib.FHD_ENGINE_MFMA
    assert hw["voxels_per_lane"] == 128 and acc["voxels_per_lane"] == 128
    assert hw["record_dwords"] == 4 + 384 and acc["record_dwords"] == 8 + 384
    # tile ~sqrt(M) for the accurate path; the four-sample engine's HW path
    # sums a whole launch row (16,384 samples) as one block
    assert hw["padded_samples"] == 262144 and hw["passes"] == 1 and hw["tile"] == 16384
    # (the accurate path's ~sqrt(M) tile, raised to 2048 samples where the
    # mirror-pair gather writes each block's sums to memory)
    assert acc["tile"] == 2048
    assert fhd_describe_plan(262144, 128 ** 3, trig="accurate", mirror_pairs=False)["tile"] == 512
    # 1024 waves of 16 groups; 16 rows of 16384 samples
    assert hw["sample_splits"] == 16
    # the HW path pairs mirror groups and picks its rows on the device, at most
    # twice the automatic count: headers, factors, 32 rows of partial sums, 1024
    # per-wave flags, the pair plan (16 int32 header, one int2 per group)
    assert hw["mirror_pairs"] == 1 and hw["max_sample_splits"] == 32
    assert acc["mirror_pairs"] == 1 and acc["sample_splits"] == 16 and acc["max_sample_splits"] == 32
    assert hw["workspace_bytes"] == 262144 * 16 + 262144 * 1536 + 32 * 128 ** 3 * 8 + 1024 * 4 + ((64 + 16384 * 8 + 15) // 16 * 16 + 16384 * 16 + 255) // 256 * 256
    off = fhd_describe_plan(262144, 128 ** 3, trig="hw", mirror_pairs=False)
    assert off["mirror_pairs"] == 0 and off["max_sample_splits"] == 16
    assert off["workspace_bytes"] == 262144 * 16 + 262144 * 1536 + 16 * 128 ** 3 * 8 + 1024 * 4
    fixed = fhd_describe_plan(262144, 128 ** 3, trig="hw", sample_splits=12)
    assert fixed["mirror_pairs"] == 1 and fixed["max_sample_splits"] == fixed["sample_splits"] == 12
    # groups of 64 (T = 4) or 32 (T = 2) on request, two-sample engine
    four = fhd_describe_plan(262144, 128 ** 3, trig="hw", voxels_per_lane=64)
    assert four["voxels_per_lane"] == 64 and four["record_dwords"] == 4 + 192
    assert four["workspace_bytes"] == 262144 * 16 + 262144 * 768 + 16 * 128 ** 3 * 8 + 1024 * 4
    two = fhd_describe_plan(262144, 128 ** 3, trig="hw", voxels_per_lane=32)
    assert two["voxels_per_lane"] == 32 and two["record_dwords"] == 4 + 96 and two["engine"] == _lib.FHD_ENGINE_MFMA
    assert two["workspace_bytes"] == 262144 * 16 + 262144 * 384 + 16 * 128 ** 3 * 8 + 2048 * 4
    assert fhd_describe_plan(1000, 96 ** 3, trig="hw")["voxels_per_lane"] == 32
    assert fhd_describe_plan(1000, 100, trig="hw")["voxels_per_lane"] == 32     # not a cube
    # 64^3: groups of 128 = two whole rows of a plane (regular); 128 waves x 16 rows
    # fill 2 waves per SIMD
    m64 = fhd_describe_plan(65536, 64 ** 3, trig="hw")
    assert m64["voxels_per_lane"] == 128 and m64["sample_splits"] == 16
    # 32^3 x 2048: regular for every group size, but even 16 rows (of 128
    # samples, the shortest a matrix-core row takes) of the fewest, longest
    # waves cannot fill the GPU -> the smallest groups, and the most rows
    tiny = fhd_describe_plan(2048, 32 ** 3, trig="hw")
    assert tiny["voxels_per_lane"] == 32 and tiny["sample_splits"] == 16 and tiny["tile"] == 256
    # 48^3: 128 and 64 are neither divisors of a row nor whole rows of a plane
    assert fhd_describe_plan(65536, 48 ** 3, trig="hw")["voxels_per_lane"] == 32
    # fewer voxels than one group: still one wave; samples padded to the 32-sample chunk
    small = fhd_describe_plan(1000, 5, trig="hw")
    assert small["padded_samples"] == 1024 and small["sample_splits"] == 8
    # batched, 16 vectors on 96^3: T = 8, groups of 8 voxels; the partial buffer cap gives 18 rows
    b16 = fhd_describe_plan(500001, 96 ** 3, batch=16)
    assert b16["voxels_per_lane"] == 8 and b16["sample_splits"] == 18 and b16["padded_samples"] == 500032
    assert b16["record_dwords"] == 8 + 384
    # 19 = 16 + 2 + 1 vectors: the single-vector pass needs 32 | 96, so T = 2 for all passes
    b19 = fhd_describe_plan(500001, 96 ** 3, batch=19)
    assert b19["passes"] == 3 and b19["voxels_per_lane"] == 2
    q = fhd_describe_plan(1048576, 128 ** 3, is_q=True, trig="hw")
    assert q["voxels_per_lane"] == 128 and q["sample_splits"] == 64
    # the forward operator at 128^3: groups of 128 (the four-group engine)
    assert fhd_describe_plan(262144, 128 ** 3, op="forward", trig="hw")["voxels_per_lane"] == 128


def test_describe_plan_zero_sizes(lib):
    """Empty voxel or sample sets plan one row and no partial buffer (no division by zero)."""
    from non_cartesian_mri_amd.fhd import fhd_describe_plan
    for M, N in ((100, 0), (0, 0), (0, 100)):
        for is_q in (False, True):
            r = fhd_describe_plan(M, N, is_q=is_q, trig="hw")
            assert r["sample_splits"] == 1
    assert fhd_describe_plan(100, 0, engine="valu")["workspace_bytes"] == (100 * 12 * 4 + 255) // 256 * 256
    assert fhd_describe_plan(100, 0)["workspace_bytes"] == 128 * 32 + 128 * 384


# ----------------------------- forward operator -----------------------------
def _fwd(lib, M=16, N=8, batch=1, opts=None, **ptrs):
    p = dict(kx=A, ky=A + 0x1000, kz=A + 0x2000, x=A + 0x3000, y=A + 0x4000, z=A + 0x5000,
             phi=A + 0x6000, rho=A + 0x8000, out=A + 0x100000)
    p.update(ptrs)
    return lib.fhd_forward(p["kx"], p["ky"], p["kz"], p["x"], p["y"], p["z"], p["phi"], p["rho"],
                           p["out"], M, N, batch, None if opts is None else ctypes.byref(opts), None)


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(N=-1), dict(batch=0), dict(kx=None), dict(phi=None), dict(out=None),
    dict(x=None), dict(rho=None), dict(out=A + 0x8000 + 8),      # output inside rho
    dict(out=A + 0x1000),                                         # output aliases ky
])
def test_forward_argument_errors(lib, kw):
    assert _fwd(lib, **kw) == _lib.FHD_ERR_INVALID_ARGUMENT
    assert lib.fhd_last_error() != b""


@pytest.mark.parametrize("field,value,text", [
    ("engine", _lib.FHD_ENGINE_VALU, b"MFMA engine only"),
    ("sum", _lib.FHD_SUM_KAHAN, b"not Kahan"),
    ("voxels_per_lane", 8, b"group sizes"),
])
def test_forward_option_errors(lib, field, value, text):
    assert _fwd(lib, opts=_opts(**{field: value})) == _lib.FHD_ERR_INVALID_ARGUMENT
    assert text in lib.fhd_last_error()


def test_forward_empty_sample_set_is_a_noop(lib):
    assert _fwd(lib, M=0, kx=None, ky=None, kz=None, phi=None, out=None) == _lib.FHD_OK


def test_forward_plan(lib):
    from non_cartesian_mri_amd.fhd import fhd_describe_plan, fhd_workspace_bytes
    a256 = lambda b: (b + 255) // 256 * 256
    # 128^3: T = 8, groups of 128 voxels -> 16,384 groups; 16,384 waves of 16 samples fill the GPU
    p = fhd_describe_plan(262144, 128 ** 3, op="forward", trig="hw", mirror_pairs=False)
    assert p["engine"] == _lib.FHD_ENGINE_MFMA and p["voxels_per_lane"] == 128
    assert p["record_dwords"] == 4 + 384 and p["padded_samples"] == 262144
    # HW trig: the launch row (all 16,384 groups) is one summation block
    assert p["sample_splits"] == 1 and p["tile"] == 16384
    # accurate trig keeps ~sqrt(groups) per tile; so does HW with rows of more
    # than 256 MiB of packed groups (512^3: 1.6 GB per row, ~4 sqrt(G))
    assert fhd_describe_plan(262144, 512 ** 3, op="forward", trig="hw", mirror_pairs=False)["tile"] == 4096
    # the 16-image pass on 96^3 (groups of 8 voxels: 110,592 groups, 170 MB per
    # row) is one block per row
    b16 = fhd_describe_plan(500001, 96 ** 3, batch=16, op="forward", trig="hw", mirror_pairs=False)
    assert b16["sample_splits"] == 1 and b16["tile"] == 110592 and b16["voxels_per_lane"] == 8
    assert fhd_describe_plan(262144, 128 ** 3, op="forward", trig="accurate", mirror_pairs=False)["tile"] == 128
    pas = lambda g, T: a256(a256(g * 16) + a256(g * 192 * T) + 4 * (g + 1))
    assert p["workspace_bytes"] == pas(16384, 8)
    # groups of 64 on request: the pair engine, 32,768 groups
    p64 = fhd_describe_plan(262144, 128 ** 3, op="forward", trig="hw", voxels_per_lane=64)
    assert p64["record_dwords"] == 4 + 192 and p64["tile"] == 1024 and p64["workspace_bytes"] == pas(32768, 4)
    assert fhd_workspace_bytes(262144, 128 ** 3, op="forward", trig="hw", mirror_pairs=False) == p["workspace_bytes"]
    # mirror pairs (the default with T = 8): entry headers, entries of 64 T floats
    # (rho_g + rho_h, rho_g - rho_h), the list of groups of irregular waves, the
    # wave flags and the pair plan; each launch row one block of at most 16,384
    # (HW) or 2,048 (accurate) entries over the partial sums
    plan_b = lambda g: ((64 + 8 * g + 15) // 16 * 16) + 16 * g
    pp = lambda g, gpad: a256(a256(gpad * 16) + a256(gpad * 64 * 8 * 4) + a256(4 * (gpad + 1)) +
                              a256(4 * ((g + 15) // 16)) + plan_b(g))
    q = fhd_describe_plan(262144, 128 ** 3, op="forward", trig="hw")
    assert q["sample_splits"] == 1 and q["tile"] == 16384 and q["workspace_bytes"] == pp(16384, 16384)
    qa = fhd_describe_plan(262144, 128 ** 3, op="forward", trig="accurate")
    assert qa["sample_splits"] == 8 and qa["tile"] == 2048
    assert qa["workspace_bytes"] == pp(16384, 16384) + a256(8 * 262144 * 8)
    q512 = fhd_describe_plan(262144, 512 ** 3, op="forward", trig="hw")
    assert q512["sample_splits"] == 64 and q512["tile"] == 16384
    q16 = fhd_describe_plan(500001, 96 ** 3, batch=16, op="forward", trig="hw")
    assert q16["sample_splits"] == 7 and q16["tile"] == 16384
    # 32^3 x 2048 samples: 64 waves; rows over the 1024 groups (at least 64 groups each)
    s = fhd_describe_plan(2048, 32 ** 3, op="forward", trig="hw")
    assert s["voxels_per_lane"] == 32 and s["sample_splits"] == 16 and s["tile"] == 128
    assert s["workspace_bytes"] == pas(1024, 2) + a256(16 * 2048 * 8)
    # batch 3 on 64^3: passes of 2 and 1 images, T = 8: groups of 64 and 128 voxels
    # (128 = two rows of a plane)
    b = fhd_describe_plan(5000, 64 ** 3, batch=3, op="forward", trig="hw", sample_splits=1, mirror_pairs=False)
    assert b["passes"] == 2 and b["voxels_per_lane"] == 64 and b["tile"] == 4096
    assert b["workspace_bytes"] == pas(4096, 8) + pas(2048, 8)
    # with groups of 32 per image on request (T = 2): groups of 16 and 32
    b2 = fhd_describe_plan(5000, 64 ** 3, batch=3, op="forward", trig="hw", sample_splits=1, voxels_per_lane=32)
    assert b2["voxels_per_lane"] == 16 and b2["workspace_bytes"] == pas(16384, 2) + pas(8192, 2)
    # explicit group size, plain sum (one row, one tile)
    g = fhd_describe_plan(1000, 128 ** 3, op="forward", voxels_per_lane=32, sum="plain")
    assert g["voxels_per_lane"] == 32 and g["sample_splits"] == 1 and g["tile"] == 65536
    # no voxels: nothing to pack
    assert fhd_describe_plan(1000, 0, op="forward")["workspace_bytes"] == 0
    info = _lib.FhdPlanInfo()
    assert lib.fhd_describe_plan(10, 10, 1, 3, None, ctypes.byref(info)) == _lib.FHD_ERR_INVALID_ARGUMENT
    assert b"operation" in lib.fhd_last_error()


# --- reconstruction entry points (Toeplitz kernel, normal operator, CG) ---

def test_reconstruction_sizes(lib):
    a256 = lambda b: (b + 255) // 256 * 256
    # transform lengths: smallest powers of two >= 2n -> 8, 16, 16
    assert lib.fhd_toeplitz_bytes(4, 5, 6) == 8 * 16 * 16 * 4
    assert lib.fhd_toeplitz_bytes(0, 5, 6) == 0
    assert lib.fhd_toeplitz_bytes(513, 2, 2) == 0            # at most 512 voxels per axis
    assert lib.fhd_toeplitz_bytes(512, 512, 512) == 1024 ** 3 * 4
    n = 4 * 5 * 6
    # two working grids nz x py x px, three images, two sets of 1024 partial sums, CG state
    assert lib.fhd_cg_workspace_bytes(4, 5, 6) == (2 * a256(6 * 16 * 8 * 8) + 3 * a256(8 * n) + 2 * a256(8 * 1024)
                                                    + a256(64))
    assert lib.fhd_cg_workspace_bytes(4, -1, 6) == 0
    assert lib.fhd_cg_workspace_bytes(1, 1, 1) == 2 * a256(2 * 2 * 8) + 3 * 256 + 2 * 8192 + 256


def _toe(lib, M=16, nx=4, ny=4, nz=4, opts=None, **ptrs):
    p = dict(kx=A, ky=A + 0x1000, kz=A + 0x2000, phi=A + 0x6000, out=A + 0x100000)
    p.update(ptrs)
    return lib.fhd_toeplitz_kernel(p["kx"], p["ky"], p["kz"], p["phi"], M, nx, ny, nz, p["out"],
                                   None if opts is None else ctypes.byref(opts), None)


@pytest.mark.parametrize("kw", [
    dict(M=-1), dict(nx=0), dict(nz=-3), dict(nx=513), dict(ny=1024),    # at most 512 per axis
    dict(kx=None), dict(phi=None), dict(out=None),
    dict(out=A + 0x6000 + 8),                                              # Qhat overlaps phi
    dict(opts=dict(workspace=A + 0x200000, workspace_bytes=1 << 20)),      # no workspace here
    dict(opts=dict(stages=_lib.FHD_STAGE_MU)),
])
def test_toeplitz_argument_errors(lib, kw):
    # option structs are built here, not at collection: loading the library
    # must not happen before a test runs
    kw = dict(kw)
    if "opts" in kw:
        kw["opts"] = _opts(**kw["opts"])
    assert _toe(lib, **kw) == _lib.FHD_ERR_INVALID_ARGUMENT
    assert lib.fhd_last_error() != b""


CG_WS = A + 0x10000000


def _normal(lib, nx=4, ny=4, nz=4, lam=0.5, ws_bytes=None, **ptrs):
    p = dict(Q=A, p=A + 0x100000, Ap=A + 0x200000, ws=CG_WS)
    p.update(ptrs)
    nb = lib.fhd_cg_workspace_bytes(nx, ny, nz) if ws_bytes is None else ws_bytes
    return lib.fhd_normal_apply(p["Q"], nx, ny, nz, lam, p["p"], p["Ap"], p["ws"], nb, None)


def _cg(lib, nx=4, ny=4, nz=4, lam=0.5, iters=3, ws_bytes=None, **ptrs):
    p = dict(Q=A, b=A + 0x100000, x=A + 0x200000, r=A + 0x300000, ws=CG_WS)
    p.update(ptrs)
    nb = lib.fhd_cg_workspace_bytes(nx, ny, nz) if ws_bytes is None else ws_bytes
    return lib.fhd_cg_solve(p["Q"], nx, ny, nz, lam, p["b"], p["x"], iters, p["r"], p["ws"], nb, None)


@pytest.mark.parametrize("kw,status", [
    (dict(nx=0), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(nz=600), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(lam=float("inf")), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(Q=None), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(p=None), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(lam=-1.0), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(lam=float("nan")), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(ws=None), _lib.FHD_ERR_WORKSPACE),
    (dict(ws_bytes=1000), _lib.FHD_ERR_WORKSPACE),
    (dict(ws=CG_WS + 8), _lib.FHD_ERR_INVALID_ARGUMENT),                 # misaligned
    (dict(Ap=A + 0x100000 + 64), _lib.FHD_ERR_INVALID_ARGUMENT),         # Ap overlaps p
    (dict(ws=A + 0x200000 - 256), _lib.FHD_ERR_INVALID_ARGUMENT),        # workspace overlaps Ap
])
def test_normal_apply_argument_errors(lib, kw, status):
    assert _normal(lib, **kw) == status
    assert lib.fhd_last_error() != b""


@pytest.mark.parametrize("kw,status", [
    (dict(ny=0), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(b=None), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(x=None), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(iters=-1), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(lam=-0.5), _lib.FHD_ERR_INVALID_ARGUMENT),
    (dict(ws_bytes=8), _lib.FHD_ERR_WORKSPACE),
    (dict(x=A + 0x100000), _lib.FHD_ERR_INVALID_ARGUMENT),               # x aliases b
    (dict(r=A + 0x200000 + 8), _lib.FHD_ERR_INVALID_ARGUMENT),           # resid inside x
    (dict(x=A + 8), _lib.FHD_ERR_INVALID_ARGUMENT),                      # x inside Qhat
])
def test_cg_argument_errors(lib, kw, status):
    assert _cg(lib, **kw) == status
    assert lib.fhd_last_error() != b""


def _grid(lib, M=16, nx=8, ny=8, nz=8, **ptrs):
    p = dict(kx=A, ky=A + 0x1000, kz=A + 0x2000, phi=A + 0x6000, D=A + 0x8000, out=A + 0x100000)
    p.update(ptrs)
    return lib.fhd_gridding(p["kx"], p["ky"], p["kz"], p["phi"], p["D"], M, nx, ny, nz, p["out"], None)


@pytest.mark.parametrize("kw", [
    dict(nx=6), dict(ny=1), dict(nz=2048), dict(nx=0), dict(M=-1),
    dict(kx=None), dict(D=None), dict(out=None),
    dict(out=A + 0x8000 + 64),                       # image overlaps D
])
def test_gridding_argument_errors(lib, kw):
    assert _grid(lib, **kw) == _lib.FHD_ERR_INVALID_ARGUMENT
    assert lib.fhd_last_error() != b""
