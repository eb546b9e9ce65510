#!/usr/bin/env python3
"""Benchmark: F^H D voxel-sample pairs/s at 128^3 voxels x 262,144 samples on one MI355X.

One step = one pass of the whole hot path (per-sample Mu/record kernel, gather
kernel, reduction of the sample-split rows) over the 128^3 stack-of-spirals
workload, inputs resident in HBM.  Prints one JSON line.  The gather stage (the
dominant kernel) is also timed on its own with HIP events on the stream it is
launched on.

Roofline (the method's work, as the FP32/transcendental roofline counts it):
per voxel-sample pair the pages' kernel computes a phase (1 mul + 2 FMA), its
reduction, a sine and a cosine, and a complex multiply-accumulate (4 FMA): 14
FLOP and 2 transcendentals (PMPP ch. 17, section 17.3: about 13 FP operations
per 2 trig).  `roofline.achieved` is that work over the gather's time against
the MI355X FP32 peak; `roofline.method_roofline` gives the pairs/s roofline
min(R_trans / 2, FP32 peak / 14) with the transcendental rate measured on the
GPU, and the fraction of it reached; `roofline.engine` gives what the timed
kernel itself executes against its own pipe.  The default matrix-core engine
factors the phase over voxel groups on a grid and executes far less than the
per-pair work, so the method fractions exceed 1; the per-pair kernel (one voxel
per lane on the vector ALU) is timed in the same run (`method`).  The CPU
oracle is timed on a bounded voxel sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

METRIC = "FhD voxel·sample pairs/s at 128³×262144 (G/s) + % of FP32/trig roofline"
FP32_PEAK_TFLOPS = 157.3          # MI355X published FP32 peak (vector, and dense matrix)
FP16_PEAK_TFLOPS = 2500.0         # MI355X published dense fp16 matrix peak
HBM_PEAK_GBS = 8000.0             # MI355X published HBM3E bandwidth
# The method's work per voxel-sample pair: phase 5 + reduction 1 + complex
# MAC 8 (Q: real weight, MAC 4), plus two transcendentals; with B data vectors
# sharing one phase, 6 + 8 B per (voxel, sample).
FLOP_PER_PAIR = {"fhd": 14, "q": 10, "forward": 14}
TRANS_PER_PAIR = 2
# Measured on one MI355X by `python bench.py --issue-rates`
# (profiles/issue_rates_gfx950.md): MB-TRANS v_sin_f32 throughput of the whole
# GPU, and MB-PAIR, the pages' per-pair loop body (phase, fract, v_sin, v_cos,
# four-FMA MAC) with no memory traffic at full occupancy: the issue ceiling of
# the per-pair form on this chip (transcendentals share the VALU issue port).
R_TRANS_PER_S = 17.528e12
PAIR_ISSUE_CEILING = 3.307e12
# What the matrix-core kernels execute: the three real multiply-accumulates
# (6 FLOP) per pair of the three-multiplication complex product on the FP32
# matrix pipe; a group phase with its sine and cosine serves 128 voxel columns.
MFMA_FLOP_PER_PAIR = {"gather": 6, "forward": 6}
# Matrix-pipe busy share of the gather from SQ_VALU_MFMA_BUSY_CYCLES (valid for
# the kernel source it was taken on, like TRAFFIC below)
MFMA_BUSY = {
    ("fhd_128cube_262144_spirals", "hw", 128): {
        "source": "fhd_mfma.hip", "kernel_sha256": "beb77294902e5603", "busy": 0.926,
        "profile": "profiles/mfma_gather_128cubed_x_262144_issue_counters.md"},
    ("fhd_128cube_262144_spirals", "accurate", 128): {
        "source": "fhd_mfma.hip", "kernel_sha256": "beb77294902e5603", "busy": 0.854,
        "profile": "profiles/mfma_gather_128cubed_x_262144_issue_counters.md"},
}


def method_roofline(kind: str, B: int) -> dict:
    """Pairs/s roofline of the per-pair method: min(R_trans / n_trans,
    FP32 peak / n_flop) per (voxel, sample), times B vectors."""
    flop_vs = (6 + 8 * B) if kind != "q" else 10   # per (voxel, sample)
    p_trans = R_TRANS_PER_S / TRANS_PER_PAIR
    p_flop = FP32_PEAK_TFLOPS * 1e12 / flop_vs
    return {"p_roof_pairs_per_s": B * min(p_trans, p_flop), "bound": "trans" if p_trans <= p_flop else "fp32",
            "r_trans_per_s": R_TRANS_PER_S, "flop_per_voxel_sample": flop_vs, "trans_per_voxel_sample": TRANS_PER_PAIR}


# HBM bytes of the gather kernel from rocprofv3 FETCH_SIZE / WRITE_SIZE runs,
# scaled by a 1 GiB copy (FETCH_SIZE reads half the bytes, WRITE_SIZE all).
# Valid only for the kernel source (with the headers it includes) they were
# taken on (sha256 prefix) and the
# same launch configuration; otherwise the benchmark reports null.
TRAFFIC = {
    ("fhd_128cube_262144_spirals", "hw", "blocked", "mfma", 128): {
        "source": "fhd_mfma.hip", "kernel_sha256": "beb77294902e5603",
        "fetch_bytes": 2438538.5 * 1024 * 2.0, "write_bytes": 507904.0 * 1024 * 1.0,
        "profile": "profiles/gather_128cubed_x_262144_hbm_counters.md"},
    ("fhd_128cube_262144_spirals", "accurate", "blocked", "mfma", 128): {
        "source": "fhd_mfma.hip", "kernel_sha256": "beb77294902e5603",
        "fetch_bytes": 3529561.1 * 1024 * 2.0, "write_bytes": 2517529.6 * 1024 * 1.0,
        "profile": "profiles/gather_128cubed_x_262144_hbm_counters.md"},
    ("fhd_128cube_262144_spirals/forward", "hw", "blocked", "mfma", 128): {
        "source": "fhd_forward.hip", "kernel_sha256": "4e60ce8e9dcf22de",
        "fetch_bytes": 1057504.1 * 1024 * 2.0, "write_bytes": 2048.0 * 1024 * 1.0,
        "profile": "profiles/forward_gather_128cubed_x_262144_hbm_counters.md"},
    ("fhd_128cube_262144_spirals/forward", "accurate", "blocked", "mfma", 128): {
        "source": "fhd_forward.hip", "kernel_sha256": "4e60ce8e9dcf22de",
        "fetch_bytes": 88648.3 * 1024 * 2.0, "write_bytes": 16384.0 * 1024 * 1.0,
        "profile": "profiles/forward_gather_128cubed_x_262144_hbm_counters.md"},
    ("fhd_128cube_262144_spirals/forward", "hw", "blocked", "mfma16", 128): {
        "source": "fhd_forward_half.hip", "kernel_sha256": "1de86f640c4e14c3",
        "fetch_bytes": 797316.6 * 1024 * 2.0, "write_bytes": 2048.0 * 1024 * 1.0,
        "profile": "profiles/forward_half_gather_128cubed_x_262144_kernel_stats.md"},
    ("fhd_128cube_262144_spirals/forward", "accurate", "blocked", "mfma16", 128): {
        "source": "fhd_forward_half.hip", "kernel_sha256": "1de86f640c4e14c3",
        "fetch_bytes": 797340.6 * 1024 * 2.0, "write_bytes": 2048.0 * 1024 * 1.0,
        "profile": "profiles/forward_half_gather_128cubed_x_262144_kernel_stats.md"},
    ("fhd_128cube_262144_spirals", "hw", "blocked", "valu", 16): {
        "source": "fhd_kernels.hip", "kernel_sha256": "09b302823e68cacf",
        "fetch_bytes": 982777.8 * 1024 * 2.0, "write_bytes": 262148.1 * 1024 * 1.0,
        "profile": "profiles/gather_128cubed_x_262144_hbm_counters.md"},
    ("fhd_128cube_262144_spirals", "accurate", "blocked", "valu", 16): {
        "source": "fhd_kernels.hip", "kernel_sha256": "09b302823e68cacf",
        "fetch_bytes": 1047734.7 * 1024 * 2.0, "write_bytes": 262147.2 * 1024 * 1.0,
        "profile": "profiles/gather_128cubed_x_262144_hbm_counters.md"},
    ("fhd_128cube_262144_spirals", "hw", "blocked", "mfma16", 128): {
        "source": "fhd_half.hip", "kernel_sha256": "8d3129522d42899d",
        "fetch_bytes": 2318758.5 * 1024 * 2.0, "write_bytes": 262148.0 * 1024 * 1.0,
        "profile": "profiles/half_gather_128cubed_x_262144_kernel_stats.md"},
    # the whole gridding reconstruction (sort, deposit + x transform, y and z passes)
    ("fhd_128cube_262144_spirals/gridding", "-", "-", "-", 0): {
        "source": ["fhd_grid.hip", "fhd_lines.hip"], "kernel_sha256": "da0ebbbcb4b5f75b",
        "fetch_bytes": 25875.8 * 1024 * 2.0, "write_bytes": 59449.8 * 1024 * 1.0,
        "profile": "profiles/gridding_128cubed_x_262144_kernel_stats.md"},
    ("fhd_512cube_262144_spirals/gridding", "-", "-", "-", 0): {
        "source": ["fhd_grid.hip", "fhd_lines.hip"], "kernel_sha256": "da0ebbbcb4b5f75b",
        "fetch_bytes": 1380804.8 * 1024 * 2.0, "write_bytes": 3156022.2 * 1024 * 1.0,
        "profile": "profiles/gridding_128cubed_x_262144_kernel_stats.md"},
    # the normal operator's five kernels, per application (128^3, lambda = 0)
    ("fhd_128cube_262144_spirals/cg", "hw", "blocked", "mfma", 64): {
        "source": ["fhd_cg.hip", "fhd_lines.hip"], "kernel_sha256": "aade9157aa9416cf",
        "fetch_bytes": 147709.3 * 1024 * 2.0, "write_bytes": 213007.2 * 1024 * 1.0,
        "profile": "profiles/cg_normal_operator_128cubed_kernel_stats.md"},
    ("fhd_512cube_262144_spirals/cg", "hw", "blocked", "mfma", 64): {
        "source": ["fhd_cg.hip", "fhd_lines.hip"], "kernel_sha256": "aade9157aa9416cf",
        "fetch_bytes": 9437532.7 * 1024 * 2.0, "write_bytes": 13639403.9 * 1024 * 1.0,
        "profile": "profiles/scale_512cubed_summary.md"},
}
WORKLOADS = {
    "fhd_128cube_262144_spirals": "FhD 128^3 voxels x 262,144 stack-of-spirals samples (64 kz planes x 4096-point spirals), complex N(0,1) phi and D",
    "fhd_64cube_65536_radial": "FhD 64^3 voxels x 65,536 radial samples",
    "fhd_128cube_262144_spirals_jittered": "FhD at 2,097,152 off-grid points (128^3 centres displaced by up to a "
                                           "quarter voxel per axis) x the 262,144 stack-of-spirals samples",
    "fhd_512cube_262144_spirals": "FhD 512^3 voxels x 262,144 stack-of-spirals samples (64 kz planes x 4096-point spirals), complex N(0,1) phi and D",
    "q_128cube_halfstep_1048576_uniform": "Q on 128^3 voxels (step 0.5) x 1,048,576 uniform samples",
    "fhd16_96cube_500001_radial": "FhD x16 vectors, 96^3 voxels x 500,001 radial samples",
    "fhd_32cube_2048_uniform": "FhD 32^3 voxels x 2048 uniform samples",
}


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--config", default="fhd_128cube_262144_spirals", choices=sorted(WORKLOADS))
    ap.add_argument("--trig", default="hw", choices=["accurate", "hw"])
    ap.add_argument("--sum", default="blocked", choices=["blocked", "kahan", "plain"])
    ap.add_argument("--engine", default="auto", choices=["auto", "valu", "mfma", "mfma16"])
    ap.add_argument("--half-steps", type=int, default=5,
                    help="steps of the opt-in half-split engine (engine=mfma16) timed beside the matrix-core "
                         "engine's (0: skip)")
    ap.add_argument("--op", default="fhd", choices=["fhd", "forward", "cg", "gridding"],
                    help="fhd: F^H D (or Q for a Q workload); forward: F rho of a seeded image "
                         "on the same trajectory and voxels; cg: conjugate-gradient reconstruction "
                         "(Toeplitz F^H F through Q) on the workload's voxel grid; gridding: the "
                         "trilinear gridding + inverse FFT baseline image on that grid")
    ap.add_argument("--cg-iters", type=int, default=10, help="CG iterations per step (--op cg)")
    ap.add_argument("--cg-lambda", type=float, default=0.0,
                    help="regulariser weight relative to sum |phi|^2 / 6 (--op cg)")
    ap.add_argument("--no-mirror-pairs", action="store_true",
                    help="sum every voxel group alone (FHD_FLAG_NO_MIRROR_PAIRS) on the four-sample HW path")
    ap.add_argument("--voxels-per-lane", type=int, default=0)
    ap.add_argument("--tile", type=int, default=0)
    ap.add_argument("--method-steps", type=int, default=3,
                    help="gather launches of the per-pair kernel timed beside the benchmark (0 skips it)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="target wall time of the CPU-oracle baseline (0 disables it)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of the benchmark, run a plain device-to-device copy of this many MiB "
                         "five times (reference reading for the HBM byte counters) and exit")
    ap.add_argument("--tune", action="store_true",
                    help="instead of the benchmark, sweep group size x sample rows x tile for --config, "
                         "time the Pareto front of the static model and print one JSON line")
    ap.add_argument("--exhaustive", action="store_true", help="with --tune: time every candidate")
    ap.add_argument("--tune-engines", default="mfma", help="with --tune: comma-separated engines (mfma,valu)")
    ap.add_argument("--issue-rates", action="store_true",
                    help="run the gfx950 issue-rate microbenchmark (FMA, v_sin, mixed issue, trig error) and exit")
    return ap.parse_args()


def copy_calibration(mib: int) -> None:
    """A plain copy kernel of known size, for scaling FETCH_SIZE / WRITE_SIZE readings."""
    import torch
    n = mib * (1 << 20) // 4
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration": {"bytes_read": n * 4, "bytes_written": n * 4, "launches": 5}}))


def cpu_baseline(p, target_s: float, rho=None) -> dict:
    """Time the oracle as it stands on a seeded voxel (or, for the forward
    operator, sample) subset of the same workload."""
    import oracle
    from non_cartesian_mri_amd import inputs
    oracle.build(force=False)
    total = p.M if rho is not None else p.N

    def run(count):
        idx = inputs.subset_indices(total, count, p.seed)
        if rho is not None:
            oracle.forward(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, rho, idx=idx)
        elif p.kind == "q":
            oracle.q(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, idx=idx)
        else:
            oracle.fhd(p.kx, p.ky, p.kz, p.x, p.y, p.z, p.phi, p.D, idx=idx)
        return oracle.last.seconds, oracle.last.threads

    probe = 64 * max(1, oracle_threads_hint())
    t, _ = run(probe)
    count = int(min(total, max(probe, probe * target_s / max(t, 1e-6))))
    t, threads = run(count)
    pairs = count * (p.N if rho is not None else p.M) * p.B
    what = (f"{count} seeded samples x all {p.N} voxels" if rho is not None
            else f"{count} seeded voxels x all {p.M} samples")
    return {"value": pairs / t / 1e9, "unit": "Gpair/s", "cores": threads, "kind": "oracle",
            "sample": f"{what} x {p.B} vector(s) of the same workload ({pairs:.3e} pairs, {t:.1f} s wall)"}


def cpu_baseline_cg(p, target_s: float, lam: float) -> dict:
    """Time the oracle's CG iteration (Toeplitz product by the plain double sum
    over voxel pairs) on a small cubic grid with the same trajectory, grown
    until one iteration takes about target_s / 3."""
    import oracle
    from oracle import recon
    oracle.build(force=False)
    rng = np.random.Generator(np.random.PCG64(p.seed + 3000))
    best = None
    for L in (4, 6, 8, 10, 12, 14, 16):
        t0 = time.perf_counter()
        qd = recon.q_differences(p.kx, p.ky, p.kz, p.phi, L, L, L)
        tq = time.perf_counter() - t0
        b = rng.standard_normal(L ** 3) + 1j * rng.standard_normal(L ** 3)
        t0 = time.perf_counter()
        recon.cg(lambda v: recon.toeplitz_apply(qd, v, L, L, L) + lam * recon.laplacian(v, L, L, L),
                 b, np.zeros(L ** 3), 2)
        ti = (time.perf_counter() - t0) / 3.0        # initial residual + 2 iterations: 3 operator calls
        best = (L, ti, tq)
        if tq + 3 * ti > target_s / 3:
            break
    L, ti, tq = best
    return {"value": 1.0 / ti, "unit": "iter/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle CG iterations on a {L}^3 grid with all {p.M} samples of the same trajectory "
                      f"(Q at the {(2 * L - 1) ** 3} coordinate differences in {tq:.1f} s with "
                      f"{oracle.last.threads} threads, then {ti * 1e3:.1f} ms per iteration, single thread); "
                      f"the GPU figure is at the full grid"}


def normal_operator_bytes(nx: int, ny: int, nz: int) -> int:
    """HBM bytes of one application of the Toeplitz normal operator when each
    transform pass reads its input and writes its output once: x pass (p in,
    nz ny rows of px out), y pass (to nz py px), z pass with the real spectrum
    (px py pz floats), inverse y pass, inverse x pass (plus p once more for the
    regulariser and the dot product, Ap out)."""
    from non_cartesian_mri_amd.fhd import toeplitz_lengths
    pz, py, px = toeplitz_lengths((nz, ny, nx))
    n, rows, grid = nx * ny * nz, nz * ny * px, nz * py * px
    c = 8
    return (c * n + c * rows) + (c * rows + c * grid) + (2 * c * grid + 4 * px * py * pz) \
        + (c * grid + c * rows) + (c * rows + 2 * c * n)


def bench_cg(args, p, t, D, dev) -> dict:
    """One step = --cg-iters CG iterations from a zero image on b = F^H D, with Qhat
    computed once per trajectory beforehand (timed separately)."""
    import torch
    from non_cartesian_mri_amd import (fhd_cg_solve, fhd_cg_workspace_bytes, fhd_compute,
                                       fhd_normal_apply, fhd_toeplitz_kernel)
    L = p.L
    if p.N != L ** 3 or p.extra.get("step", 1.0) != 1.0 or p.B != 1:
        print("--op cg needs a single-vector workload on a unit-step cubic grid", file=sys.stderr)
        sys.exit(2)
    stream = torch.cuda.current_stream()
    opts = dict(trig=args.trig, sum=args.sum, voxels_per_lane=args.voxels_per_lane, tile=args.tile,
                engine=args.engine)
    lam = args.cg_lambda * float(np.sum(np.abs(p.phi.astype(np.complex128)) ** 2)) / 6.0
    e = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    e[0].record(stream)
    b = fhd_compute(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], D[0], **opts).reshape(L, L, L)
    e[1].record(stream)
    Qhat = fhd_toeplitz_kernel(t["kx"], t["ky"], t["kz"], t["phi"], (L, L, L), **opts)
    e[2].record(stream)
    torch.cuda.synchronize()
    fhd_ms, toe_ms = e[0].elapsed_time(e[1]), e[1].elapsed_time(e[2])
    ws = torch.empty(fhd_cg_workspace_bytes(L, L, L), dtype=torch.uint8, device=dev)
    x = torch.zeros_like(b)
    r = torch.empty(args.cg_iters + 1, dtype=torch.float64, device=dev)

    def step():
        x.zero_()
        fhd_cg_solve(Qhat, b, args.cg_iters, lam, out=x, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, c in ev:
        a.record(stream)
        step()
        c.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(c) for a, c in ev])
    # the normal operator alone (pad, FFT, spectral product, inverse FFT, crop + regulariser)
    Ap = torch.empty_like(b)
    nev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(20)]
    for a, c in nev:
        a.record(stream)
        fhd_normal_apply(Qhat, x, lam, out=Ap, workspace=ws)
        c.record(stream)
    torch.cuda.synchronize()
    op_ms = float(np.mean([a.elapsed_time(c) for a, c in nev]))
    _, rr = fhd_cg_solve(Qhat, b, args.cg_iters, lam, workspace=ws, resid=True)
    rr = rr.cpu().numpy()
    n = L ** 3
    op_bytes = normal_operator_bytes(L, L, L)
    ms_per_step = wall * 1e3 / args.steps
    achieved = op_bytes / (op_ms * 1e-3) / 1e9
    res = {
        "metric": f"CG iterations/s, (F^H F + lambda W^H W) x = F^H D with Toeplitz F^H F through Q, {L}^3 grid",
        "value": round(args.cg_iters / (ms_per_step * 1e-3), 3),
        "unit": "iter/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config] + f"; CG on the {L}^3 grid, {args.cg_iters} "
                               f"iterations per step from a zero image",
                   "op": "cg", "name": args.config, "grid": [L, L, L], "samples": p.M,
                   "iterations_per_step": args.cg_iters, "lambda_rel": args.cg_lambda, "trig": args.trig,
                   "parallelism": "single GPU"},
        "timing_ms": {"step_event_median": round(float(np.median(step_ms)), 4),
                      "normal_operator_event_mean": round(op_ms, 4),
                      "fhd_setup": round(fhd_ms, 3), "toeplitz_setup": round(toe_ms, 3)},
        "residual": {"first": float(rr[0]), "last": float(rr[-1])},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None,
                     "traffic_unit": "GB/s (HBM bytes per application from FETCH_SIZE/WRITE_SIZE / time)",
                     "traffic_detail": None,
                     "kernel": "the normal operator timed as one unit: x, y transforms, z transform with the "
                               "spectral product, inverse y, inverse x with the regulariser and <p, Ap>",
                     "algorithmic_bytes": op_bytes},
    }
    if args.cg_lambda == 0.0:
        # the operator does not depend on the trig path (it only reads Qhat)
        traffic, detail = traffic_for(args.config + "/cg", "hw", "blocked", "mfma", 64, op_ms)
        if traffic is not None:
            res["roofline"]["traffic"] = round(traffic, 3)
            res["roofline"]["traffic_unit"] = "GB/s (HBM bytes per application from FETCH_SIZE/WRITE_SIZE / time)"
            res["roofline"]["traffic_detail"] = detail
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_cg(p, args.cpu_seconds, lam)
    return res


def cpu_baseline_gridding(p, target_s: float) -> dict:
    """Time the gridding oracle as it stands (all samples gridded, the image at
    a seeded voxel sample), grown until it takes about target_s."""
    from oracle import gridding as G_
    from non_cartesian_mri_amd import inputs
    L = p.L
    t0 = time.perf_counter()
    G = G_.grid_samples(p.kx, p.ky, p.kz, p.phi, p.D[0], L, L, L)
    tg = time.perf_counter() - t0
    count = 8
    while True:
        idx = inputs.subset_indices(L ** 3, count, p.seed)
        t0 = time.perf_counter()
        G_.lattice_image_at(G, idx)
        ti = time.perf_counter() - t0
        if ti > target_s / 4 or count >= L ** 3:
            break
        count *= 4
    per_image = tg + ti * (L ** 3 / count)
    return {"value": 1.0 / per_image, "unit": "images/s", "cores": 1, "kind": "oracle",
            "sample": f"oracle gridding of all {p.M} samples ({tg:.2f} s) and the lattice sum at {count} seeded "
                      f"voxels of {L ** 3} ({ti:.2f} s), scaled to the whole image; single thread"}


def bench_gridding(args, p, t, D, dev) -> dict:
    """One step = one gridding reconstruction (plane sort, tile deposit + x transform, y and z passes)."""
    import torch
    from non_cartesian_mri_amd import fhd_gridding
    L = p.L
    if p.N != L ** 3 or p.extra.get("step", 1.0) != 1.0 or p.B != 1 or (L & (L - 1)) != 0:
        print("--op gridding needs a single-vector workload on a unit-step cubic power-of-two grid", file=sys.stderr)
        sys.exit(2)
    stream = torch.cuda.current_stream()
    out = torch.empty((L, L, L), dtype=torch.complex64, device=dev)

    def step():
        fhd_gridding(t["kx"], t["ky"], t["kz"], t["phi"], D[0], (L, L, L), out=out)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a, c in ev:
        a.record(stream)
        step()
        c.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = float(np.median([a.elapsed_time(c) for a, c in ev]))
    ms_per_step = wall * 1e3 / args.steps
    n = L ** 3
    # bytes one reconstruction must move: the samples (k 12 B, phi 8 B, D 8 B)
    # once, the lattice leaving the chip once with its x rows already
    # transformed (a tile holds whole rows), then read and written by the y and
    # z passes (the sort's entries are the implementation's, not counted)
    alg = p.M * 28 + 8 * n + 2 * 16 * n
    achieved = alg / (step_ms * 1e-3) / 1e9
    traffic, traffic_detail = traffic_for(args.config + "/gridding", "-", "-", "-", 0, step_ms)
    res = {
        "metric": f"gridding/iFFT reconstructions/s, {L}^3 grid",
        "value": round(1e3 / ms_per_step, 3), "unit": "images/s",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "f32", "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config] + f"; trilinear gridding onto the {L}^3 k-lattice, "
                               "inverse FFT", "op": "gridding", "name": args.config, "grid": [L, L, L],
                   "samples": p.M, "parallelism": "single GPU"},
        "timing_ms": {"step_event_median": round(step_ms, 4)},
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": None if traffic is None else round(traffic, 3),
                     "traffic_unit": "GB/s (HBM bytes per reconstruction from FETCH_SIZE/WRITE_SIZE / its time)",
                     "traffic_detail": traffic_detail,
                     "kernel": "the whole reconstruction timed as one unit (plane sort of the deposits, LDS tile "
                               "deposit fused with the x transform, y and z FFT passes)",
                     "algorithmic_bytes": alg},
    }
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline_gridding(p, args.cpu_seconds)
    return res


def kernel_source_sha(name) -> str:
    """sha256 prefix of a kernel source (or a list of them, in order) together
    with every library header it includes, directly or through other headers
    (each once, depth first in sorted order)."""
    import hashlib
    import re
    csrc = os.path.join(os.path.dirname(os.path.abspath(__file__)), "non_cartesian_mri_amd", "csrc")
    h = hashlib.sha256()
    seen = set()

    def add(fname):
        path = os.path.join(csrc, fname)
        if fname in seen or not os.path.exists(path):
            return
        seen.add(fname)
        with open(path, "rb") as f:
            text = f.read()
        h.update(text)
        for inc in sorted(set(re.findall(rb'#include "([^"]+)"', text))):
            add(inc.decode())

    for one in ([name] if isinstance(name, str) else name):
        add(one)
    return h.hexdigest()[:16]


def traffic_for(config: str, trig: str, summ: str, engine: str, group: int, gather_ms: float):
    """Counter-derived HBM traffic (GB/s over the launch) or None if not measured for this kernel."""
    t = TRAFFIC.get((config, trig, summ, engine, group))
    if t is None or t["kernel_sha256"] != kernel_source_sha(t["source"]):
        return None, None
    total = t["fetch_bytes"] + t["write_bytes"]
    return total / (gather_ms * 1e-3) / 1e9, {"bytes_per_launch": total, "fetch_bytes": t["fetch_bytes"],
                                               "write_bytes": t["write_bytes"], "profile": t["profile"]}


def mirror_pair_work(ws, ws_bytes: int, p, plan: dict) -> dict:
    """The pair plan the device wrote for the last gather pass (at the end of
    the workspace: 16 int32 of header, one int2 per voxel group, then each
    group's reference voxel as a float4), and the
    matrix work it implies: per block of four samples every wave of 16 list
    entries (a group with its partner, or a group alone) issues 4 MFMAs per
    tile of 16 columns (8 tiles); the unpaired kernel's waves of 16 groups
    issue 3.  Each v_mfma_f32_16x16x4_f32 is 16 x 16 x 4 multiply-adds."""
    V = plan["voxels_per_lane"]
    G = -(-p.N // V)
    pair_bytes = ((64 + 8 * G + 15) // 16 * 16 + 16 * G + 255) // 256 * 256
    head = ws[ws_bytes - pair_bytes:ws_bytes - pair_bytes + 64].view(torch_int32()).cpu().numpy()
    E, Cp, R, U = int(head[0]), int(head[1]), int(head[2]), int(head[4])
    mpad = plan["padded_samples"]
    mfmas = U * 32 * (mpad // 4) * plan["passes"]
    flop = mfmas * 16 * 16 * 4 * 2
    alone_mfmas = -(-G // 16) * 24 * (mpad // 4) * plan["passes"]
    return {"paired_groups": Cp, "groups_alone": E - Cp, "groups": G, "launch_rows": R,
            "wave_slots": U, "executed_flop_per_pair": flop / (p.N * p.M * p.B),
            "mfma_ratio_to_unpaired": round(mfmas / alone_mfmas, 4)}


def forward_pair_work(ws, p, plan: dict) -> dict:
    """The forward operator's pair plan (first pass; one pass for every
    workload here) and its matrix work: per wave of 16 samples and block of
    four list entries, 4 MFMAs per tile of 16 columns (8 tiles), over the
    entries padded to 32.  Pass layout: entry headers, entries (64 T floats
    each), the list of groups of irregular waves, the wave flags, the plan."""
    a256 = lambda b: (b + 255) // 256 * 256
    V = plan["voxels_per_lane"]
    G = -(-p.N // V)
    gpad = -(-G // 32) * 32
    off = a256(gpad * 16) + a256(gpad * 64 * 8 * 4) + a256(4 * (gpad + 1)) + a256(4 * -(-G // 16))
    head = ws[off:off + 64].view(torch_int32()).cpu().numpy()
    E, Cp = int(head[0]), int(head[1])
    epad = -(-E // 32) * 32
    mfmas = -(-p.M // 16) * (epad // 4) * 32 * plan["passes"]
    alone = -(-p.M // 16) * (gpad // 4) * 24 * plan["passes"]
    return {"paired_groups": Cp, "groups_alone": E - Cp, "groups": G, "launch_rows": plan["sample_splits"],
            "executed_flop_per_pair": mfmas * 16 * 16 * 4 * 2 / (p.N * p.M * p.B),
            "mfma_ratio_to_unpaired": round(mfmas / alone, 4)}


def torch_int32():
    import torch
    return torch.int32


def oracle_threads_hint() -> int:
    try:
        return int(os.environ.get("OMP_NUM_THREADS", "")) or os.cpu_count() or 1
    except ValueError:
        return os.cpu_count() or 1


def time_per_pair_kernel(p, t, D, args, stream, mr) -> dict:
    """The pages' per-pair gather (VALU engine, one voxel per lane) on the same
    workload and trig path: its gather stage timed alone with HIP events on the
    stream it runs on (records built once beforehand)."""
    import torch
    from non_cartesian_mri_amd import fhd_compute, fhd_workspace_bytes, q_compute
    is_q = p.kind == "q"
    opts = dict(trig=args.trig, sum="blocked", engine="valu", voxels_per_lane=1)
    ws = torch.empty(max(1, fhd_workspace_bytes(p.M, p.N, p.B, is_q=is_q, **opts)), dtype=torch.uint8,
                     device=t["kx"].device)
    out = torch.empty((p.B, p.N), dtype=torch.complex64, device=t["kx"].device)

    def stage(which):
        if is_q:
            q_compute(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], stages=which, workspace=ws,
                      out=out.view(-1), **opts)
        else:
            fhd_compute(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], D, stages=which,
                        workspace=ws, out=out, **opts)

    stage("mu")
    stage("gather")
    torch.cuda.synchronize()
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.method_steps)]
    for a, b in ev:
        a.record(stream)
        stage("gather")
        b.record(stream)
    torch.cuda.synchronize()
    ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    pairs = p.N * p.M * p.B
    rate = pairs / (ms * 1e-3)
    tflops = mr["flop_per_voxel_sample"] * p.N * p.M / (ms * 1e-3) / 1e12
    return {"kernel": "gather_kernel with one voxel per lane (VALU engine, voxels_per_lane=1): the pages' "
                      "per-pair form, one phase, fract, sin, cos and complex MAC per voxel-sample pair",
            "gather_event_mean_ms": round(ms, 3), "launches_timed": args.method_steps,
            "value": round(rate / 1e9, 3), "unit": "Gpair/s",
            "achieved": round(tflops, 3), "peak": FP32_PEAK_TFLOPS, "achieved_unit": "TFLOP/s",
            "frac": round(tflops / FP32_PEAK_TFLOPS, 4),
            "frac_method": round(rate / mr["p_roof_pairs_per_s"], 4),
            "issue_ceiling_pairs_per_s": PAIR_ISSUE_CEILING,
            "frac_issue": None if not PAIR_ISSUE_CEILING else round(rate / PAIR_ISSUE_CEILING, 4)}


def time_half_engine(p, t, D, args, stream) -> dict:
    """The opt-in half-split engine (engine="mfma16") on the same workload and
    trig path: whole steps (scale + records, gather, row reduction) and the
    gather alone, timed with HIP events on its stream."""
    import torch
    from non_cartesian_mri_amd import fhd_compute, fhd_workspace_bytes, q_compute
    from non_cartesian_mri_amd.fhd import fhd_describe_plan
    is_q = p.kind == "q"
    opts = dict(trig=args.trig, sum=args.sum, engine="mfma16")
    ws = torch.empty(max(1, fhd_workspace_bytes(p.M, p.N, p.B, is_q=is_q, **opts)), dtype=torch.uint8,
                     device=t["kx"].device)
    out = torch.empty((p.B, p.N), dtype=torch.complex64, device=t["kx"].device)

    def stage(which):
        if is_q:
            q_compute(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], stages=which, workspace=ws,
                      out=out.view(-1), **opts)
        else:
            fhd_compute(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], D, stages=which,
                        workspace=ws, out=out, **opts)

    for _ in range(2):
        for w in ("mu", "gather", "reduce"):
            stage(w)
    torch.cuda.synchronize()
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(args.half_steps)]
    for e0, e1, e2, e3 in ev:
        e0.record(stream)
        stage("mu")
        e1.record(stream)
        stage("gather")
        e2.record(stream)
        stage("reduce")
        e3.record(stream)
    torch.cuda.synchronize()
    step = float(np.median([a.elapsed_time(d) for a, b, c, d in ev]))
    gather = float(np.mean([b.elapsed_time(c) for a, b, c, d in ev]))
    pairs = p.N * p.M * p.B
    ex = 18 * pairs / (gather * 1e-3) / 1e12
    plan = fhd_describe_plan(p.M, p.N, p.B, op="q" if is_q else "fhd", **opts)
    traffic, traffic_detail = traffic_for(args.config, args.trig, args.sum, "mfma16", plan["voxels_per_lane"], gather)
    return {"engine": "mfma16", "steps": args.half_steps,
            "value": round(pairs / (step * 1e-3) / 1e9, 3), "unit": "Gpair/s", "step_event_median_ms": round(step, 4),
            "gather_event_mean_ms": round(gather, 4),
            "gather_pairs_per_s": round(pairs / (gather * 1e-3), 1),
            "achieved": round(ex, 3), "peak": FP16_PEAK_TFLOPS, "unit_engine": "TFLOP/s",
            "frac": round(ex / FP16_PEAK_TFLOPS, 4), "executed_flop_per_pair": 18,
            "traffic": None if traffic is None else round(traffic, 3), "traffic_detail": traffic_detail,
            "note": "opt-in engine (not the default that value reports): the same factored sum with every fp32 "
                    "product formed from fp16 parts (hi hi + hi lo + lo hi) on v_mfma_f32_16x16x32_f16 with fp32 "
                    "accumulation; parity against the oracle at the fp32 bars in tests/test_gpu_half.py and "
                    "tests/test_gpu_configs.py"}


def main():
    args = parse()
    if args.issue_rates:
        import subprocess
        from non_cartesian_mri_amd.build import ISSUE_RATES
        if not os.path.exists(ISSUE_RATES):
            print(f"{ISSUE_RATES} is not built (python -m non_cartesian_mri_amd.build)", file=sys.stderr)
            sys.exit(1)
        sys.exit(subprocess.run([ISSUE_RATES]).returncode)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py runs on exactly one GPU: the F^H D path here is a single-GPU build "
              "(voxel sharding across GPUs is a design note only); use --gpus 1", file=sys.stderr)
        sys.exit(2)
    import torch
    from non_cartesian_mri_amd import fhd_compute, fhd_forward, fhd_workspace_bytes, inputs, q_compute
    if not torch.cuda.is_available():
        print("no GPU visible", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(args.copy_calibration)
        return
    dev = torch.device("cuda:0")
    p = inputs.make_config(args.config)
    t = {k: torch.from_numpy(np.ascontiguousarray(getattr(p, k))).to(dev)
         for k in ("kx", "ky", "kz", "x", "y", "z", "phi")}
    D = None if p.D is None else torch.from_numpy(np.ascontiguousarray(p.D)).to(dev)
    is_q = p.kind == "q"
    if args.tune:
        from non_cartesian_mri_amd import tune
        t0 = time.perf_counter()
        res = tune.sweep(t, D, trig=args.trig, sum=args.sum, engines=tuple(args.tune_engines.split(",")),
                         exhaustive=args.exhaustive, grid_edge=p.L if p.N == p.L ** 3 else None)
        res.update(config=args.config, trig=args.trig, engines=args.tune_engines, seconds=time.perf_counter() - t0)
        print(json.dumps(res), flush=True)
        return
    if args.op == "cg":
        print(json.dumps(bench_cg(args, p, t, D, dev)), flush=True)
        return
    if args.op == "gridding":
        print(json.dumps(bench_gridding(args, p, t, D, dev)), flush=True)
        return
    forward = args.op == "forward"
    if forward and is_q:
        print("--op forward needs an F^H D workload (the image replaces the data vectors)", file=sys.stderr)
        sys.exit(2)
    opts = dict(trig=args.trig, sum=args.sum, voxels_per_lane=args.voxels_per_lane, tile=args.tile,
                engine=args.engine)
    if args.no_mirror_pairs:
        opts["mirror_pairs"] = False
    op = "forward" if forward else ("q" if is_q else "fhd")
    ws_bytes = max(1, fhd_workspace_bytes(p.M, p.N, p.B, op=op, **opts))
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    if forward:
        rng = np.random.Generator(np.random.PCG64(p.seed + 2000))
        rho = torch.from_numpy(np.stack([inputs.complex_normal(rng, p.N) for _ in range(p.B)])).to(dev)
        out = torch.empty((p.B, p.M), dtype=torch.complex64, device=dev)
    else:
        out = torch.empty((p.B, p.N), dtype=torch.complex64, device=dev)

    def stage(which):
        if forward:
            fhd_forward(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], rho,
                        stages=which, workspace=ws, out=out, **opts)
        elif is_q:
            q_compute(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], stages=which,
                      workspace=ws, out=out.view(-1), **opts)
        else:
            fhd_compute(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], D,
                        stages=which, workspace=ws, out=out, **opts)

    stream = torch.cuda.current_stream()
    for _ in range(args.warmup):
        stage("all")
    torch.cuda.synchronize()
    # the timed steps: one whole call per step (records, gather, row reduction)
    sev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e3 in sev:
        e0.record(stream)
        stage("all")
        e3.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = np.array([a.elapsed_time(d) for a, d in sev])
    # the same steps again, one call per stage, to time the gather alone
    ev = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(4)) for _ in range(args.steps)]
    for e0, e1, e2, e3 in ev:
        e0.record(stream)
        stage("mu")
        e1.record(stream)
        stage("gather")
        e2.record(stream)
        stage("reduce")
        e3.record(stream)
    torch.cuda.synchronize()
    gather_ms = np.array([b.elapsed_time(c) for a, b, c, d in ev])
    mu_ms = np.array([a.elapsed_time(b) for a, b, c, d in ev])
    reduce_ms = np.array([c.elapsed_time(d) for a, b, c, d in ev])
    ms_per_step = wall * 1e3 / args.steps
    pairs = p.N * p.M * p.B
    value = pairs / (ms_per_step * 1e-3) / 1e9
    g_avg = float(gather_ms.mean())
    from non_cartesian_mri_amd.fhd import fhd_describe_plan
    plan = fhd_describe_plan(p.M, p.N, p.B, op=op, **opts)
    engine = {1: "valu", 2: "mfma", 3: "mfma16"}[plan["engine"]]
    kind = "forward" if forward else p.kind
    # the method's work: per (voxel, sample) one phase, reduction and sin/cos,
    # and per vector a complex MAC (14 FLOP + 2 transcendentals for one vector,
    # PMPP ch. 17 section 17.3's count of ~13 FP operations per 2 trig)
    mr = method_roofline(kind, p.B)
    method_flop = mr["flop_per_voxel_sample"] * p.N * p.M
    achieved = method_flop / (g_avg * 1e-3) / 1e12
    gather_rate = pairs / (g_avg * 1e-3)
    mr["frac"] = round(gather_rate / mr["p_roof_pairs_per_s"], 4)
    mr["per_pair_issue_ceiling_pairs_per_s"] = PAIR_ISSUE_CEILING
    if engine == "mfma16":
        # three real products per complex pair, each as three fp16 products
        ex = 18 * pairs / (g_avg * 1e-3) / 1e12
        bound = "mfma"
        eng = {"engine": "mfma16", "bound": "mfma", "executed_flop_per_pair": 18, "achieved": round(ex, 3),
               "peak": FP16_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ex / FP16_PEAK_TFLOPS, 4),
               "note": "half-split factorisation: the grid-factored sum of the MFMA engine with every fp32 "
                       "product formed from fp16 parts (hi hi + hi lo + lo hi, fp32 accumulation) on "
                       "v_mfma_f32_16x16x32_f16; the factors are scaled by a power of two into fp16 range"}
        kernel = ("half_gather_kernel: its launch rows in one step, timed alone with the (empty on a grid) "
                  "half_direct_kernel; the scale, records and reduction kernels are outside the interval")
        if forward:
            kernel = ("fwd_half_gather_kernel: its launch rows in one step, timed alone; the image packing, "
                      "scale and fp16 parts, row reduction and (on a grid, empty) direct kernels are outside "
                      "the interval")
    elif forward or engine == "mfma":
        flop_per_pair = MFMA_FLOP_PER_PAIR["forward" if forward else "gather"]
        pairing = None
        if plan.get("mirror_pairs"):
            pairing = forward_pair_work(ws, p, plan) if forward else mirror_pair_work(ws, ws_bytes, p, plan)
            flop_per_pair = pairing["executed_flop_per_pair"]
        ex = flop_per_pair * pairs / (g_avg * 1e-3) / 1e12
        busy = MFMA_BUSY.get((args.config, args.trig, plan["voxels_per_lane"])) if not forward else None
        if busy is not None and busy["kernel_sha256"] != kernel_source_sha(busy["source"]):
            busy = None
        bound = "mfma"
        eng = {"engine": "mfma", "bound": "mfma", "executed_flop_per_pair": round(flop_per_pair, 4),
               "achieved": round(ex, 3),
               "peak": FP32_PEAK_TFLOPS, "unit": "TFLOP/s", "frac": round(ex / FP32_PEAK_TFLOPS, 4),
               "matrix_busy_counter": None if busy is None else busy["busy"],
               "matrix_busy_profile": None if busy is None else busy["profile"],
               "note": "grid-separable factorisation: voxels in groups of %d on a common grid share one phase, "
                       "sine and cosine per sample; the rest is an FP32 matrix product of the group phases with "
                       "per-sample factor columns (3 real MACs per pair), so the kernel executes %.3g of the "
                       "method's transcendentals and the method fractions exceed 1"
                       % (plan["voxels_per_lane"], 1.0 / max(plan["voxels_per_lane"], 1))}
        if pairing is not None:
            eng["mirror_pairs"] = pairing
            eng["note"] += ("; mirror pairs: a group and the group at the negated reference share the phase "
                            "(conjugate), so two groups take one phase and 4 real MACs per pair of columns "
                            "where alone they take two phases and 6")
        if forward:
            kernel = ("fwd_gather_kernel: its launch rows in one step, timed alone; the image packing, "
                      "row reduction and (on a grid, empty) direct kernels are outside the interval")
        else:
            kernel = ("mfma_gather_kernel: its launch rows in one step, timed alone with the (empty on a "
                      "grid) mfma_direct_kernel; records and reduction kernels are outside the interval")
    else:
        bound = "alu"
        V = plan["voxels_per_lane"]
        eng = {"engine": "valu", "bound": "alu", "voxels_per_lane": V,
               "note": "one voxel per lane: the per-pair form (phase, fract, sin, cos, MAC per pair)" if V == 1 else
                       "%d voxels per lane share one phase, sine and cosine per sample (their offsets are folded "
                       "into per-sample factors); 3 FMAs per pair plus the shared work / %d" % (V, V)}
        kernel = ("gather_kernel: its launches in one step, timed alone; the per-sample and reduce "
                  "kernels are outside this interval")
    traffic, traffic_detail = traffic_for(args.config + ("/forward" if forward else ""), args.trig,
                                          args.sum, engine, plan["voxels_per_lane"], g_avg)
    summ = args.sum
    if engine in ("mfma", "mfma16") and plan["tile"] >= (plan["padded_samples"] + plan["sample_splits"] - 1) // plan["sample_splits"] \
            and args.sum == "blocked" and not forward:
        summ = "row-block"   # each launch row summed as one block, rows added in a fixed order
    res = {
        "metric": METRIC if not forward else METRIC.replace("FhD", "Forward-operator F rho"),
        "value": round(value, 3),
        "unit": "Gpair/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": WORKLOADS[args.config] + ("; forward operator F rho of a seeded "
                                                          "complex N(0,1) image" if forward else ""),
                   "op": op, "name": args.config, "voxels": p.N,
                   "samples": p.M, "vectors": p.B, "trig": args.trig, "sum": summ,
                   "engine": engine, "group_voxels": plan["voxels_per_lane"], "tile": plan["tile"],
                   "sample_splits": plan["sample_splits"], "gather_launches": plan["passes"],
                   "mirror_pairs": bool(plan.get("mirror_pairs")),
                   "parallelism": "single GPU, data-parallel over voxels"},
        "timing_ms": {"step_event_median": round(float(np.median(step_ms)), 4),
                      "gather_event_mean": round(g_avg, 4),
                      "gather_event_min": round(float(gather_ms.min()), 4),
                      "mu_event_mean": round(float(mu_ms.mean()), 4),
                      "reduce_event_mean": round(float(reduce_ms.mean()), 4)},
        "roofline": {"bound": bound, "achieved": round(achieved, 3), "peak": FP32_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / FP32_PEAK_TFLOPS, 4),
                     "traffic": None if traffic is None else round(traffic, 3),
                     "traffic_unit": "GB/s (HBM bytes per launch from FETCH_SIZE/WRITE_SIZE / launch time)",
                     "traffic_detail": traffic_detail,
                     "kernel": kernel,
                     "flop_per_pair": round(mr["flop_per_voxel_sample"] / p.B, 4),
                     "achieved_is": "the method's FLOP per launch (flop_per_pair x pairs) / gather time",
                     "method_roofline": mr, "engine": eng},
    }
    if p.B > 1:
        # value counts voxel-sample-vector triples; a trajectory pass is the N M
        # voxel-sample pairs whose phase, sine and cosine the B vectors share
        res["per_trajectory_pass"] = {"value": round(value / p.B, 3), "unit": "Gpair/s",
                                      "is": "N M / step time (value = B N M / step time)"}
    if not forward and engine == "mfma" and args.half_steps > 0:
        res["half_split_engine"] = time_half_engine(p, t, D, args, stream)
    if not forward and not (engine == "valu" and plan["voxels_per_lane"] == 1) and args.method_steps > 0:
        res["method"] = time_per_pair_kernel(p, t, D, args, stream, mr)
    if args.cpu_seconds > 0:
        res["cpu_baseline"] = cpu_baseline(p, args.cpu_seconds, rho.cpu().numpy() if forward else None)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
