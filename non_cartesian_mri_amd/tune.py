"""Launch-configuration sweep with Pareto pruning for F^H D / Q.

PMPP ch. 17 "Iterative MRI reconstruction", section 17.3 step 4: the kernel's
configuration parameters interact (more of one uses resources another could
have used), so they are tuned jointly by experiment; a systematic search over
all combinations beat heuristic tuning by about 20 %, and Ryoo et al. (2008)
prune most poor combinations with a Pareto-optimal curve of two static
metrics before timing anything.

Here the parameters are the engine's group size (voxels per lane for the VALU
engine; voxels per group phase, hence factor tiles, for the matrix-core
engine), the number of sample rows (split-M) and the summation tile.  Each
candidate gets two static metrics from the library's own plan
(fhd_describe_plan) and a simple issue model of the engine:

  efficiency   1 / (modelled SIMD issue cycles of the whole operation: the
               gather's per-sample work on every wave and row, the tile folds,
               and the row reduction's memory traffic at HBM speed);
  utilization  the fraction of resident-wave slots the launch keeps busy over
               its rounds (waves / (rounds * resident capacity)), times the
               share of a row's record stream that an XCD's L2 can hold
               (1 / (1 + row stream bytes / 4 MiB)): more rows mean shorter
               streams that the waves of an XCD share, at the price of more
               partial sums to reduce (the efficiency side).

Only candidates on the Pareto front of (efficiency, utilization) are timed
(optionally all of them, to check that pruning kept the best).  Timing uses
HIP events on the current stream around fhd_compute / q_compute; every timed
output is compared with the default plan's output.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

SIMDS = 256 * 4                   # MI355X: 256 CUs x 4 SIMDs
L2_BYTES = 4 << 20                # L2 per XCD
CLOCK_HZ = 2.4e9
HBM_BYTES_PER_S = 5.0e12          # sustained streaming rate used for the reduction term

# Issue model (cycles on one SIMD), from the gfx950 issue-rate measurements:
# a wave64 VALU op occupies its SIMD for 4 cycles; on the matrix-core engine a
# 32x32x2 f32 MFMA keeps the matrix pipe busy 64 cycles (a 16x16x4 one 32),
# and VALU work that does not overlap it adds ~2.7 cycles per FMA and ~8.8
# per v_sin.
MFMA_CYCLES = 64.0
MFMA_FMA_EXTRA = 2.7
MFMA_SIN_EXTRA = 8.8
VALU_CYCLES = 4.0


@dataclass
class Candidate:
    engine: str
    voxels_per_lane: int
    sample_splits: int
    tile: int
    plan: dict = field(default_factory=dict)
    efficiency: float = 0.0
    utilization: float = 0.0
    ms: float | None = None
    rel_to_default: float | None = None

    def opts(self) -> dict:
        return dict(engine=self.engine, voxels_per_lane=self.voxels_per_lane,
                    sample_splits=self.sample_splits, tile=self.tile)


def pareto_front(points) -> list[int]:
    """Indices of the points (a, b) not dominated by any other (both maximised)."""
    front = []
    for i, (a, b) in enumerate(points):
        dominated = False
        for j, (c, d) in enumerate(points):
            if j != i and c >= a and d >= b and (c > a or d > b):
                dominated = True
                break
        if not dominated:
            front.append(i)
    return front


def _regular(group: int, edge: int | None) -> bool:
    """Whether groups of `group` consecutive voxels tile a cubic grid's rows."""
    if not edge:
        return True
    if edge % group == 0:
        return True
    return group % edge == 0 and (edge * edge) % group == 0


def static_metrics(c: Candidate, M: int, N: int, batch: int, is_q: bool, trig: str) -> tuple[float, float]:
    p = c.plan
    rows = max(1, p["sample_splits"])
    mpad = p["padded_samples"]
    tile = max(1, p["tile"])
    V = max(1, p["voxels_per_lane"])
    if p["engine"] == 2:   # matrix-core engine, three real products per complex product
        T = max(1, (V * min(batch, 16)) // 16) if not is_q else max(1, V // 16)
        four = T >= 8      # four-sample engine: 16 groups per wave, 4 samples per 16x16x4 MFMA
        ks = 4 if four else 2
        waves_row = math.ceil(N / ((16 if four else 32) * V))
        capacity = SIMDS * (2 if T >= 4 else 4)
        # per sample and wave: 3 T / ks MFMAs of 64 cycles (32x32x2, 32 groups x
        # 32 columns) or 3 T / 4 of 32 cycles (16x16x4); one phase with its sine
        # and cosine per lane and ks samples; tile folds of the accumulators
        mfma = 3 * (T / 2) * MFMA_CYCLES / 2 if not four else 3 * T * (MFMA_CYCLES / 2) / 4
        trig_extra = (2 * MFMA_SIN_EXTRA + 6 * MFMA_FMA_EXTRA) if trig == "hw" else 33 * MFMA_FMA_EXTRA
        per_sample = mfma + trig_extra / ks + ((28 if four else 56) * T / tile) * MFMA_FMA_EXTRA
    else:                  # VALU engine: a lane owns V voxels, 64 lanes per wave
        waves_row = math.ceil(N / (64 * V))
        capacity = SIMDS * 4
        trig_ops = 8 if trig == "hw" else 30
        per_sample = (3 * V * min(batch, 16) + trig_ops + (6 * V / tile)) * VALU_CYCLES
    waves = waves_row * rows * max(1, p["passes"])
    gather_cycles = waves * (mpad / rows) * per_sample / SIMDS      # spread over all SIMDs
    reduce_bytes = 0 if rows == 1 else 2 * rows * batch * N * 8
    reduce_cycles = reduce_bytes / HBM_BYTES_PER_S * CLOCK_HZ
    rounds = math.ceil(waves / capacity)
    fill = waves / (rounds * capacity)
    row_stream = (mpad / rows) * p["record_dwords"] * 4
    utilization = fill / (1.0 + row_stream / L2_BYTES)
    # a launch that cannot fill the GPU runs at the share of SIMDs it uses
    efficiency = 1.0 / ((gather_cycles / fill) + reduce_cycles)
    return efficiency, utilization


def candidates(M: int, N: int, batch: int = 1, is_q: bool = False, *, engines=("mfma",), trig="hw",
               sum="blocked", grid_edge: int | None = None) -> list[Candidate]:
    """Every configuration of the sweep with a valid plan and its static metrics."""
    from .fhd import fhd_describe_plan
    out = []
    rows_set = [1, 2, 4, 8, 16, 32, 64]
    # the last tile covers every launch row whole: the row-block summation
    # (on the four-sample engine, the kernel without running totals)
    row_tile = max(4096, (M + 31) // 32 * 32)
    tiles = [128, 256, 512, 1024, 2048, 4096] + ([row_tile] if row_tile > 4096 else [])
    for engine in engines:
        groups = [32, 64, 128] if engine == "mfma" else [1, 2, 4, 8, 16]
        for V in groups:
            if engine == "mfma" and not _regular(V, grid_edge):
                continue
            for rows in rows_set:
                if rows > max(1, M // 64):
                    continue
                for tile in tiles:
                    if tile > max(128, M) and tile != row_tile:
                        continue
                    c = Candidate(engine, V, rows, tile)
                    try:
                        c.plan = fhd_describe_plan(M, N, batch, is_q, trig=trig, sum=sum, **c.opts())
                    except Exception:
                        continue
                    if c.plan["sample_splits"] != rows:
                        continue   # capped by the partial-sum limit: same as another candidate
                    c.efficiency, c.utilization = static_metrics(c, M, N, batch, is_q, trig)
                    out.append(c)
    return out


def sweep(t: dict, D=None, *, trig="hw", sum="blocked", engines=("mfma",), exhaustive=False, reps=3,
          grid_edge: int | None = None) -> dict:
    """Time the Pareto front (or every candidate) on device tensors t = {kx, ky, kz, x, y, z, phi}.

    D: complex64 [B, M] data vectors for F^H D, or None for Q.
    """
    import numpy as np
    import torch
    from .fhd import fhd_compute, fhd_workspace_bytes, q_compute
    is_q = D is None
    M, N = t["kx"].numel(), t["x"].numel()
    B = 1 if is_q else D.shape[0]
    cands = candidates(M, N, B, is_q, engines=engines, trig=trig, sum=sum, grid_edge=grid_edge)
    front = pareto_front([(c.efficiency, c.utilization) for c in cands])
    stream = torch.cuda.current_stream()

    def run(opts, out, ws):
        if is_q:
            q_compute(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], trig=trig, sum=sum,
                      out=out.view(-1), workspace=ws, **opts)
        else:
            fhd_compute(t["kx"], t["ky"], t["kz"], t["x"], t["y"], t["z"], t["phi"], D, trig=trig, sum=sum,
                        out=out, workspace=ws, **opts)

    def time_opts(opts):
        nbytes = fhd_workspace_bytes(M, N, B, is_q, trig=trig, sum=sum, **opts)
        ws = torch.empty(max(1, nbytes), dtype=torch.uint8, device=t["kx"].device)
        out = torch.empty((B, N), dtype=torch.complex64, device=t["kx"].device)
        run(opts, out, ws)
        best = math.inf
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            run(opts, out, ws)
            e1.record(stream)
            e1.synchronize()
            best = min(best, e0.elapsed_time(e1))
        return best, out.cpu().numpy()

    import time
    default_opts = {"engine": engines[0]} if engines[0] != "auto" else {}
    t_end = time.perf_counter() + 0.5
    for _ in range(3):      # bring the clocks up before the first timing: 3 runs and at least 0.5 s
        time_opts(default_opts)
    while time.perf_counter() < t_end:
        time_opts(default_opts)
    default_ms, ref = time_opts(default_opts)
    timed = range(len(cands)) if exhaustive else front
    for i in timed:
        c = cands[i]
        c.ms, got = time_opts(c.opts())
        c.rel_to_default = float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30))
    default_ms = min(default_ms, time_opts(default_opts)[0])   # and once more after the sweep
    timed_c = [cands[i] for i in timed]
    best = min(timed_c, key=lambda c: c.ms)
    result = {
        "candidates": len(cands), "front": len(front), "timed": len(timed_c),
        "timings": [dict(cands[i].opts(), ms=cands[i].ms, on_front=i in front) for i in timed],
        "default_ms": default_ms,
        "best": dict(best.opts(), ms=best.ms, efficiency=best.efficiency, utilization=best.utilization),
        "front_configs": [dict(cands[i].opts(), ms=cands[i].ms, efficiency=cands[i].efficiency,
                               utilization=cands[i].utilization) for i in front],
        "max_rel_to_default": max(c.rel_to_default for c in timed_c),
    }
    if exhaustive:
        best_front = min((cands[i] for i in front), key=lambda c: c.ms)
        result["best_on_front"] = dict(best_front.opts(), ms=best_front.ms)
        result["front_loss"] = best_front.ms / best.ms - 1.0
    return result
