"""The configuration sweep on the GPU (non_cartesian_mri_amd/tune.py): every
timed configuration computes the same F^H D as the default plan (within the
accurate-trig parity bar), and the Pareto-pruned sweep times fewer
configurations than the exhaustive one."""
import numpy as np
import pytest
import torch

from non_cartesian_mri_amd import inputs
from tests.gpu_util import dev_problem, require_gpu

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def test_sweep_configs_agree_and_pruning_times_fewer():
    from non_cartesian_mri_amd import tune
    p = inputs.make_config("fhd_32cube_2048_uniform")
    d = dev_problem(p)
    full = tune.sweep(d, d["D"], trig="accurate", exhaustive=True, reps=1, grid_edge=32)
    pruned = tune.sweep(d, d["D"], trig="accurate", exhaustive=False, reps=1, grid_edge=32)
    print(f"[tune] 32^3 x 2048: {full['candidates']} candidates, front {full['front']}, "
          f"best {full['best']}, best on front {full['best_on_front']}, loss {full['front_loss']:.3f}", flush=True)
    assert full["timed"] == full["candidates"] and pruned["timed"] == pruned["front"] < pruned["candidates"]
    assert full["max_rel_to_default"] <= 1e-5 and pruned["max_rel_to_default"] <= 1e-5
