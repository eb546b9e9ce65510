"""Host logic of the configuration sweep (non_cartesian_mri_amd/tune.py): the
Pareto front and the candidate set, no GPU."""
import pytest

from non_cartesian_mri_amd import tune


def test_pareto_front_hand_example():
    pts = [(1, 5), (2, 4), (3, 3), (2, 2), (1, 1), (3, 1), (0, 6), (3, 3)]
    # (2,2), (1,1), (3,1) are dominated; the two (3,3) tie and both stay
    assert tune.pareto_front(pts) == [0, 1, 2, 6, 7]


def test_pareto_front_single_and_chain():
    assert tune.pareto_front([(1.0, 1.0)]) == [0]
    assert tune.pareto_front([(i, i) for i in range(5)]) == [4]
    assert tune.pareto_front([(i, -i) for i in range(5)]) == [0, 1, 2, 3, 4]


@pytest.fixture(scope="module")
def lib():
    import os
    from non_cartesian_mri_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from non_cartesian_mri_amd.build import build_library
        build_library()
    return _lib.load()


def test_candidates_have_valid_plans_and_metrics(lib):
    cs = tune.candidates(262144, 128 ** 3, grid_edge=128)
    assert len(cs) == 3 * 7 * 7      # groups of 32, 64, 128 x rows x (6 tiles + the whole row)
    for c in cs:
        assert c.plan["sample_splits"] == c.sample_splits
        assert c.plan["voxels_per_lane"] == c.voxels_per_lane
        assert c.efficiency > 0 and 0 < c.utilization <= 1
    front = tune.pareto_front([(c.efficiency, c.utilization) for c in cs])
    assert 1 <= len(front) < len(cs)
    # groups that do not tile the rows of a 48^3 grid are left out of the matrix-core sweep
    assert all(c.voxels_per_lane not in (64, 128) for c in tune.candidates(4096, 48 ** 3, grid_edge=48))


def test_more_rows_trade_efficiency_for_utilization(lib):
    cs = [c for c in tune.candidates(262144, 128 ** 3, grid_edge=128)
          if c.voxels_per_lane == 64 and c.tile == 512]
    cs.sort(key=lambda c: c.sample_splits)
    # one row: 1024 waves of 32 groups x 64 voxels half-fill the 2048 slots
    assert cs[0].sample_splits == 1 and cs[0].efficiency < 0.6 * cs[1].efficiency
    full = cs[1:]     # 2 rows and more fill the GPU
    eff = [c.efficiency for c in full]
    util = [c.utilization for c in cs]
    assert eff == sorted(eff, reverse=True)
    assert util == sorted(util)
