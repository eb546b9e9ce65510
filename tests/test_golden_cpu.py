"""The figures the pages print (tests/golden/pages_figures.json, each with its
citation), checked for internal consistency, and the reconstruction-quality
gate the GPU phantom test takes from them.

The pages print no F^H D or Q values for a worked input; those outputs are
pinned by closed forms and brute force in the oracle pin tests.
"""
import json
import math
import os

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def figures() -> dict:
    with open(GOLDEN) as f:
        return json.load(f)


def psnr_drop_gate_db() -> float:
    """Largest PSNR loss allowed when hardware trigonometry replaces the
    software path: the drop the pages report for their phantom."""
    p = figures()["psnr_db"]
    return round(p["iterative_software_trig"] - p["iterative_hardware_trig"], 6)


def test_psnr_figures():
    p = figures()["psnr_db"]
    assert psnr_drop_gate_db() == 0.1
    # the iterative image beats gridding by a wide margin on the pages' data
    assert p["iterative_hardware_trig"] - p["gridding"] > 10.0


def test_op_per_byte_figures():
    o = figures()["op_per_byte"]
    for name, accesses in o["accesses"].items():
        ratio = o["fp_ops_per_iteration"] / (accesses * o["bytes_per_access"])
        # the pages print two decimals, truncated or rounded
        assert abs(ratio - o["ratios"][name]) < 0.006, name


def test_launch_arithmetic():
    a = figures()["launch_arithmetic"]
    assert math.ceil(a["samples"] / a["threads_per_block"]) == a["cmpmu_blocks"]
    assert a["block"] * a["threads_per_block"] + a["thread"] == a["iteration"]
    assert a["voxels"] == 128 ** 3 and a["voxels"] // a["threads_per_block"] == a["cmpfhd_blocks"]
