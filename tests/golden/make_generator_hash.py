"""Records the SHA-256 of the tiny input set (run once, when the recipe changes)."""
import os
import sys

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__)))))
from tests.test_workloads import _digest  # noqa: E402
from mhc_hyper_connection_boundary_amd import workloads as WL  # noqa: E402

with open(os.path.join(os.path.dirname(os.path.abspath(__file__)), "generator_tiny.sha256"), "w") as f:
    f.write(_digest(WL.make_inputs("tiny")) + "  tiny input set (d=256, T=8, seed 0)\n")
