"""fp64 CPU oracle for block-causal / staircase attention.

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP library (see ``attention.py`` for what it computes and the
passages it follows; ``packing.py`` holds the compute-balanced packing rule).

Every function here is pinned by ``tests/test_oracle.py`` against facts that
do not come from the oracle itself: torch's fp64 scaled-dot-product attention
for the block_size = 1 (causal) and block_size = L (full) special cases, a
hand-derived table of admitted keys, closed forms at Q = 0, finite differences
and torch autograd for the gradients, and the invariants of softmax attention.
"""
from .attention import (allowed_matrix, allowed_matrix_groups, attention_bwd,
                        attention_dq_rows, attention_fwd, decode, segment_allowed,
                        segment_prefix_len)
from .fp8 import e4m3_to_float
from .packing import lpt, optimal_makespan, trajectory_cost, trajectory_cost_groups

__all__ = ["allowed_matrix", "allowed_matrix_groups", "segment_allowed", "attention_bwd", "attention_dq_rows", "attention_fwd", "decode",
           "segment_prefix_len", "lpt", "optimal_makespan", "trajectory_cost", "trajectory_cost_groups",
           "e4m3_to_float"]
