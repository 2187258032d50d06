"""Plain CPU oracle for compute-balanced packing of trajectories.

TEST INFRASTRUCTURE ONLY: used by the tests, never by the product path; it
shares no code with the library.

"On-Policy Residual Learning for Diffusion Language Models" (paper cards page,
abstract and Figure 3 caption; thread page, Insight 3) packs the captured
trajectories and balances them by compute before replay.  The pages give no
balancing rule; the one taken is the longest-processing-time greedy rule:
take the trajectories in order of decreasing cost (ties: lower index first)
and put each into the bin whose cost so far is least (ties: lower bin).  The
cost of a trajectory is the number of (query, key) pairs its attention admits
per query head -- here counted directly from the admitted-key matrix.
"""
from __future__ import annotations

import numpy as np

from .attention import allowed_matrix, allowed_matrix_groups


def trajectory_cost(seqlen: int, s_copies: int, block_size: int) -> int:
    """Admitted pairs of one trajectory, counted cell by cell from the mask."""
    return int(allowed_matrix(seqlen, s_copies, block_size).sum())


def trajectory_cost_groups(seqlen: int, groups, block_size: int) -> int:
    """Admitted pairs of one general-staircase trajectory (copy groups
    [(pe, copies), ...]), counted cell by cell from its mask."""
    return int(allowed_matrix_groups(seqlen, groups, block_size).sum())


def lpt(costs, nbins: int):
    """Greedy longest-processing-time assignment of items with ``costs``.

    Returns (bin_of [n], bin_cost [nbins], order [n], bin_start [nbins + 1])
    with the same conventions as the library: ``order`` lists each bin's items
    in the order they were placed.
    """
    costs = [int(c) for c in costs]
    n = len(costs)
    by_cost = sorted(range(n), key=lambda i: (-costs[i], i))
    bin_cost = [0] * nbins
    members = [[] for _ in range(nbins)]
    bin_of = [0] * n
    for i in by_cost:
        b = min(range(nbins), key=lambda j: (bin_cost[j], j))
        bin_of[i] = b
        bin_cost[b] += costs[i]
        members[b].append(i)
    order = [i for b in range(nbins) for i in members[b]]
    bin_start = [0]
    for b in range(nbins):
        bin_start.append(bin_start[-1] + len(members[b]))
    return (np.array(bin_of, dtype=np.int32), np.array(bin_cost, dtype=np.int64),
            np.array(order, dtype=np.int32), np.array(bin_start, dtype=np.int32))


def optimal_makespan(costs, nbins: int) -> int:
    """Smallest possible largest-bin cost, by trying every assignment (tiny inputs)."""
    costs = [int(c) for c in costs]
    best = None
    n = len(costs)
    for code in range(nbins ** n):
        load = [0] * nbins
        c = code
        for i in range(n):
            load[c % nbins] += costs[i]
            c //= nbins
        m = max(load)
        best = m if best is None or m < best else best
    return int(best if best is not None else 0)
