"""Brute-force optimum of the one-GPU packing problem (CPU, exact, small n).

TEST INFRASTRUCTURE ONLY: used by ``tests/`` and the CPU leg of ``bench.py``.

The problem is the planner's [PLoRA technical summary (gist.science, arXiv
2508.02932), 方法论 > 1. LoRA 打包规划器] on a pool of one GPU: split the jobs
into packs that run one after another, each within the memory budget, so
that the total time is smallest.  A pack costs fixed_ms * (its longest job's
steps) + sum over its jobs of steps * ms_per_step.  Memory is counted in whole
quanta: a job takes ceil(mem_bytes / quantum) of the floor(budget / quantum)
a pack has.  This file tries every partition of the jobs into packs (set
partitions, Bell-number many) and every subset for one knapsack fill; it is
the definition written out, for instances small enough to enumerate.

Pins (``tests/test_planner.py``): the partition counts are the Bell numbers;
closed forms (every job fits in one pack; no two jobs fit together); a
hand-worked instance.
"""
from __future__ import annotations

import itertools
import math


def quanta(mem, q):
    return math.ceil(mem / q - 1e-9)


def set_partitions(items):
    """Every partition of the list `items` into non-empty blocks."""
    if not items:
        yield []
        return
    first, rest = items[0], items[1:]
    for part in set_partitions(rest):
        for i in range(len(part)):  # put `first` into an existing block
            yield part[:i] + [[first] + part[i]] + part[i + 1:]
        yield [[first]] + part      # or into a block of its own


def pack_cost(jobs, pack, fixed_ms):
    """jobs: list of (steps, mem_bytes, ms_per_step)."""
    return fixed_ms * max(jobs[k][0] for k in pack) + sum(jobs[k][0] * jobs[k][2] for k in pack)


def feasible(jobs, pack, budget, q):
    return sum(quanta(jobs[k][1], q) for k in pack) <= math.floor(budget / q + 1e-9)


def best_plan(jobs, budget, fixed_ms, q):
    """(smallest makespan, one partition achieving it) over every feasible partition."""
    best = (math.inf, None)
    for part in set_partitions(list(range(len(jobs)))):
        if all(feasible(jobs, p, budget, q) for p in part):
            cost = sum(pack_cost(jobs, p, fixed_ms) for p in part)
            if cost < best[0]:
                best = (cost, part)
    return best


def best_fill(jobs, cands, cap_quanta, q):
    """Largest total steps of a subset of `cands` within cap_quanta quanta."""
    best = 0
    for n in range(len(cands) + 1):
        for sub in itertools.combinations(cands, n):
            if sum(quanta(jobs[k][1], q) for k in sub) <= cap_quanta:
                best = max(best, sum(jobs[k][0] for k in sub))
    return best
