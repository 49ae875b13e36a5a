"""Oracle (test infrastructure only): the stage partition, by exhaustive search.

RoundPipe popular article §六 and the RoundPipe paper summary (方法步骤详情, step 2): per-layer
times and memory are profiled, and layers are cut into contiguous stages so that the slowest stage
is as short as possible while each stage fits the GPU memory cap; forward and backward get separate
(asymmetric) partitions (user guide, stage 与 layer 的关系: a 12-layer model with backward about
three times forward splits into four 3-layer forward stages and twelve 1-layer backward stages);
backward stages are filled starting from the last layer.

The pages' objective "minimise the slowest stage" alone is degenerate (one-layer stages always
win), and the bubble model of the popular article (§三) charges N(N-1) warm-up/cool-down stage
slots against M*S useful ones. Reading used here: minimise

    J = (M * (S_f + S_b) + N * (N - 1)) * t_max

over all pairs of contiguous partitions (forward from layer 0, backward from layer L-1) whose
every stage has sum(time) <= t_max and sum(mem) <= cap; among minimisers take the smallest t_max,
then the pair whose stage-length sequences are lexicographically largest (longest stages first,
counted from the start of each pass). Integers throughout, so the answer is exact.

This module enumerates every partition (2^(L-1) per pass), so it is for small L only; it is the
definition the library's O(L^3) candidate-threshold search is checked against.
"""
from __future__ import annotations

import itertools
from typing import List, Optional, Sequence, Tuple


def _partitions(L: int):
    """Every composition of L (stage lengths, in pass order)."""
    for cuts in itertools.product((0, 1), repeat=L - 1):
        lens, run = [], 1
        for c in cuts:
            if c:
                lens.append(run)
                run = 1
            else:
                run += 1
        lens.append(run)
        yield tuple(lens)


def _stage_stats(lens, t, m):
    """Max stage time and max stage memory of a partition of the cost arrays t, m (pass order)."""
    pos, tmax, mmax = 0, 0, 0
    for ln in lens:
        tmax = max(tmax, sum(t[pos:pos + ln]))
        mmax = max(mmax, sum(m[pos:pos + ln]))
        pos += ln
    return tmax, mmax


def partition_bruteforce(t_f: Sequence[int], t_b: Sequence[int], m_f: Sequence[int],
                         m_b: Sequence[int], mem_cap: int, n_gpus: int, n_micro: int
                         ) -> Optional[Tuple[List[int], List[int], int, int]]:
    """Returns (forward stage lengths from layer 0, backward stage lengths from layer L-1,
    t_max, J), or None when some single layer exceeds the memory cap."""
    L = len(t_f)
    tb_rev, mb_rev = list(t_b)[::-1], list(m_b)[::-1]
    fwd = []
    for lens in _partitions(L):
        tm, mm = _stage_stats(lens, t_f, m_f)
        if mm <= mem_cap:
            fwd.append((lens, tm))
    bwd = []
    for lens in _partitions(L):
        tm, mm = _stage_stats(lens, tb_rev, mb_rev)
        if mm <= mem_cap:
            bwd.append((lens, tm))
    if not fwd or not bwd:
        return None
    best = None
    for (lf, tf), (lb, tb) in itertools.product(fwd, bwd):
        tmax = max(tf, tb)
        J = (n_micro * (len(lf) + len(lb)) + n_gpus * (n_gpus - 1)) * tmax
        key = (J, tmax, tuple(-x for x in lf), tuple(-x for x in lb))
        if best is None or key < best[0]:
            best = (key, lf, lb, tmax, J)
    _, lf, lb, tmax, J = best
    return list(lf), list(lb), tmax, J


def stage_bounds(lens: Sequence[int], L: int, backward: bool) -> List[int]:
    """Stage start layers: forward from layer 0 upward; backward as the highest layer of each stage
    counted from layer L-1 downward."""
    out, pos = [], 0
    for ln in lens:
        out.append(L - 1 - pos if backward else pos)
        pos += ln
    return out
