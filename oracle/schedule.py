"""CPU oracle of the balanced split plan of the verify attention -- TEST INFRASTRUCTURE ONLY.

Only tests/, the smoke check in __graft_entry__ and bench.py's CPU-baseline leg may import this
module; the HIP library shares no code with it.

The plan partitions a ragged batch over a fixed budget of `units` splits ("From Capture Safety to
MoE Ceiling", section "The Architecture of Capture Safety": a fixed grid whose chunk bounds come from
the actual lengths on the device; section "The Occupancy Calculation": the split count is chosen so
every SM has work). Reading taken where the pages are silent: work is counted in 32-column tiles,
T_b = ceil(L_b / 32); the split size is the smallest C with sum_b ceil(T_b / C) <= units; request b
gets n_b = ceil(T_b / C) splits, split s covering tiles [floor(s T_b / n_b), floor((s+1) T_b / n_b));
splits are numbered request after request.

Pins (tests/test_schedule_oracle.py): brute force over every split-count vector on small cases
(the plan's largest split is the smallest possible), exact tiling of every request's columns, and
the per-request special case units = B (one split per request).
"""
from __future__ import annotations

import math

TILE = 32


def tiles(kv_indptr, B, q_len):
    return [math.ceil((max(0, int(kv_indptr[b + 1]) - int(kv_indptr[b])) + q_len) / TILE) for b in range(B)]


def balanced_plan(kv_indptr, B: int, q_len: int, units: int):
    """Returns (split_start [B+1], req_of_split [units], column ranges [(b, c_begin, c_end)] per split)."""
    if units < B:
        raise ValueError("units must be at least B")
    T = tiles(kv_indptr, B, q_len)
    C = 1
    while sum(math.ceil(t / C) for t in T) > units:   # smallest split size that fits the budget
        C += 1
    n = [math.ceil(t / C) for t in T]
    split_start = [0]
    for b in range(B):
        split_start.append(split_start[-1] + n[b])
    req = [-1] * units
    ranges = []
    for b in range(B):
        L = max(0, int(kv_indptr[b + 1]) - int(kv_indptr[b])) + q_len
        for s in range(n[b]):
            req[split_start[b] + s] = b
            t0, t1 = (s * T[b]) // n[b], ((s + 1) * T[b]) // n[b]
            ranges.append((b, t0 * TILE, min(L, t1 * TILE)))
    return split_start, req, ranges
