"""Pins of the balanced split plan oracle (no GPU)."""
import itertools
import math

import numpy as np
import pytest

from oracle import schedule as S


def _indptr(lengths, q_len):
    return np.concatenate([[0], np.cumsum([L - q_len for L in lengths])])


@pytest.mark.parametrize("seed", range(25))
def test_largest_split_is_minimal_brute_force(seed):
    rng = np.random.default_rng(seed)
    B = int(rng.integers(1, 4))
    q_len = int(rng.integers(1, 5))
    lengths = [int(x) for x in rng.integers(q_len, 400, B)]
    units = int(rng.integers(B, B + 7))
    ip = _indptr(lengths, q_len)
    split_start, req, ranges = S.balanced_plan(ip, B, q_len, units)
    T = S.tiles(ip, B, q_len)
    got = max((c1 - c0 + 31) // 32 for _, c0, c1 in ranges)
    best = min(max(math.ceil(T[b] / n[b]) for b in range(B))
               for n in itertools.product(range(1, units + 1), repeat=B) if sum(n) <= units)
    assert got == best
    assert split_start[-1] <= units and all(split_start[b + 1] > split_start[b] for b in range(B))


@pytest.mark.parametrize("seed", range(10))
def test_splits_tile_every_request_exactly(seed):
    rng = np.random.default_rng(50 + seed)
    B, q_len = int(rng.integers(1, 9)), int(rng.integers(1, 17))
    lengths = [int(x) for x in rng.integers(q_len, 5000, B)]
    units = int(rng.integers(B, 300))
    ip = _indptr(lengths, q_len) + 3
    split_start, req, ranges = S.balanced_plan(ip, B, q_len, units)
    for b in range(B):
        mine = [(c0, c1) for rb, c0, c1 in ranges if rb == b]
        assert mine[0][0] == 0 and mine[-1][1] == lengths[b]
        assert all(mine[k][1] == mine[k + 1][0] and mine[k][0] < mine[k][1] for k in range(len(mine) - 1))
        assert all(req[j] == b for j in range(split_start[b], split_start[b + 1]))
    assert all(r == -1 for r in req[split_start[-1]:])


def test_units_equal_b_is_one_split_per_request():
    ip = np.array([0, 100, 100, 5000])
    split_start, req, ranges = S.balanced_plan(ip, 3, 9, 3)
    assert split_start == [0, 1, 2, 3] and req == [0, 1, 2]
    assert ranges == [(0, 0, 109), (1, 0, 9), (2, 0, 4909)]


def test_ragged_185k_batch_plan():
    """The ragged B=4 batch (prefixes 4096/32768/120000/185000, q_len 16) over 32 splits: the 4k request
    gets one split, the rest near-equal splits of at most C tiles."""
    ip = np.concatenate([[0], np.cumsum([4096, 32768, 120000, 185000])])
    split_start, req, ranges = S.balanced_plan(ip, 4, 16, 32)
    T = S.tiles(ip, 4, 16)
    assert T == [129, 1025, 3751, 5782]
    sizes = [(c1 - c0 + 31) // 32 for _, c0, c1 in ranges]
    assert split_start[1] == 1 and max(sizes) <= math.ceil(sum(T) / (32 - 4)) + 1
    assert split_start[-1] <= 32
