"""Pins for the oracle's selected density (CPU only).

The density is the fraction of the N x N (query token, key token) pairs that the selection lets
attend, per head: the quantity the attention's work is proportional to (VMoBA review, "What
carries the argument": only the selected blocks' key-value pairs contribute, so the cost scales
with the number of selected pairs). Pinned by closed forms and by a direct count over token
pairs that uses no block sizes at all.
"""
import numpy as np
import pytest

import oracle


def _sizes(blocks):
    return np.asarray([len(b) for b in blocks], np.int64)


@pytest.mark.parametrize("grid,part", [((4, 8, 8), ("flat", 32)),
                                       ((3, 5, 7), ("tile", (2, 2, 4))),
                                       ((5, 6, 9), ("tile", (5, 3, 2)))])
def test_every_block_selected_is_dense(grid, part):
    blocks = oracle.partition(grid, part)
    n = len(blocks)
    H, B = 3, 2
    rows = [np.arange(n) for _ in range(B * H * n)]
    d = oracle.density(rows, _sizes(blocks), _sizes(blocks), H, B)
    assert d == pytest.approx(1.0, abs=1e-15)


def test_one_one_token_block_per_row_is_one_over_n():
    # Query partition in 4-token runs, kv partition in one-token blocks; every query block
    # selects exactly one kv block, so each of the N queries attends to one key: density 1/N.
    grid = (2, 3, 4)
    N = 24
    qb = oracle.partition(grid, ("flat", 4))
    kb = oracle.partition(grid, ("flat", 1))
    rng = np.random.default_rng(5)
    H = 2
    rows = [np.asarray([int(rng.integers(0, N))]) for _ in range(H * len(qb))]
    d = oracle.density(rows, _sizes(qb), _sizes(kb), H)
    assert d == pytest.approx(1.0 / N, rel=1e-15)


def test_empty_rows_count_zero():
    blocks = oracle.partition((2, 4, 4), ("tile", (1, 2, 2)))
    n = len(blocks)
    rows = [np.zeros(0, np.int64) for _ in range(n)]
    assert oracle.density(rows, _sizes(blocks), _sizes(blocks), 1) == 0.0


@pytest.mark.parametrize("seed", range(6))
def test_density_equals_a_direct_count_of_token_pairs(seed):
    # Brute force: mark every (query token, key token) pair that a selected block admits in an
    # N x N boolean matrix per head, then count the marks.
    rng = np.random.default_rng(seed)
    grid = tuple(int(v) for v in rng.integers(2, 6, size=3))
    N = grid[0] * grid[1] * grid[2]
    qpart = ("tile", tuple(int(v) for v in rng.integers(1, 4, size=3)))
    kpart = ("tile", tuple(int(v) for v in rng.integers(1, 4, size=3)))
    qb, kb = oracle.partition(grid, qpart), oracle.partition(grid, kpart)
    B, H = 2, 2
    rows = []
    for _ in range(B * H * len(qb)):
        k = int(rng.integers(0, len(kb) + 1))
        rows.append(np.sort(rng.choice(len(kb), size=k, replace=False)))
    marked = 0
    for r, sel in enumerate(rows):
        I = r % len(qb)
        mask = np.zeros((N, N), bool)
        for J in sel:
            for i in qb[I]:
                for j in kb[J]:
                    mask[i, j] = True
        marked += int(mask.sum())
    d = oracle.density(rows, _sizes(qb), _sizes(kb), H, B)
    assert d == pytest.approx(marked / (B * H * N * N), rel=1e-14)
