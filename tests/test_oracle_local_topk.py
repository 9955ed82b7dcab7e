"""Pins for the oracle's Local + TopK selection (VMoBA review: the training-free experiments'
selection, k = 2, 6 or 18): local blocks from a token-to-block map, brute force over the
non-local blocks, and the limiting cases (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle


def _local_by_token_map(grid, qpart, kvpart):
    # an independent construction: label every token with its kv block, read the labels of each
    # query block's tokens
    qb, kb = oracle.partition(grid, qpart), oracle.partition(grid, kvpart)
    label = np.empty(int(np.prod(grid)), np.int64)
    for j, b in enumerate(kb):
        label[b] = j
    return [np.unique(label[b]) for b in qb], qb, kb


@pytest.mark.parametrize("grid,qpart,kvpart", [
    ((6, 9, 20), ("tile", (4, 4, 8)), ("tile", (4, 4, 8))),
    ((6, 9, 20), ("tile", (4, 4, 8)), ("tile", (3, 9, 20))),
    ((6, 9, 20), ("tile", (4, 4, 8)), ("tile", (6, 3, 5))),
    ((4, 8, 8), ("flat", 32), ("flat", 20)),
])
def test_local_blocks_match_the_token_labels(grid, qpart, kvpart):
    ref, qb, kb = _local_by_token_map(grid, qpart, kvpart)
    got = oracle.local_blocks(qb, kb)
    assert len(got) == len(qb)
    for a, b in zip(got, ref):
        np.testing.assert_array_equal(a, b)
    if qpart == kvpart:                      # one partition: each block is its own local block
        assert all(g.tolist() == [i] for i, g in enumerate(got))


@pytest.mark.parametrize("seed", range(15))
def test_topk_part_is_the_best_k_subset_by_brute_force(seed):
    rng = np.random.default_rng(300 + seed)
    nq, nkv = 3, int(rng.integers(3, 8))
    S = rng.random((1, 2, nq, nkv))
    local = [np.sort(rng.choice(nkv, size=int(rng.integers(0, 3)), replace=False))
             for _ in range(nq)]
    k = int(rng.integers(0, nkv))
    rows = oracle.select_local_topk(S, k, local)
    for r, sel in enumerate(rows):
        h, i = divmod(r, nq)
        loc = set(local[i].tolist())
        assert loc <= set(sel.tolist())
        extra = [j for j in sel.tolist() if j not in loc]
        others = [j for j in range(nkv) if j not in loc]
        kk = min(k, len(others))
        assert len(extra) == kk
        best = max(itertools.combinations(others, kk), key=lambda c: S[0, h, i, list(c)].sum())
        assert sorted(best) == sorted(extra)


def test_limits_and_ties():
    S = np.asarray([0.4, 0.1, 0.2, 0.2, 0.1]).reshape(1, 1, 1, 5)
    assert oracle.select_local_topk(S, 0, [np.asarray([3])])[0].tolist() == [3]
    assert oracle.select_local_topk(S, 9, [np.asarray([3])])[0].tolist() == [0, 1, 2, 3, 4]
    # equal scores go to the lower index: 0.2 at 2 (3 is local), then 0.1 at 1 before 4
    assert oracle.select_local_topk(S, 3, [np.asarray([3])])[0].tolist() == [0, 1, 2, 3]
    assert oracle.select_local_topk(S, 1, [np.zeros(0, np.int64)])[0].tolist() == [0]
