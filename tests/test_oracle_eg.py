"""Pins for the oracle's entropy-routed selection (EG-Sparse abstract): closed forms of the head
entropy, scipy's entropy as an independent reference, reductions to per-row top-p, brute force
over the pooled pairs of a group, and the pool's weight normalisation (CPU only)."""
import itertools
import math

import numpy as np
import pytest
from scipy.stats import entropy as scipy_entropy

import oracle


def _row_norm(x):
    return x / x.sum(-1, keepdims=True)


def test_entropy_closed_forms():
    nq, nkv = 3, 8
    qs = [128, 64, 8]
    uniform = np.full((1, 1, nq, nkv), 1.0 / nkv)
    onehot = np.zeros((1, 1, nq, nkv))
    onehot[0, 0, np.arange(nq), [0, 3, 7]] = 1.0
    assert oracle.head_entropy(uniform, qs)[0, 0] == pytest.approx(1.0, abs=1e-15)
    assert oracle.head_entropy(onehot, qs)[0, 0] == 0.0
    # two equal blocks per row: ln 2 / ln nkv for every row, whatever the weights
    two = np.zeros((1, 1, nq, nkv))
    two[0, 0, :, :2] = 0.5
    assert oracle.head_entropy(two, qs)[0, 0] == pytest.approx(math.log(2) / math.log(nkv))
    # one kv block: defined as 0
    assert oracle.head_entropy(np.ones((1, 2, 3, 1)), qs)[0, 1] == 0.0


def test_entropy_is_the_size_weighted_mean_of_scipy_entropies():
    rng = np.random.default_rng(7)
    B, H, nq, nkv = 2, 3, 5, 9
    S = _row_norm(rng.exponential(size=(B, H, nq, nkv)) ** 3)
    S[0, 1, 2, 4] = 0.0            # a zero score contributes nothing
    S = _row_norm(S)
    qs = np.asarray([128, 128, 64, 32, 8])
    ent = oracle.head_entropy(S, qs)
    for b in range(B):
        for h in range(H):
            rows = [scipy_entropy(S[b, h, i]) for i in range(nq)]
            ref = float(np.dot(qs, rows)) / (qs.sum() * math.log(nkv))
            assert ent[b, h] == pytest.approx(ref, rel=1e-12)


def test_no_pooled_head_is_per_row_topp():
    rng = np.random.default_rng(1)
    S = _row_norm(rng.exponential(size=(2, 5, 4, 7)) ** 2)
    qs = [100, 80, 60, 20]
    for gs in (1, 2, 5):
        rows = oracle.select_group(S, 0.8, qs, np.zeros((2, 5), bool), gs)
        assert all(np.array_equal(a, b) for a, b in zip(rows, oracle.select_row(S, 0.8)))
    rows, ent, pooled = oracle.select_eg(S, 0.8, qs, 0.0, 2)   # theta 0 routes nothing
    assert not pooled.any()


def _brute_force(w, p):
    n = len(w)
    for k in range(1, n + 1):
        feasible = [c for c in itertools.combinations(range(n), k) if w[list(c)].sum() >= p]
        if feasible:
            return k, max(w[list(c)].sum() for c in feasible)
    return n, w.sum()


@pytest.mark.parametrize("seed", range(12))
def test_group_pool_brute_force(seed):
    rng = np.random.default_rng(200 + seed)
    H, nq, nkv = 3, int(rng.integers(1, 3)), int(rng.integers(2, 4))
    S = _row_norm(rng.exponential(size=(1, H, nq, nkv)) ** 2)
    qs = rng.integers(1, 9, size=nq)
    pooled = np.zeros((1, H), bool)
    pooled[0, rng.permutation(H)[: int(rng.integers(1, 3))]] = True
    members = [h for h in range(H) if pooled[0, h]]
    p = float(rng.uniform(0.1, 0.95))
    rows = oracle.select_group(S, p, qs, pooled, H)
    # the pooled weights, written out directly: each pooled head contributes total weight 1/m
    m = len(members)
    w = np.concatenate([(S[0, h] * qs[:, None] / (qs.sum() * m)).reshape(-1) for h in members])
    assert w.sum() == pytest.approx(1.0)
    chosen = [(k, i, j) for k, h in enumerate(members) for i in range(nq)
              for j in rows[h * nq + i].tolist()]
    k_best, best = _brute_force(w, p)
    assert len(chosen) == k_best
    got = sum(w[(k * nq + i) * nkv + j] for k, i, j in chosen)
    assert got == pytest.approx(best, abs=1e-12)
    # the other heads select per row
    for h in range(H):
        if not pooled[0, h]:
            for i in range(nq):
                assert np.array_equal(rows[h * nq + i], oracle.select_topp(S[0, h, i], p))


def test_groups_are_independent_runs_of_heads():
    rng = np.random.default_rng(5)
    H, nq, nkv = 5, 3, 4
    S = _row_norm(rng.exponential(size=(1, H, nq, nkv)) ** 4)
    qs = [64, 64, 16]
    pooled = np.ones((1, H), bool)
    rows = oracle.select_group(S, 0.7, qs, pooled, 2)           # groups {0,1} {2,3} {4}
    for g in ([0, 1], [2, 3], [4]):
        alone = oracle.select_group(S[:, g], 0.7, qs, np.ones((1, len(g)), bool), len(g))
        for k, h in enumerate(g):
            for i in range(nq):
                assert np.array_equal(rows[h * nq + i], alone[k * nq + i])


def test_identical_heads_keep_identical_sets_at_full_weight_ties():
    # two identical pooled heads with distinct pair weights: the pool orders each weight's two
    # copies head 0 first, and when p is reached exactly after a pair of copies both heads end
    # with the same set
    S = np.zeros((1, 2, 1, 4))
    S[0, :, 0] = [0.5, 0.3, 0.15, 0.05]
    rows = oracle.select_group(S, 0.8, [10], np.ones((1, 2), bool), 2)
    assert rows[0].tolist() == [0, 1] and rows[1].tolist() == [0, 1]
    # p = 0.65 is reached after 0.25 + 0.25 + 0.15: head 0 keeps one block more than head 1
    rows = oracle.select_group(S, 0.65, [10], np.ones((1, 2), bool), 2)
    assert rows[0].tolist() == [0, 1] and rows[1].tolist() == [0]


def test_low_entropy_heads_are_routed():
    nq, nkv = 4, 16
    S = np.full((1, 2, nq, nkv), 1.0 / nkv)              # head 1 uniform: entropy 1
    S[0, 0] = 1e-3
    S[0, 0, np.arange(nq), np.arange(nq)] = 1.0           # head 0 nearly one-hot
    S = _row_norm(S)
    rows, ent, pooled = oracle.select_eg(S, 0.9, [16] * nq, 0.5, 2)
    assert ent[0, 0] < 0.5 < ent[0, 1]
    assert pooled.tolist() == [[True, False]]
    # head 0 alone in the pool: its diagonal pairs carry most of the pool
    assert all(rows[i].tolist() == [i] or i in rows[i].tolist() for i in range(nq))
    # head 1 per row: uniform rows keep ceil(0.9 * 16) blocks
    assert all(len(rows[nq + i]) == math.ceil(0.9 * nkv) for i in range(nq))
