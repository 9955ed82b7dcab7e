"""Pins for the oracle's selection rules: worked examples, brute force, invariants (CPU only)."""
import itertools
import json
import math
import os

import numpy as np
import pytest

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _gold():
    with open(os.path.join(GOLD, "selection_examples.json")) as f:
        return json.load(f)


def test_topp_worked_examples():
    for ex in _gold()["topp"]:
        sel = oracle.select_topp(np.asarray(ex["scores"]), ex["p"])
        assert sel.tolist() == ex["selected"], ex


def test_scope_min_k_worked_example():
    g = _gold()["scope_min_k"]
    k = oracle.head_min_k(g["counts"], g["qsizes"], g["nkv"])
    assert k == g["head_k"]
    assert [max(c, k) for c in g["counts"]] == g["final_counts"]


def _brute_force(s, p):
    n = len(s)
    best = None
    for k in range(1, n + 1):
        feasible = [c for c in itertools.combinations(range(n), k) if s[list(c)].sum() >= p]
        if feasible:
            best = (k, max(s[list(c)].sum() for c in feasible))
            break
    return best


@pytest.mark.parametrize("seed", range(40))
def test_topp_is_minimal_by_brute_force(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(2, 13))
    s = rng.exponential(size=n) ** rng.uniform(0.5, 3)
    s /= s.sum()
    p = float(rng.uniform(0.05, 0.99))
    sel = oracle.select_topp(s, p)
    k, best_mass = _brute_force(s, p)
    assert len(sel) == k
    assert abs(s[sel].sum() - best_mass) < 1e-12
    assert len(sel) <= math.ceil(p * n)


def test_topp_uniform_scores_exact_count():
    for n in (4, 8, 16, 32, 64):
        s = np.full(n, 1.0 / n)
        for p in (0.1, 0.25, 0.5, 0.6, 0.9, 0.99):
            assert len(oracle.select_topp(s, p)) == math.ceil(p * n)


def test_topp_nested_and_full():
    rng = np.random.default_rng(7)
    s = rng.dirichlet(np.full(50, 0.3))
    prev = set()
    for p in np.linspace(0.05, 0.999, 30):
        cur = set(oracle.select_topp(s, p).tolist())
        assert prev <= cur
        prev = cur
    assert oracle.select_topp(s, 1.0).tolist() == list(range(50))
    # never-reached threshold (sum < p) keeps everything
    assert oracle.select_topp(s * 0.5, 0.9).tolist() == list(range(50))


def test_select_row_shapes_and_order():
    rng = np.random.default_rng(8)
    S = rng.dirichlet(np.ones(9), size=(1, 2, 4))
    rows = oracle.select_row(S, 0.7)
    assert len(rows) == 8
    for r, sel in enumerate(rows):
        h, i = divmod(r, 4)
        assert np.all(np.diff(sel) > 0)
        assert sel.tolist() == oracle.select_topp(S[0, h, i], 0.7).tolist()


def test_hybrid_invariants():
    rng = np.random.default_rng(9)
    for trial in range(20):
        nq, nkv = int(rng.integers(2, 9)), int(rng.integers(3, 20))
        S = rng.dirichlet(np.full(nkv, rng.uniform(0.1, 3)), size=(1, 2, nq))
        sizes = rng.choice([8, 16, 32, 64, 128], size=nq)
        base = oracle.select_row(S, 0.8)
        rows, head_k = oracle.select_hybrid(S, 0.8, sizes)
        for h in range(2):
            c = [len(base[h * nq + i]) for i in range(nq)]
            k = head_k[h]
            assert min(c) <= k <= max(c)
            for i in range(nq):
                r = h * nq + i
                if c[i] >= k:
                    assert rows[r].tolist() == base[r].tolist()
                else:
                    assert len(rows[r]) == k
                    assert set(base[r].tolist()) <= set(rows[r].tolist())
                    # the added blocks are the next ones of the same ranking
                    order = np.lexsort((np.arange(nkv), -S[0, h, i]))
                    assert set(rows[r].tolist()) == set(order[:k].tolist())
    # identical counts: nothing is added
    S = np.tile(np.asarray([0.5, 0.3, 0.1, 0.1]), (1, 1, 3, 1))
    rows, head_k = oracle.select_hybrid(S, 0.75, [128, 64, 8])
    assert head_k[0] == 2 and all(len(r) == 2 for r in rows)


@pytest.mark.parametrize("seed", range(25))
def test_head_pool_brute_force(seed):
    rng = np.random.default_rng(100 + seed)
    nq, nkv = int(rng.integers(1, 5)), int(rng.integers(1, 5))
    W = rng.exponential(size=(1, 1, nq, nkv)) ** 2
    W /= W.sum()
    tau = float(rng.uniform(0.05, 0.95))
    rows = oracle.select_head(W, tau)
    pairs = [(i, j) for i in range(nq) for j in rows[i].tolist()]
    flat = W[0, 0].reshape(-1)
    k, best = _brute_force(flat, tau)
    assert len(pairs) == k
    assert abs(sum(W[0, 0, i, j] for i, j in pairs) - best) < 1e-12
    assert len(pairs) <= math.ceil(tau * nq * nkv)


def test_head_pool_empty_rows_and_full():
    W = np.zeros((1, 1, 3, 4))
    W[0, 0, 0, 1] = 0.7
    W[0, 0, 2, 3] = 0.2
    W[0, 0] += 0.1 / 12
    W /= W.sum()
    rows = oracle.select_head(W, 0.5)
    assert [r.tolist() for r in rows] == [[1], [], []]
    rows = oracle.select_head(W, 1.0)
    assert all(r.tolist() == [0, 1, 2, 3] for r in rows)


def test_csr_roundtrip():
    rows = [np.array([0, 3]), np.array([], np.int64), np.array([1, 2, 5])]
    rp, ci = oracle.to_csr(rows)
    assert rp.tolist() == [0, 2, 2, 5] and ci.tolist() == [0, 3, 1, 2, 5]
    assert [r.tolist() for r in oracle.csr_rows(rp, ci)] == [[0, 3], [], [1, 2, 5]]


def test_fixed_k_minimum():
    # fixed minimum k: every row keeps max(top-p count, k) blocks of the same ranking
    S = np.asarray([[[[0.7, 0.2, 0.05, 0.05], [0.3, 0.3, 0.2, 0.2]]]])
    rows, head_k = oracle.select_hybrid(S, 0.6, [8, 8], fixed_k=2)
    assert head_k.tolist() == [2]
    assert [r.tolist() for r in rows] == [[0, 1], [0, 1]]
    rows, _ = oracle.select_hybrid(S, 0.6, [8, 8], fixed_k=9)
    assert all(r.tolist() == [0, 1, 2, 3] for r in rows)
