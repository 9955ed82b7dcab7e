"""Pins for the oracle's per-token global threshold selection (VMoBA review: global selection
over a head's whole query-by-block matrix, Eq. 3-4, read per query token) and for attention over
token sets of any length, empty ones included (CPU only).

Pinned by brute force over every subset of tiny gate matrices, by its reduction to the
block-level head pool (select_head on score_head) when every query block has the same size and
its tokens share one query vector, by the limits tau = 1 and nesting in tau, and by dense
attention from torch for full sets."""
import itertools
import math

import numpy as np
import pytest
import torch

import oracle


def _norm(g):
    w = np.exp(g - g.max())
    return w / w.sum()


@pytest.mark.parametrize("seed", range(30))
def test_minimal_prefix_by_brute_force(seed):
    rng = np.random.default_rng(seed)
    N = int(rng.integers(1, 5))
    nkv = int(rng.integers(1, 17 // N + 1))
    G = rng.normal(scale=rng.uniform(0.3, 3.0), size=(1, 1, N, nkv))
    tau = float(rng.uniform(0.05, 0.95))
    sets = oracle.select_tokens_global(G, tau)
    chosen = [(i, int(J)) for i in range(N) for J in sets[i]]
    w = _norm(G[0, 0].reshape(-1))
    n = N * nkv
    best = None
    for k in range(1, n + 1):
        masses = [w[list(c)].sum() for c in itertools.combinations(range(n), k)
                  if w[list(c)].sum() >= tau]
        if masses:
            best = (k, max(masses))
            break
    assert len(chosen) == best[0]
    got = sum(w[i * nkv + J] for i, J in chosen)
    assert abs(got - best[1]) < 1e-12
    for i in range(N):
        assert np.all(np.diff(sets[i]) > 0)


def test_tau_one_keeps_every_pair_and_sets_nest():
    rng = np.random.default_rng(1)
    G = rng.normal(size=(2, 3, 20, 7))
    full = oracle.select_tokens_global(G, 1.0)
    assert all(np.array_equal(s, np.arange(7)) for s in full)
    prev = None
    for tau in (0.05, 0.2, 0.5, 0.9):
        cur = oracle.select_tokens_global(G, tau)
        if prev is not None:
            for a, b in zip(prev, cur):
                assert set(a.tolist()) <= set(b.tolist())
        prev = cur


def test_small_tau_leaves_empty_tokens():
    rng = np.random.default_rng(2)
    G = rng.normal(scale=2.0, size=(1, 1, 64, 9))
    sets = oracle.select_tokens_global(G, 0.25)
    assert any(len(s) == 0 for s in sets) and any(len(s) > 0 for s in sets)


def test_constant_shift_of_a_head_changes_nothing():
    rng = np.random.default_rng(3)
    G = rng.normal(size=(1, 2, 30, 6))
    a = oracle.select_tokens_global(G, 0.4)
    G2 = G.copy()
    G2[0, 1] += 5.0
    b = oracle.select_tokens_global(G2, 0.4)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))


@pytest.mark.parametrize("seed", range(5))
def test_reduces_to_the_block_level_head_pool(seed):
    # Equal-size query blocks whose tokens share one query vector: each block pair (I, J) of
    # the head pool (weight W_IJ from score_head, |I|-weighted) becomes |I| tied token pairs of
    # weight W_IJ / |I|. So the token selection is the head pool's, expanded to tokens, except
    # that the last pair of the head pool keeps only the m lowest-index tokens its cumulative
    # weight needs: m = ceil((tau - C) |I| / W) with C the weight of the pairs before it.
    rng = np.random.default_rng(10 + seed)
    grid, s = (2, 4, 4), 4                       # FLAT 4: 8 query blocks of 4 tokens
    N = 32
    qb = oracle.partition(grid, ("flat", s))
    kb = oracle.partition(grid, ("tile", (1, 2, 2)))
    nq, nkv = len(qb), len(kb)
    d = 16
    Q = np.empty((1, 1, N, d))
    for I, toks in enumerate(qb):
        Q[0, 0, toks] = rng.normal(size=d)
    K = rng.normal(size=(1, 1, N, d))
    hs = np.array([0.9])
    Kbar = oracle.pool(K, kb)
    G = oracle.token_gates(Q, Kbar, hs)
    tau = float(rng.uniform(0.2, 0.8))
    sets = oracle.select_tokens_global(G, tau)
    W = oracle.score_head(oracle.pool(Q, qb), Kbar, hs, oracle.block_sizes(qb))
    rows = oracle.select_head(W, tau)
    for I in range(nq):   # the union over a block's tokens is the block's row
        union = sorted(set(J for i in qb[I] for J in sets[i].tolist()))
        assert union == rows[I].tolist()
    # the head pool's ranking and its last pair
    flat = W[0, 0].reshape(-1)
    order = np.lexsort((np.arange(flat.size), -flat))
    k = sum(len(r) for r in rows)
    C = flat[order[:k - 1]].sum()
    Ilast, Jlast = divmod(int(order[k - 1]), nkv)
    m = math.ceil((tau - C) * s / flat[order[k - 1]])
    for I in range(nq):
        for J in rows[I].tolist():
            holders = [i for i in qb[I] if J in sets[i].tolist()]
            if (I, J) == (Ilast, Jlast):
                assert holders == list(qb[I][:m])
            else:
                assert holders == list(qb[I])


def test_token_set_attention_full_and_empty_sets():
    rng = np.random.default_rng(4)
    grid = (2, 4, 4)
    N, d = 32, 16
    kb = oracle.partition(grid, ("tile", (1, 2, 2)))
    Q, K, V = (rng.normal(size=(1, 2, N, d)) for _ in range(3))
    hs = np.array([0.3, 1.1])
    sets = [np.arange(len(kb))] * (2 * N)
    sets[5] = np.zeros(0, np.int64)
    O, L = oracle.attention_token_sets(Q, K, V, hs, sets, kb)
    for h in range(2):
        s = hs[h] * (torch.from_numpy(Q[0, h]) @ torch.from_numpy(K[0, h]).T)
        o = torch.softmax(s, -1) @ torch.from_numpy(V[0, h])
        lse = torch.logsumexp(s, -1)
        for i in range(N):
            if h == 0 and i == 5:
                assert np.all(O[0, 0, 5] == 0) and L[0, 0, 5] == -np.inf
                continue
            np.testing.assert_allclose(O[0, h, i], o[i].numpy(), atol=1e-12)
            assert abs(L[0, h, i] - float(lse[i])) < 1e-12
