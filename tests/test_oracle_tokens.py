"""Pins for the oracle's per-token Local + TopK (VMoBA: every query token scores the block means):
the gates against a direct loop, brute force over the k best others, and attention that reduces
to dense softmax attention (all blocks) or to the block-level oracle (shared sets) (CPU only)."""
import itertools

import numpy as np
import pytest

import oracle


def _setup(seed, grid=(2, 4, 4), part=("tile", (1, 2, 4)), H=2, d=8):
    rng = np.random.default_rng(seed)
    N = int(np.prod(grid))
    Q, K, V = (rng.standard_normal((1, H, N, d)) for _ in range(3))
    hs = rng.uniform(0.2, 0.6, size=H)
    kb = oracle.partition(grid, part)
    return Q, K, V, hs, kb


def test_gates_by_direct_loop():
    Q, K, _, hs, kb = _setup(0)
    Kbar = oracle.pool(K, kb)
    G = oracle.token_gates(Q, Kbar, hs)
    for h in range(2):
        for i in (0, 5, 31):
            for j in range(len(kb)):
                ref = hs[h] * sum(Q[0, h, i, c] * K[0, h, kb[j], c].mean() for c in range(8))
                assert G[0, h, i, j] == pytest.approx(ref, rel=1e-12, abs=1e-14)


@pytest.mark.parametrize("seed", range(6))
def test_selection_is_own_block_plus_best_k_by_brute_force(seed):
    Q, K, _, hs, kb = _setup(10 + seed)
    G = oracle.token_gates(Q, oracle.pool(K, kb), hs)
    k = 1 + seed % 3
    sel = oracle.select_tokens(G, k, kb)
    own = {int(t): j for j, b in enumerate(kb) for t in b}
    for h in range(2):
        for i in range(G.shape[2]):
            s = set(sel[0, h, i].tolist())
            assert own[i] in s and len(s) == 1 + k
            others = [j for j in range(len(kb)) if j != own[i]]
            best = max(itertools.combinations(others, k), key=lambda c: G[0, h, i, list(c)].sum())
            assert s - {own[i]} == set(best)


def test_all_blocks_is_dense_attention():
    Q, K, V, hs, kb = _setup(3)
    G = oracle.token_gates(Q, oracle.pool(K, kb), hs)
    sel = oracle.select_tokens(G, 99, kb)
    assert sel.shape[-1] == len(kb)
    O, L = oracle.attention_tokens(Q, K, V, hs, sel, kb)
    for h in range(2):
        s = hs[h] * Q[0, h] @ K[0, h].T
        w = np.exp(s - s.max(1, keepdims=True))
        np.testing.assert_allclose(O[0, h], (w / w.sum(1, keepdims=True)) @ V[0, h], atol=1e-12)
        np.testing.assert_allclose(L[0, h], np.log(np.exp(s).sum(1)), atol=1e-12)


def test_shared_sets_match_the_block_level_oracle():
    # every token of a query block given the same set: per-token attention = block attention
    Q, K, V, hs, kb = _setup(4)
    qb = oracle.partition((2, 4, 4), ("tile", (1, 4, 4)))
    rng = np.random.default_rng(9)
    rows = [np.sort(rng.choice(len(kb), size=3, replace=False)) for _ in range(2 * len(qb))]
    sel = np.empty((1, 2, 32, 3), np.int64)
    for h in range(2):
        for I, blk in enumerate(qb):
            sel[0, h, blk] = rows[h * len(qb) + I]
    O1, L1 = oracle.attention_tokens(Q, K, V, hs, sel, kb)
    rp, ci = oracle.to_csr(rows)
    O2, L2 = oracle.attention_fwd(Q, K, V, hs, qb, kb, rp, ci)
    np.testing.assert_allclose(O1, O2, atol=1e-12)
    np.testing.assert_allclose(L1, L2, atol=1e-12)
