"""Pins for the oracle's partition, pooling and scoring (CPU only)."""
import json
import os

import numpy as np
import pytest
import torch

import oracle
from gen import CONFIGS

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _load(name):
    with open(os.path.join(GOLD, name)) as f:
        return json.load(f)


# ----------------------------------------------------------------------------- partition (O1)

def test_partition_tiny_golden():
    g = _load("partition_tiny.json")
    blocks = oracle.partition(g["grid"], ("tile", g["tile"]))
    assert [b.tolist() for b in blocks] == g["blocks"]
    flat = oracle.partition(g["flat_grid"], ("flat", g["flat"]))
    assert [b.tolist() for b in flat] == g["flat_blocks"]


def test_block_counts_golden():
    for case in _load("block_counts.json")["cases"]:
        blocks = oracle.partition(case["grid"], ("tile", case["tile"]))
        assert len(blocks) == case["nblk"], case


@pytest.mark.parametrize("grid,tile", [((21, 30, 52), (4, 4, 8)), ((5, 7, 9), (2, 3, 4)),
                                       ((21, 45, 80), (3, 45, 80)), ((3, 4, 5), (3, 4, 5)),
                                       ((4, 8, 8), (1, 1, 1))])
def test_partition_covers_once_and_sizes(grid, tile):
    T, Hg, Wg = grid
    blocks = oracle.partition(grid, ("tile", tile))
    allidx = np.concatenate(blocks)
    assert np.array_equal(np.sort(allidx), np.arange(T * Hg * Wg))
    nbh, nbw = -(-Hg // tile[1]), -(-Wg // tile[2])
    for j, b in enumerate(blocks):
        a, rem = divmod(j, nbh * nbw)
        bb, c = divmod(rem, nbw)
        ext = [min(tile[0], T - a * tile[0]), min(tile[1], Hg - bb * tile[1]),
               min(tile[2], Wg - c * tile[2])]
        assert len(b) == ext[0] * ext[1] * ext[2]
        assert np.all(np.diff(b) > 0)


def test_flat32_equals_tile_148_on_tiny_grid():
    a = oracle.partition((4, 8, 8), ("flat", 32))
    b = oracle.partition((4, 8, 8), ("tile", (1, 4, 8)))
    assert [x.tolist() for x in a] == [x.tolist() for x in b]


def test_workload_geometry():
    w2, w4, w5 = CONFIGS[2], CONFIGS[4], CONFIGS[5]
    b2 = oracle.block_sizes(oracle.partition(w2.grid, w2.qpart))
    assert len(b2) == 336 and (b2 == 128).sum() == 210 and b2.min() == 8
    b4 = oracle.block_sizes(oracle.partition(w4.grid, w4.qpart))
    assert len(b4) == 1080 and (b4 == 128).sum() == 880
    b5 = oracle.block_sizes(oracle.partition(w5.grid, w5.qpart))
    assert len(b5) == 720 and (b5 == 128).sum() == 550
    assert [len(oracle.partition(w5.grid, p)) for p in w5.kv_cycle] == [7, 48, 60]


# ----------------------------------------------------------------------------- pooling (O2)

def test_pool_preserves_totals_and_constants():
    rng = np.random.default_rng(0)
    X = rng.standard_normal((1, 2, 5 * 7 * 9, 6))
    blocks = oracle.partition((5, 7, 9), ("tile", (2, 3, 4)))
    Xb = oracle.pool(X, blocks)
    sizes = oracle.block_sizes(blocks)
    tot = (Xb * sizes[None, None, :, None]).sum(axis=2)
    np.testing.assert_allclose(tot, X.sum(axis=2), rtol=1e-12, atol=1e-12)
    C = np.full_like(X, 3.25)
    np.testing.assert_allclose(oracle.pool(C, blocks), 3.25, rtol=0, atol=1e-14)
    ones = oracle.partition((5, 7, 9), ("tile", (1, 1, 1)))
    np.testing.assert_array_equal(oracle.pool(X, ones), X)


def test_pool_matches_torch_avg_pool3d_on_divisible_grid():
    # A library routine: 3D average pooling over non-overlapping tiles of a divisible grid.
    rng = np.random.default_rng(1)
    T, Hg, Wg, d = 4, 6, 8, 3
    X = rng.standard_normal((1, 1, T * Hg * Wg, d))
    blocks = oracle.partition((T, Hg, Wg), ("tile", (2, 3, 4)))
    Xb = oracle.pool(X, blocks)[0, 0]
    grid = torch.from_numpy(X[0, 0].T.reshape(1, d, T, Hg, Wg).copy())
    ref = torch.nn.functional.avg_pool3d(grid, (2, 3, 4)).reshape(d, -1).T.numpy()
    np.testing.assert_allclose(Xb, ref, rtol=1e-12, atol=1e-12)


# ----------------------------------------------------------------------------- scores (O3a/b)

def _means(seed, H=2, nq=5, nkv=7, d=8):
    rng = np.random.default_rng(seed)
    return rng.standard_normal((1, H, nq, d)), rng.standard_normal((1, H, nkv, d))


def test_score_row_normalised_and_shift_invariant():
    Qb, Kb = _means(2)
    hs = np.array([0.3, 0.7])
    S = oracle.score_row(Qb, Kb, hs)
    np.testing.assert_allclose(S.sum(-1), 1.0, atol=1e-13)
    shift = np.random.default_rng(3).standard_normal(8)
    S2 = oracle.score_row(Qb, Kb + shift, hs)
    np.testing.assert_allclose(S2, S, atol=1e-13)
    S3 = oracle.score_row(Qb, np.repeat(Kb[:, :, :1], 7, axis=2), hs)
    np.testing.assert_allclose(S3, 1.0 / 7, atol=1e-14)


def test_score_row_equals_sdpa_weights_for_one_token_blocks():
    # With one token per block the block means are the tokens themselves, so the row scores are
    # attention probabilities: S @ V must equal the library's scaled dot-product attention.
    rng = np.random.default_rng(4)
    Q, K, V = (rng.standard_normal((1, 2, 9, 8)) for _ in range(3))
    hs = np.array([0.35, 1.2])
    ones = oracle.partition((1, 3, 3), ("tile", (1, 1, 1)))
    S = oracle.score_row(oracle.pool(Q, ones), oracle.pool(K, ones), hs)
    for h in range(2):
        ref = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q[:, h]), torch.from_numpy(K[:, h]), torch.from_numpy(V[:, h]),
            scale=float(hs[h])).numpy()
        np.testing.assert_allclose(S[0, h] @ V[0, h], ref[0], rtol=1e-12, atol=1e-12)


def test_score_head_weights():
    Qb, Kb = _means(5)
    hs = np.array([0.5, 0.9])
    sizes = np.array([128, 64, 32, 128, 8])
    W = oracle.score_head(Qb, Kb, hs, sizes)
    np.testing.assert_allclose(W.sum(axis=(2, 3)), 1.0, atol=1e-13)
    # equal query-block sizes: a softmax over the flattened matrix (library routine)
    W_eq = oracle.score_head(Qb, Kb, hs, np.full(5, 16))
    for h in range(2):
        L = torch.from_numpy(Qb[0, h] @ Kb[0, h].T * hs[h]).reshape(-1)
        np.testing.assert_allclose(W_eq[0, h].reshape(-1), torch.softmax(L, 0).numpy(),
                                   atol=1e-14)
    # two query blocks with identical means: row totals in the ratio of their sizes
    Qs = np.repeat(Qb[:, :, :1], 5, axis=2)
    Wi = oracle.score_head(Qs, Kb, hs, sizes)
    tot = Wi.sum(axis=3)[0, 0]
    np.testing.assert_allclose(tot / tot[0], sizes / sizes[0], rtol=1e-12)
    # a single query block reduces to the row softmax
    W1 = oracle.score_head(Qb[:, :, :1], Kb, hs, sizes[:1])
    np.testing.assert_allclose(W1, oracle.score_row(Qb[:, :, :1], Kb, hs), atol=1e-14)
