"""Pins for the oracle's exact block masses, sparse attention and its backward (CPU only)."""
import numpy as np
import pytest
import torch

import oracle


def _problem(seed=0, grid=(4, 8, 8), part=("flat", 32), H=2, d=16):
    rng = np.random.default_rng(seed)
    N = grid[0] * grid[1] * grid[2]
    Q, K, V = (rng.standard_normal((1, H, N, d)) for _ in range(3))
    blocks = oracle.partition(grid, part)
    hs = rng.uniform(0.1, 0.5, size=H)
    return Q, K, V, blocks, hs


def _sdpa(q, k, v, scale, mask=None):
    t = [torch.from_numpy(np.ascontiguousarray(x))[None] for x in (q, k, v)]
    m = None if mask is None else torch.from_numpy(mask)[None]
    return torch.nn.functional.scaled_dot_product_attention(*t, attn_mask=m, scale=scale)[0].numpy()


# ----------------------------------------------------------------------------- exact mass (O3c)

def test_exact_mass_rows_sum_to_one_and_closed_form():
    Q, K, V, blocks, hs = _problem(1, grid=(3, 5, 7), part=("tile", (2, 2, 3)))
    M = oracle.exact_mass(Q, K, hs, blocks, blocks)
    np.testing.assert_allclose(M.sum(-1), 1.0, atol=1e-13)
    # q = 0 gives uniform attention, so each block's mass is its share of tokens
    M0 = oracle.exact_mass(np.zeros_like(Q), K, hs, blocks, blocks)
    sizes = oracle.block_sizes(blocks)
    np.testing.assert_allclose(M0, np.broadcast_to(sizes / sizes.sum(), M0.shape), atol=1e-14)


def test_exact_mass_equals_block_average_of_library_attention_matrix():
    Q, K, V, blocks, hs = _problem(2, grid=(2, 4, 6), part=("tile", (1, 3, 4)))
    M = oracle.exact_mass(Q, K, hs, blocks, blocks)
    for h in range(Q.shape[1]):
        P = torch.softmax(torch.from_numpy(Q[0, h] @ K[0, h].T) * hs[h], dim=-1).numpy()
        for i, bi in enumerate(blocks):
            for j, bj in enumerate(blocks):
                assert abs(M[0, h, i, j] - P[np.ix_(bi, bj)].sum(1).mean()) < 1e-13


def test_exact_mass_sampled_rows_leave_nan():
    Q, K, V, blocks, hs = _problem(3)
    M = oracle.exact_mass(Q, K, hs, blocks, blocks, rows=[(0, 1, 2)])
    assert np.isfinite(M[0, 1, 2]).all() and np.isnan(M[0, 0]).all()


# ----------------------------------------------------------------------------- attention (O5)

def test_p1_reproduces_dense_attention():
    Q, K, V, blocks, hs = _problem(4, grid=(3, 5, 7), part=("tile", (2, 3, 4)))
    nb = len(blocks)
    rows = [np.arange(nb) for _ in range(Q.shape[1] * nb)]
    rp, ci = oracle.to_csr(rows)
    O, LSE = oracle.attention_fwd(Q, K, V, hs, blocks, blocks, rp, ci)
    for h in range(Q.shape[1]):
        ref = _sdpa(Q[0, h], K[0, h], V[0, h], float(hs[h]))
        np.testing.assert_allclose(O[0, h], ref, rtol=1e-12, atol=1e-12)
        s = torch.from_numpy(Q[0, h] @ K[0, h].T) * hs[h]
        np.testing.assert_allclose(LSE[0, h], torch.logsumexp(s, -1).numpy(), atol=1e-12)


def test_sparse_equals_masked_dense_and_is_order_free():
    Q, K, V, blocks, hs = _problem(5, grid=(3, 5, 7), part=("tile", (2, 2, 3)))
    rng = np.random.default_rng(6)
    nb, H = len(blocks), Q.shape[1]
    rows = [np.sort(rng.choice(nb, size=int(rng.integers(1, nb)), replace=False))
            for _ in range(H * nb)]
    rp, ci = oracle.to_csr(rows)
    O, LSE = oracle.attention_fwd(Q, K, V, hs, blocks, blocks, rp, ci)
    for h in range(H):
        allowed = np.zeros((Q.shape[2], Q.shape[2]), bool)
        for i, bi in enumerate(blocks):
            for j in rows[h * nb + i]:
                allowed[np.ix_(bi, blocks[j])] = True
        ref = _sdpa(Q[0, h], K[0, h], V[0, h], float(hs[h]), mask=allowed)
        np.testing.assert_allclose(O[0, h], ref, rtol=1e-12, atol=1e-12)
    shuffled = [rng.permutation(r) for r in rows]
    rp2, ci2 = oracle.to_csr(shuffled)
    O2, LSE2 = oracle.attention_fwd(Q, K, V, hs, blocks, blocks, rp2, ci2)
    np.testing.assert_allclose(O2, O, atol=1e-13)
    np.testing.assert_allclose(LSE2, LSE, atol=1e-13)


def test_attention_special_cases():
    Q, K, V, blocks, hs = _problem(7)
    nb, H = len(blocks), Q.shape[1]
    rows = [np.array([(r * 3) % nb, (r * 5 + 1) % nb]) for r in range(H * nb)]
    rows = [np.unique(r) for r in rows]
    rp, ci = oracle.to_csr(rows)
    O, _ = oracle.attention_fwd(Q, K, np.full_like(V, -1.75), hs, blocks, blocks, rp, ci)
    np.testing.assert_allclose(O, -1.75, atol=1e-13)
    # one selected one-token block: the output is that token's value
    ones = oracle.partition((4, 8, 8), ("flat", 1))
    rows1 = [np.array([7]) for _ in range(H * nb)]
    rp1, ci1 = oracle.to_csr(rows1)
    O1, L1 = oracle.attention_fwd(Q, K, V, hs, blocks, ones, rp1, ci1)
    for h in range(H):
        np.testing.assert_allclose(O1[0, h], np.broadcast_to(V[0, h, 7], O1[0, h].shape),
                                   atol=1e-14)
    # empty rows: O = 0, LSE = -inf
    rows0 = [np.array([], np.int64) for _ in range(H * nb)]
    rp0, ci0 = oracle.to_csr(rows0)
    O0, L0 = oracle.attention_fwd(Q, K, V, hs, blocks, blocks, rp0, ci0)
    assert np.all(O0 == 0) and np.all(np.isneginf(L0))


# ----------------------------------------------------------------------------- backward (O6)

def _rows_for(H, nb, seed, allow_empty=True):
    rng = np.random.default_rng(seed)
    rows = []
    for r in range(H * nb):
        lo = 0 if allow_empty else 1
        k = int(rng.integers(lo, nb + 1))
        rows.append(np.sort(rng.choice(nb, size=k, replace=False)))
    return rows


def test_backward_matches_finite_differences():
    Q, K, V, blocks, hs = _problem(8, grid=(2, 2, 6), part=("tile", (1, 2, 3)), d=4)
    nb, H = len(blocks), Q.shape[1]
    rows = _rows_for(H, nb, 9)
    rp, ci = oracle.to_csr(rows)
    dO = np.random.default_rng(10).standard_normal(Q.shape)

    def loss(Q_, K_, V_):
        O, _ = oracle.attention_fwd(Q_, K_, V_, hs, blocks, blocks, rp, ci)
        return float((np.nan_to_num(O) * dO).sum())

    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, hs, blocks, blocks, rp, ci)
    eps = 1e-6
    rng = np.random.default_rng(11)
    for X, G, which in ((Q, dQ, 0), (K, dK, 1), (V, dV, 2)):
        for _ in range(12):
            idx = tuple(int(rng.integers(0, s)) for s in X.shape)
            Xp, Xm = X.copy(), X.copy()
            Xp[idx] += eps
            Xm[idx] -= eps
            args_p = [Q, K, V]
            args_m = [Q, K, V]
            args_p[which], args_m[which] = Xp, Xm
            fd = (loss(*args_p) - loss(*args_m)) / (2 * eps)
            assert abs(fd - G[idx]) < 1e-6 * max(1.0, abs(fd)), (which, idx, fd, G[idx])


def test_backward_matches_autograd_of_masked_dense():
    Q, K, V, blocks, hs = _problem(12, grid=(2, 4, 8), part=("tile", (1, 2, 4)), d=8)
    nb, H = len(blocks), Q.shape[1]
    rows = _rows_for(H, nb, 13, allow_empty=False)
    rp, ci = oracle.to_csr(rows)
    dO = np.random.default_rng(14).standard_normal(Q.shape)
    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, hs, blocks, blocks, rp, ci)
    for h in range(H):
        allowed = np.zeros((Q.shape[2], Q.shape[2]), bool)
        for i, bi in enumerate(blocks):
            for j in rows[h * nb + i]:
                allowed[np.ix_(bi, blocks[j])] = True
        q, k, v = (torch.tensor(x[0, h], requires_grad=True) for x in (Q, K, V))
        o = torch.nn.functional.scaled_dot_product_attention(
            q[None], k[None], v[None], attn_mask=torch.from_numpy(allowed)[None],
            scale=float(hs[h]))[0]
        (o * torch.from_numpy(dO[0, h])).sum().backward()
        np.testing.assert_allclose(dQ[0, h], q.grad.numpy(), rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(dK[0, h], k.grad.numpy(), rtol=1e-10, atol=1e-11)
        np.testing.assert_allclose(dV[0, h], v.grad.numpy(), rtol=1e-10, atol=1e-11)


def test_backward_empty_rows_contribute_nothing():
    Q, K, V, blocks, hs = _problem(15, d=8)
    nb, H = len(blocks), Q.shape[1]
    rows = [np.array([], np.int64) for _ in range(H * nb)]
    rows[3] = np.array([2, 5])
    rp, ci = oracle.to_csr(rows)
    dO = np.random.default_rng(16).standard_normal(Q.shape)
    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, hs, blocks, blocks, rp, ci)
    h, i = divmod(3, nb)
    others = np.setdiff1d(np.arange(Q.shape[2]), blocks[i])
    assert np.all(dQ[0, 1 - h] == 0) and np.all(dQ[0, h][others] == 0)
    assert np.any(dQ[0, h][blocks[i]] != 0)
    touched = np.concatenate([blocks[2], blocks[5]])
    untouched = np.setdiff1d(np.arange(Q.shape[2]), touched)
    assert np.all(dK[0, h][untouched] == 0) and np.all(dV[0, h][untouched] == 0)
    assert np.all(dK[0, 1 - h] == 0) and np.all(dV[0, 1 - h] == 0)
    assert np.any(dK[0, h][touched] != 0)
