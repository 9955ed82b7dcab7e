"""GPU parity of the per-token head-global threshold selection (bsa_select_tokens_global) and of
attention over per-token block bitmaps (bsa_attn_fwd_token_bits) against the oracle's
select_tokens_global / attention_token_sets.

Selections: per head, the GPU's (token, block) pair set equals the oracle's, or is another valid
answer at a near-tie, judged on the oracle's fp64 weights W (one softmax over the head's N x nkv
gates): (A) it is a top set of W up to a relative 2e-4 (the GPU's gates carry Kbar to 2^-17 and
sum in fp32, so exp(g - max) differs by about 1e-4 relative at |g| ~ 5), (B) it reaches
tau - 5e-5 and (C) dropping its smallest member falls below tau + 5e-5. Ties in W (identical
tokens, constant queries) must match exactly. Attention: the oracle's own sets are fed to both
sides; O within max-abs 1e-2 and LSE within 1e-3; tokens with no block give O = 0 and
LSE = -inf."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from gen import CONFIGS, make_inputs
from helpers import dev_to_f64, log, to_dev, to_f64

pytestmark = pytest.mark.gpu

REL_TIE, SUM_TOL = 2e-4, 5e-5


def _layer(w, x):
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    return BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart, dtype=w.dtype,
                                head_scale=x["head_scale"])


def _bits_to_sets(bits, nkv):
    """[B, H, N, nw] int32 words -> list of ascending block arrays in (b, h, i) order."""
    b = np.ascontiguousarray(bits.reshape(-1, bits.shape[-1])).view(np.uint32)
    flags = np.unpackbits(b.view(np.uint8), axis=1, bitorder="little")[:, :nkv]
    return [np.flatnonzero(f).astype(np.int64) for f in flags]


def _sets_to_bits(sets, B, H, N, nkv):
    nw = (nkv + 31) // 32
    bits = np.zeros((B * H * N, nw), np.uint32)
    for r, s in enumerate(sets):
        for j in np.asarray(s, np.int64):
            bits[r, j // 32] |= np.uint32(1) << np.uint32(j % 32)
    return bits.view(np.int32).reshape(B, H, N, nw)


def _weights(G_head):
    g = np.asarray(G_head, np.float64).reshape(-1)
    w = np.exp(g - g.max())
    return w / w.sum()


def _check_head(gpu_sets, ref_sets, G_head, tau, nkv, exact_ties=False):
    N = len(ref_sets)
    gi = np.asarray([i * nkv + j for i in range(N) for j in gpu_sets[i]], np.int64)
    oi = np.asarray([i * nkv + j for i in range(N) for j in ref_sets[i]], np.int64)
    if np.array_equal(np.sort(gi), np.sort(oi)):
        return True, 0
    if exact_ties:
        return False, len(np.setxor1d(gi, oi))
    W = _weights(G_head)
    inside = W[gi]
    mask = np.ones(W.size, bool)
    mask[gi] = False
    out_max = W[mask].max() if mask.any() else 0.0
    A = inside.min() >= out_max * (1 - REL_TIE)
    B_ = inside.sum() >= tau - SUM_TOL
    C = inside.sum() - inside.min() < tau + SUM_TOL
    return bool(A and B_ and C), len(np.setxor1d(gi, oi))


def _run_select(w, x, tau, q_override=None):
    import torch
    layer = _layer(w, x)
    q = to_dev(x["q"] if q_override is None else q_override)
    layer.pool(q, to_dev(x["k"]))
    bits = layer.select_tokens_global(q, tau)
    torch.cuda.synchronize()
    rp, ci = layer.csr_host()
    return layer, q, bits.cpu().numpy(), rp, ci


def _oracle_gates(w, x, q_bits=None):
    Q = to_f64(x["q"] if q_bits is None else q_bits)
    kb = oracle.partition(w.grid, w.kvpart)
    Kbar = oracle.pool(to_f64(x["k"]), kb)
    return oracle.token_gates(Q, Kbar, x["head_scale"].astype(np.float64)), kb


@pytest.mark.parametrize("case,tau", [("small", 0.25), ("small", 0.05), ("small", 0.9),
                                      ("ragged", 0.25), ("batch2", 0.25), ("temporal", 0.5),
                                      ("small", 1.0)])
def test_selection_against_oracle(case, tau):
    w = {"small": replace(CONFIGS[2], grid=(5, 8, 16), H=2),
         "ragged": replace(CONFIGS[2], grid=(5, 7, 13), H=3),
         "batch2": replace(CONFIGS[2], B=2, grid=(6, 9, 20), H=2),
         "temporal": replace(CONFIGS[2], grid=(6, 9, 20), H=2, kvpart=("tile", (2, 9, 20)))}[case]
    x = make_inputs(w)
    layer, q, bits, rp, ci = _run_select(w, x, tau)
    G, kb = _oracle_gates(w, x)
    nkv, N = len(kb), w.N
    ref = oracle.select_tokens_global(G, tau)
    gpu = _bits_to_sets(bits, nkv)
    for b in range(w.B):
        for h in range(w.H):
            r0 = (b * w.H + h) * N
            ok, ndiff = _check_head(gpu[r0:r0 + N], ref[r0:r0 + N], G[b, h], tau, nkv)
            log(f"{case} tau={tau} head ({b},{h}): pairs {sum(len(s) for s in gpu[r0:r0+N])}, "
                f"differing {ndiff}, empty tokens {sum(len(s) == 0 for s in gpu[r0:r0+N])}")
            assert ok
    # the union CSR row of each query block is the OR of its tokens' sets
    qb = oracle.partition(w.grid, w.qpart)
    rows = oracle.csr_rows(rp, ci)
    for r, row in enumerate(rows):
        bh, I = divmod(r, len(qb))
        union = sorted(set(j for t in qb[I] for j in gpu[bh * N + t].tolist()))
        assert row.tolist() == union
    if tau >= 1.0:
        assert all(len(s) == nkv for s in gpu)


def test_exact_ties_constant_and_duplicated_queries():
    # All gates equal (q = 0): every pair ties, the prefix takes the lowest pair indices. Then
    # queries duplicated in pairs: equal weights across tokens, ties broken by pair index.
    w = replace(CONFIGS[2], grid=(4, 8, 8), H=2)
    x = make_inputs(w)
    zero = np.zeros_like(x["q"])
    for qb_, tau in ((zero, 0.3), (zero, 0.77)):
        _, _, bits, _, _ = _run_select(w, x, tau, q_override=qb_)
        G, kb = _oracle_gates(w, x, qb_)
        ref = oracle.select_tokens_global(G, tau)
        gpu = _bits_to_sets(bits, len(kb))
        for h in range(w.H):
            r0 = h * w.N
            ok, nd = _check_head(gpu[r0:r0 + w.N], ref[r0:r0 + w.N], G[0, h], tau, len(kb),
                                 exact_ties=True)
            assert ok, f"constant queries, tau {tau}: {nd} pairs differ"
    dup = x["q"].copy()
    dup[:, :, 1::2] = dup[:, :, 0::2]
    _, _, bits, _, _ = _run_select(w, x, 0.4, q_override=dup)
    G, kb = _oracle_gates(w, x, dup)
    ref = oracle.select_tokens_global(G, 0.4)
    gpu = _bits_to_sets(bits, len(kb))
    for h in range(w.H):
        r0 = h * w.N
        ok, nd = _check_head(gpu[r0:r0 + w.N], ref[r0:r0 + w.N], G[0, h], 0.4, len(kb))
        assert ok, f"duplicated queries: {nd} pairs differ"


@pytest.mark.parametrize("case", ["small", "ragged_batch2", "wide"])
def test_token_bits_attention_on_oracle_sets(case):
    import torch
    # wide: 1024 kv blocks of 4 tokens, above the 768 blocks whose bitmap rows fit two
    # workgroups per CU (the kernel for wider rows)
    w = {"small": replace(CONFIGS[2], grid=(5, 8, 16), H=2),
         "ragged_batch2": replace(CONFIGS[2], B=2, grid=(5, 7, 13), H=2),
         "wide": replace(CONFIGS[2], grid=(8, 16, 32), H=2, kvpart=("tile", (1, 2, 2)))}[case]
    x = make_inputs(w)
    G, kb = _oracle_gates(w, x)
    sets = oracle.select_tokens_global(G, 0.25)
    sets[3] = np.arange(len(kb))            # one token with every block
    sets[5] = np.zeros(0, np.int64)         # and one with none
    layer = _layer(w, x)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    bits = torch.from_numpy(_sets_to_bits(sets, w.B, w.H, w.N, len(kb))).cuda()
    # the union CSR of the oracle's sets, built on the host
    qb = oracle.partition(w.grid, w.qpart)
    unions = [np.asarray(sorted(set(j for t in qb[I] for j in sets[bh * w.N + t].tolist())),
                         np.int64) for bh in range(w.B * w.H) for I in range(len(qb))]
    rp, ci = oracle.to_csr(unions)
    layer.row_ptr.copy_(torch.from_numpy(rp))
    layer.col_idx[:len(ci)].copy_(torch.from_numpy(ci))
    O, L = layer.attention_token_bits(q, k, v, bits)
    O2, _ = layer.attention_token_bits(q, k, v, bits, with_lse=False)
    torch.cuda.synchronize()
    O_ref, L_ref = oracle.attention_token_sets(*(to_f64(x[n]) for n in ("q", "k", "v")),
                                               x["head_scale"].astype(np.float64), sets, kb)
    Og, Lg, O2g = dev_to_f64(O), dev_to_f64(L), dev_to_f64(O2)
    err_o, err_o2 = np.abs(Og - O_ref).max(), np.abs(O2g - O_ref).max()
    fin = np.isfinite(L_ref)
    err_l = np.abs(Lg[fin] - L_ref[fin]).max()
    empty = sum(len(s) == 0 for s in sets)
    log(f"{case}: O max-abs {err_o:.2e} (output-only {err_o2:.2e}), LSE {err_l:.2e}, "
        f"empty tokens {empty}")
    assert err_o <= 1e-2 and err_o2 <= 1e-2 and err_l <= 1e-3
    assert np.array_equal(np.isfinite(Lg), fin) and np.all(Lg[~fin] == -np.inf)
    assert np.all(Og[~fin] == 0)


def test_full_480p_one_head():
    import torch
    w = CONFIGS[2]
    x = make_inputs(w)
    layer, q, bits, rp, ci = _run_select(w, x, 0.25)
    h = 7
    kb = oracle.partition(w.grid, w.kvpart)
    nkv, N = len(kb), w.N
    Q = to_f64(x["q"])[:, h:h + 1]
    Kbar = oracle.pool(to_f64(x["k"])[:, h:h + 1], kb)
    G = oracle.token_gates(Q, Kbar, x["head_scale"][h:h + 1].astype(np.float64))
    ref = oracle.select_tokens_global(G, 0.25)
    gpu = _bits_to_sets(bits[:, h:h + 1], nkv)
    ok, nd = _check_head(gpu, ref, G[0, 0], 0.25, nkv)
    empty = sum(len(s) == 0 for s in gpu)
    log(f"480p head {h}: pairs {sum(len(s) for s in gpu)} of {N * nkv}, differing {nd}, "
        f"empty tokens {empty} of {N}")
    assert ok
    # attention on the GPU's own selection; O compared on sampled tokens whose sets equal the
    # oracle's (the oracle attends over its own sets), empty tokens among them
    O, L = layer.attention_token_bits(q, to_dev(x["k"]), to_dev(x["v"]),
                                      torch.from_numpy(bits).cuda())
    torch.cuda.synchronize()
    same = [i for i in range(N) if np.array_equal(gpu[i], ref[i])]
    rng = np.random.default_rng(9)
    pick = sorted(rng.choice(same, size=min(192, len(same)), replace=False).tolist())
    empties = [i for i in same if len(ref[i]) == 0][:16]
    toks = sorted(set(pick + empties))
    sets_all = [np.zeros(0, np.int64)] * (w.H * N)
    sets_all[h * N:(h + 1) * N] = ref
    O_ref, L_ref = oracle.attention_token_sets(to_f64(x["q"]), to_f64(x["k"]), to_f64(x["v"]),
                                               x["head_scale"].astype(np.float64), sets_all, kb,
                                               tokens=[(0, h, i) for i in toks])
    Og, Lg = dev_to_f64(O)[0, h, toks], dev_to_f64(L)[0, h, toks]
    Or, Lr = O_ref[0, h, toks], L_ref[0, h, toks]
    fin = np.isfinite(Lr)
    err_o = np.abs(Og - Or).max()
    log(f"  O max-abs {err_o:.2e} over {len(toks)} tokens ({int((~fin).sum())} empty)")
    assert err_o <= 1e-2
    assert np.abs(Lg[fin] - Lr[fin]).max() <= 1e-3
    assert np.all(Lg[~fin] == -np.inf) and np.all(Og[~fin] == 0)


def test_rejects_bad_parameters():
    import block_sparse_attention_bsa_amd as bsa
    w = replace(CONFIGS[2], grid=(4, 8, 8), H=2)
    x = make_inputs(w)
    layer = _layer(w, x)
    q = to_dev(x["q"])
    for tau in (0.0, -1.0, 1.5, float("nan")):
        with pytest.raises(bsa.BsaError):
            layer.select_tokens_global(q, tau)
