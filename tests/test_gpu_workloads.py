"""Full-size GPU parity for the HunyuanVideo-720p hybrid selection workload and the Wan2.1-14B
training workload (head-global selection, cycled 1D/2D/3D kv partitions, forward + backward).

The oracle runs the whole selection at full size (pooling, scores, selection in fp64) and checks
O and the gradients on sampled query blocks (and, for dK/dV, on the kv blocks with the fewest,
the median and the most selecting query blocks of sampled heads, whose gradient the oracle sums
query block by query block).
Bars: selections bit-exact except near-ties (within 1e-5 of the threshold), O max-abs 1e-2,
gradients max-abs 2e-2 * max(1, max|ref|)."""
import functools

import numpy as np
import pytest

import oracle
from gen import CONFIGS, kv_partition_for_layer, make_inputs
from helpers import TIE_EPS_CUM, TIE_EPS_SCORE, check_csr_rows, dev_to_f64, log, to_dev, to_f64

pytestmark = pytest.mark.gpu


@functools.lru_cache(maxsize=1)
def _inputs(cid):
    w = CONFIGS[cid]
    tensors = ("q", "k", "v", "do") if w.backward else ("q", "k", "v")
    log(f"generating inputs for {w.name}")
    return make_inputs(w, tensors=tensors)


@functools.lru_cache(maxsize=1)
def _row_scores(cid):
    """The oracle's row-normalised block scores of the workload's inputs (fp64)."""
    w = CONFIGS[cid]
    x = _inputs(cid)
    Q, K = to_f64(x["q"]), to_f64(x["k"])
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    return oracle.score_row(oracle.pool(Q, qb), oracle.pool(K, kb),
                            x["head_scale"].astype(np.float64))


def _layer(w, kvpart, x):
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    return BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, kvpart, dtype=w.dtype,
                                head_scale=x["head_scale"])


def test_hybrid_min_k_full_size():
    import torch
    w = CONFIGS[4]
    x = _inputs(4)
    layer = _layer(w, w.kvpart, x)
    q, k, v = (to_dev(x[n]) for n in ("q", "k", "v"))
    O, L = layer.forward(q, k, v, w.p, min_k_mode=2)
    torch.cuda.synchronize()
    rp, ci = layer.csr_host()
    rows_gpu = oracle.csr_rows(rp, ci)
    head_k = layer.head_k.cpu().numpy()
    Q, K, V = (to_f64(x[n]) for n in ("q", "k", "v"))
    hs = x["head_scale"].astype(np.float64)
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    qs = oracle.block_sizes(qb)
    S = _row_scores(4)
    rows_ref, k_ref = oracle.select_hybrid(S, w.p, qs)
    log(f"head k: gpu {head_k.tolist()}")
    log(f"        ref {k_ref.tolist()}")
    assert np.array_equal(head_k, k_ref)
    nq = len(qb)
    flat = S.reshape(-1, S.shape[-1])
    same = [np.array_equal(a, b) for a, b in zip(rows_gpu, rows_ref)]
    bad = []
    for r, ok in enumerate(same):
        if ok:
            continue
        g, o = rows_gpu[r], rows_ref[r]
        kh = int(k_ref[r // nq])
        if len(o) > kh:  # a top-p row: the tie-tolerant checker decides
            if check_csr_rows([g], [o], flat[r:r + 1], w.p)[2]:
                bad.append(r)
        else:  # a topped-up row: same size, and a top set of the scores up to 1e-6
            s = flat[r]
            m = np.ones(len(s), bool)
            m[g] = False
            if len(g) != len(o) or s[g].min() < s[m].max() - TIE_EPS_SCORE:
                bad.append(r)
    log(f"rows exact {sum(same)}/{len(same)}, bad {len(bad)}")
    assert not bad
    dens = oracle.density(rows_gpu, qs, oracle.block_sizes(kb), w.H)
    rng = np.random.default_rng(4)
    cand = [r for r in range(len(same)) if same[r]]
    pick = sorted(rng.choice(cand, size=16, replace=False).tolist())
    rp_ref, ci_ref = oracle.to_csr(rows_ref)
    sample = [(0, r // nq, r % nq) for r in pick]
    O_ref, _ = oracle.attention_fwd(Q, K, V, hs, qb, kb, rp_ref, ci_ref, rows=sample)
    Og = dev_to_f64(O)
    worst = max(float(np.abs(Og[0, h, qb[i]] - O_ref[0, h, qb[i]]).max()) for _, h, i in sample)
    log(f"density {dens:.3f}; O max-abs {worst:.2e} over {len(sample)} q-blocks")
    assert worst <= 1e-2


def test_entropy_routed_full_size_720p():
    """EG-Sparse's entropy-routed selection on the 720p hybrid workload's inputs, groups of four
    heads, theta between two of the 24 head entropies near their median (the heads' entropies lie
    within 1e-3 of each other here, so theta keeps 1e-5 from both neighbours; the GPU's entropies
    are within 1e-7 of the oracle's)."""
    from test_gpu_select_eg import _run as eg_run
    eg_run(CONFIGS[4], 4, x=_inputs(4), S_ref=_row_scores(4), margin=1e-5)


def test_token_topk_full_size_720p():
    """Per-token Local + TopK (k = 18, the widest list) on the 720p inputs: every token's list of
    the first and last head against the oracle's, O and LSE on 256 sampled tokens of each."""
    from test_gpu_tokens import _run as tok_run
    tok_run(CONFIGS[4], 18, heads=[0, 23], o_sample=256, x=_inputs(4))


def _head_check(W, rows_gpu, rows_ref, nq, tau):
    """Per head: the GPU's pair set equals the oracle's, or is a valid near-tie answer."""
    H = W.shape[1]
    for h in range(H):
        g = sorted((i, j) for i in range(nq) for j in rows_gpu[h * nq + i].tolist())
        o = sorted((i, j) for i in range(nq) for j in rows_ref[h * nq + i].tolist())
        if g == o:
            continue
        flat = W[0, h].reshape(-1)
        nkv = W.shape[3]
        gi = np.asarray([i * nkv + j for i, j in g])
        m = np.ones(len(flat), bool)
        m[gi] = False
        tot = flat[gi].sum()
        okA = flat[gi].min() >= flat[m].max() - TIE_EPS_SCORE
        okB = tot >= tau - TIE_EPS_CUM
        okC = tot - flat[gi].min() < tau + TIE_EPS_CUM
        assert okA and okB and okC, f"head {h}: pair set differs beyond a near-tie"


@pytest.mark.parametrize("layer_idx", [0, 1, 2])
def test_training_step_full_size(layer_idx):
    import torch
    w = CONFIGS[5]
    kvpart = kv_partition_for_layer(w, layer_idx)
    x = _inputs(5)
    layer = _layer(w, kvpart, x)
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    O, L = layer.forward(q, k, v, w.p, mode="head")
    torch.cuda.synchronize()
    rp, ci = layer.csr_host()
    rows_gpu = oracle.csr_rows(rp, ci)
    Q, K, V, dO = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    hs = x["head_scale"].astype(np.float64)
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, kvpart)
    qs, ks = oracle.block_sizes(qb), oracle.block_sizes(kb)
    W = oracle.score_head(oracle.pool(Q, qb), oracle.pool(K, kb), hs, qs)
    rows_ref = oracle.select_head(W, w.p)
    nq = len(qb)
    _head_check(W, rows_gpu, rows_ref, nq, w.p)
    empty = sum(len(r) == 0 for r in rows_gpu)
    dens = oracle.density(rows_gpu, qs, ks, w.H)
    log(f"kv {kvpart}: {len(kb)} blocks, density {dens:.4f}, empty rows {empty}/{len(rows_gpu)}")
    # backward on the GPU's own selection (validated above); the oracle differentiates the same
    dq, dk, dv = layer.backward(q, k, v, O, do, L)
    torch.cuda.synchronize()
    rng = np.random.default_rng(10 + layer_idx)
    nonempty = [r for r in range(len(rows_gpu)) if len(rows_gpu[r])]
    pick = sorted(rng.choice(nonempty, size=min(12, len(nonempty)), replace=False).tolist())
    Og, dQg, dKg, dVg = (dev_to_f64(t) for t in (O, dq, dk, dv))
    worst_o = worst_q = 0.0
    scale_q = 1.0
    for r in pick:
        h, i = divmod(r, nq)
        keys = np.concatenate([kb[j] for j in rows_gpu[r]])
        o_ref, _ = oracle.attention_rows(Q[0, h, qb[i]], K[0, h], V[0, h], hs[h], keys)
        gq, _, _ = oracle.row_backward(Q[0, h, qb[i]], dO[0, h, qb[i]], K[0, h], V[0, h], hs[h],
                                       keys)
        worst_o = max(worst_o, float(np.abs(Og[0, h, qb[i]] - o_ref).max()))
        worst_q = max(worst_q, float(np.abs(dQg[0, h, qb[i]] - gq).max()))
        scale_q = max(scale_q, float(np.abs(gq).max()))
    log(f"  O max-abs {worst_o:.2e}; dQ max-abs {worst_q:.2e} (scale {scale_q:.2f}) "
        f"over {len(pick)} q-blocks")
    assert worst_o <= 1e-2
    assert worst_q <= 2e-2 * scale_q
    # dK, dV per sampled head on three kv blocks: the one with the fewest selecting query
    # blocks, the median one and the one with the most (the longest CSC column, where the dK/dV
    # kernel streams the most query chunks). Each selecting query block's gradient is formed once
    # by the oracle over its whole selection and its segment added to every checked column.
    worst_k = worst_v = 0.0
    scale_kv = 1.0
    for h in rng.choice(w.H, size=2, replace=False):
        cols = {}
        for i in range(nq):
            for j in rows_gpu[h * nq + i].tolist():
                cols.setdefault(j, []).append(i)
        if not cols:
            continue
        by_len = sorted(cols, key=lambda j: (len(cols[j]), j))
        checked = sorted({by_len[0], by_len[len(by_len) // 2], by_len[-1]})
        gk = {J: np.zeros((len(kb[J]), w.d)) for J in checked}
        gv = {J: np.zeros((len(kb[J]), w.d)) for J in checked}
        for i in sorted({i for J in checked for i in cols[J]}):
            sel = rows_gpu[h * nq + i]
            keys = np.concatenate([kb[j] for j in sel])
            _, dk_keys, dv_keys = oracle.row_backward(Q[0, h, qb[i]], dO[0, h, qb[i]], K[0, h],
                                                      V[0, h], hs[h], keys)
            for J in checked:
                if i not in cols[J]:
                    continue
                start = int(sum(len(kb[j]) for j in sel if j < J))  # J's segment within keys
                idx = np.arange(start, start + len(kb[J]))
                gk[J] += dk_keys[idx]
                gv[J] += dv_keys[idx]
        for J in checked:
            worst_k = max(worst_k, float(np.abs(dKg[0, h, kb[J]] - gk[J]).max()))
            worst_v = max(worst_v, float(np.abs(dVg[0, h, kb[J]] - gv[J]).max()))
            scale_kv = max(scale_kv, float(np.abs(gk[J]).max()), float(np.abs(gv[J]).max()))
        log(f"  head {h} kv blocks {checked}: {[len(cols[J]) for J in checked]} selecting "
            f"q-blocks")
    log(f"  dK max-abs {worst_k:.2e} dV max-abs {worst_v:.2e} (scale {scale_kv:.2f})")
    assert worst_k <= 2e-2 * scale_kv and worst_v <= 2e-2 * scale_kv
    # kv blocks no query block selected get exactly zero gradient
    for h in range(w.H):
        used = set()
        for i in range(nq):
            used.update(rows_gpu[h * nq + i].tolist())
        for J in sorted(set(range(len(kb))) - used)[:3]:
            assert np.all(dKg[0, h, kb[J]] == 0) and np.all(dVg[0, h, kb[J]] == 0)
