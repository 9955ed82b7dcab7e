"""GPU parity of bsa_select with BSA_POOL_LOCAL_TOPK (VMoBA's training-free Local + TopK, k = 2,
6 or 18) against the oracle's select_local_topk on the same seeded inputs (each side pools and
scores them itself).

Bar: every row keeps exactly its local blocks plus min(k, nkv - |local|) others; the others equal
the oracle's, or, at a near-tie, form a top set of the oracle's fp64 scores within 1e-6."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from gen import CONFIGS, make_inputs
from helpers import log, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _run(w, k):
    import torch
    import block_sparse_attention_bsa_amd as bsa
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    x = make_inputs(w, tensors=("q", "k"))
    hs = x["head_scale"]
    Q, K = to_f64(x["q"]), to_f64(x["k"])
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    S = oracle.score_row(oracle.pool(Q, qb), oracle.pool(K, kb), hs.astype(np.float64))
    local = oracle.local_blocks(qb, kb)
    ref = oracle.select_local_topk(S, k, local)
    log(f"local+top{k} {w.name} grid={w.grid} B={w.B} H={w.H} q={w.qpart} kv={w.kvpart} "
        f"local sizes {min(map(len, local))}..{max(map(len, local))}")
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart, head_scale=hs)
    layer.pool(to_dev(x["q"]), to_dev(x["k"]))
    layer.score(0)
    layer.select(0.5, pool=bsa.BSA_POOL_LOCAL_TOPK, fixed_k=k)
    torch.cuda.synchronize()
    rp, ci = layer.csr_host()
    rows = oracle.csr_rows(rp, ci)
    nq, nkv = len(qb), len(kb)
    exact = tol = 0
    for r, (g, o) in enumerate(zip(rows, ref)):
        i = r % nq
        b, h = divmod(r // nq, w.H)
        assert len(g) < 2 or np.all(np.diff(g) > 0)
        if np.array_equal(g, o):
            exact += 1
            continue
        loc = set(local[i].tolist())
        assert loc <= set(g.tolist()), r
        extra = [j for j in g.tolist() if j not in loc]
        others = [j for j in range(nkv) if j not in loc]
        assert len(extra) == min(k, len(others)), r
        s = S[b, h, i]
        rest = [j for j in others if j not in extra]
        assert not rest or min(s[extra]) >= max(s[rest]) - 1e-6, r
        tol += 1
    log(f"  rows exact {exact}, tolerated near-ties {tol}")
    return layer


SMALL = replace(CONFIGS[2], grid=(9, 14, 26), H=3)


@pytest.mark.parametrize("k", [0, 2, 6, 18])
def test_local_topk_same_partition(k):
    _run(SMALL, k)


def test_local_topk_several_local_blocks():
    # 3D query tiles against 1D temporal kv blocks: every query block meets one or two of them
    _run(replace(SMALL, kvpart=("tile", (3, 14, 26))), 2)
    # and against 2D spatial blocks, several per query block
    _run(replace(SMALL, kvpart=("tile", (9, 7, 13))), 6)


def test_local_topk_more_than_available_and_batch2():
    w = replace(CONFIGS[2], grid=(5, 8, 16), H=2, B=2)
    layer = _run(w, 1000)
    rp, _ = layer.csr_host()
    assert np.all(np.diff(rp) == layer.plan.nkv)


def test_local_topk_full_size_480p():
    _run(CONFIGS[2], 6)


def test_local_topk_full_size_720p_wide_rows():
    _run(CONFIGS[4], 18)          # 1080 kv blocks: the 32-values-per-lane path


def test_local_topk_rejects_bad_parameters():
    import torch
    import block_sparse_attention_bsa_amd as bsa
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    w = replace(CONFIGS[2], grid=(5, 8, 16), H=2)
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart)
    for fixed_k, mink in ((-1, bsa.BSA_MINK_NONE), (2, bsa.BSA_MINK_FIXED)):
        with pytest.raises(bsa.BsaError) as ei:
            layer.select(0.5, pool=bsa.BSA_POOL_LOCAL_TOPK, min_k_mode=mink, fixed_k=fixed_k)
        assert ei.value.code == bsa.BSA_EINVAL
    torch.cuda.synchronize()
