"""GPU parity of bsa_attn_bwd (and the forward it consumes) against the oracle's fp64 gradients,
on the oracle's own selection so both sides differentiate the same block-sparse attention.

Tolerance (bf16 inputs and outputs, fp32 accumulation): per gradient tensor, max-abs error
<= 2e-2 * max(1, max |ref|) and relative L2 error <= 1e-2. Tokens that no selected pair touches
must get exactly zero gradient."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from gen import CONFIGS, make_inputs
from helpers import dev_to_f64, log, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _grad_ok(name, got, ref):
    err = np.abs(got - ref).max()
    scale = max(1.0, float(np.abs(ref).max()))
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    log(f"  {name}: max-abs {err:.3e} (bar {2e-2 * scale:.3e}) rel-L2 {rel:.3e}")
    assert err <= 2e-2 * scale
    assert rel <= 1e-2


def _head_rows(w, x, kvpart, tau):
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, kvpart)
    Q, K = to_f64(x["q"]), to_f64(x["k"])
    W = oracle.score_head(oracle.pool(Q, qb), oracle.pool(K, kb), x["head_scale"].astype(float),
                          oracle.block_sizes(qb))
    return oracle.select_head(W, tau), qb, kb


def _run(w, kvpart, rows=None, tau=None):
    import torch
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    w = replace(w, kvpart=kvpart)
    x = make_inputs(w, tensors=("q", "k", "v", "do"))
    if rows is None:
        rows, qb, kb = _head_rows(w, x, kvpart, tau if tau is not None else w.p)
    else:
        qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, kvpart)
    rp, ci = oracle.to_csr(rows)
    empty = sum(len(r) == 0 for r in rows)
    log(f"bwd grid={w.grid} H={w.H} kv={kvpart}: {len(rows)} rows, {empty} empty")
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, kvpart, dtype=w.dtype,
                                 head_scale=x["head_scale"])
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    rp_d = torch.from_numpy(rp).cuda()
    ci_d = torch.from_numpy(ci if len(ci) else np.zeros(1, np.int32)).cuda()
    O, L = layer.attention(q, k, v, row_ptr=rp_d, col_idx=ci_d)
    dq, dk, dv = layer.backward(q, k, v, O, do, L, row_ptr=rp_d, col_idx=ci_d)
    torch.cuda.synchronize()
    Q, K, V, dO = (to_f64(x[n]) for n in ("q", "k", "v", "do"))
    hs = x["head_scale"].astype(np.float64)
    O_ref, _ = oracle.attention_fwd(Q, K, V, hs, qb, kb, rp, ci)
    assert np.abs(dev_to_f64(O) - O_ref).max() <= 1e-2
    dQ, dK, dV = oracle.attention_bwd(Q, K, V, dO, hs, qb, kb, rp, ci)
    g = {n: dev_to_f64(t) for n, t in (("dQ", dq), ("dK", dk), ("dV", dv))}
    _grad_ok("dQ", g["dQ"], dQ)
    _grad_ok("dK", g["dK"], dK)
    _grad_ok("dV", g["dV"], dV)
    # exact zeros where no selected pair reaches
    nq = len(qb)
    for r, sel in enumerate(rows):
        if len(sel) == 0:
            bh, I = divmod(r, nq)
            b, h = divmod(bh, w.H)
            assert np.all(g["dQ"][b, h, qb[I]] == 0)
    for bh in range(w.B * w.H):
        b, h = divmod(bh, w.H)
        used = set()
        for I in range(nq):
            used.update(rows[bh * nq + I].tolist())
        for J in set(range(len(kb))) - used:
            assert np.all(g["dK"][b, h, kb[J]] == 0) and np.all(g["dV"][b, h, kb[J]] == 0)
    return g


@pytest.mark.parametrize("kvpart", [("tile", (3, 9, 20)), ("tile", (6, 3, 5)),
                                    ("tile", (3, 3, 4))])
def test_bwd_head_pool_reduced(kvpart):
    w = replace(CONFIGS[5], grid=(6, 9, 20), H=2)
    _run(w, kvpart)


def test_bwd_random_rows_with_empty_rows_and_ragged_blocks():
    w = replace(CONFIGS[5], grid=(5, 9, 20), H=2)
    kvpart = ("tile", (4, 4, 8))
    qb = oracle.partition(w.grid, w.qpart)
    kb = oracle.partition(w.grid, kvpart)
    rng = np.random.default_rng(21)
    rows = []
    for r in range(w.H * len(qb)):
        k = int(rng.integers(0, len(kb) + 1))
        rows.append(np.sort(rng.choice(len(kb), size=k, replace=False)))
    _run(w, kvpart, rows=rows)


def test_bwd_batch2_random_rows():
    w = replace(CONFIGS[5], B=2, grid=(5, 9, 20), H=2)
    kvpart = ("tile", (4, 4, 8))
    qb = oracle.partition(w.grid, w.qpart)
    kb = oracle.partition(w.grid, kvpart)
    rng = np.random.default_rng(23)
    rows = []
    for r in range(w.B * w.H * len(qb)):
        k = int(rng.integers(0, len(kb) + 1))
        rows.append(np.sort(rng.choice(len(kb), size=k, replace=False)))
    _run(w, kvpart, rows=rows)
