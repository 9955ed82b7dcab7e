"""GPU parity of bsa_score_select, the scores and ROW-pool selection in one pass (no score matrix
in memory): bit-identical to bsa_score(ROW) followed by bsa_select at the 480p and 720p shapes
(with and without the per-head minimum count, whose top-up reads the scores it writes), and
against the oracle's selection at reduced, ragged, batch-2 and fp32 shapes with the near-tie
rule (selections bit-exact except near-ties within 1e-5 of p)."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from gen import CONFIGS, make_inputs
from helpers import check_csr_rows, log, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _layer(w, x):
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    return BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart, dtype=w.dtype,
                                head_scale=x["head_scale"])


def _csr(layer):
    import torch
    torch.cuda.synchronize()
    rp = layer.row_ptr.cpu().numpy().copy()
    ci = layer.col_idx[: int(rp[-1])].cpu().numpy().copy()
    return rp, ci, layer.counts.cpu().numpy().copy(), layer.head_k.cpu().numpy().copy()


@pytest.mark.parametrize("cid,min_k", [(2, 0), (4, 2), (4, 0), (3, 0)])
def test_fused_equals_score_then_select(cid, min_k):
    import torch
    w = CONFIGS[cid]
    x = make_inputs(w)
    layer = _layer(w, x)
    q, k = to_dev(x["q"]), to_dev(x["k"])
    layer.pool(q, k)
    S_ref = layer.score(0).clone()
    layer.select(w.p, min_k_mode=min_k)
    ref = _csr(layer)
    layer.S.fill_(-1.0)
    layer.score_select(w.p, min_k_mode=min_k, write_scores=True)
    got = _csr(layer)
    assert torch.equal(layer.S, S_ref), "scores written by the fused kernel differ"
    for name, a, b in zip(("row_ptr", "col_idx", "counts", "head_k"), ref, got):
        assert np.array_equal(a, b), f"{w.name}: {name} differs"
    layer.score_select(w.p, min_k_mode=min_k)  # without writing S unless the top-up needs it
    got2 = _csr(layer)
    for name, a, b in zip(("row_ptr", "col_idx", "counts", "head_k"), ref, got2):
        assert np.array_equal(a, b), f"{w.name}: {name} differs (scores not written)"
    log(f"{w.name} min_k={min_k}: fused selection identical, nnz {ref[0][-1]}")


@pytest.mark.parametrize("case", ["ragged", "batch2", "fp32", "p1", "d64_bf16"])
def test_fused_against_oracle(case):
    w = {"ragged": replace(CONFIGS[2], grid=(5, 7, 13), H=3),
         "batch2": replace(CONFIGS[2], B=2, grid=(6, 9, 20), H=2),
         "fp32": CONFIGS[1],
         "p1": replace(CONFIGS[2], grid=(5, 8, 16), H=2, p=1.0),
         "d64_bf16": replace(CONFIGS[1], dtype="bf16", d=64)}[case]
    x = make_inputs(w)
    layer = _layer(w, x)
    layer.pool(to_dev(x["q"]), to_dev(x["k"]))
    layer.score_select(w.p)
    rp, ci, _, _ = _csr(layer)
    Q, K = to_f64(x["q"]), to_f64(x["k"])
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    S = oracle.score_row(oracle.pool(Q, qb), oracle.pool(K, kb), x["head_scale"].astype(float))
    rows_ref = oracle.select_row(S, w.p)
    exact, tol, bad = check_csr_rows(oracle.csr_rows(rp, ci), rows_ref,
                                     S.reshape(-1, S.shape[-1]), w.p)
    log(f"{case}: rows exact {exact} tolerated {tol} bad {len(bad)}")
    assert not bad


def test_fused_rejects_other_pools():
    import ctypes
    import block_sparse_attention_bsa_amd as bsa
    w = replace(CONFIGS[2], grid=(4, 8, 8), H=2)
    layer = _layer(w, make_inputs(w))
    prm = bsa.SelectParams(0.25, bsa.BSA_POOL_HEAD, 0, 0)
    rc = bsa.lib().bsa_score_select(layer.plan.handle, layer.qbar.data_ptr(),
                                    layer.kbar.data_ptr(), ctypes.byref(prm), None,
                                    layer.row_ptr.data_ptr(), layer.col_idx.data_ptr(),
                                    layer.col_cap, None, None, layer.ws_select.data_ptr(),
                                    layer.plan.ws_select, None)
    assert rc == bsa.BSA_EUNSUPPORTED
