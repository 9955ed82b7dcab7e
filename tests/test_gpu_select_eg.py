"""GPU parity of bsa_select_eg (entropy-routed competition domains, EG-Sparse abstract) against
the oracle's select_eg on the same seeded inputs (each side pools and scores them itself).

Bar: head entropies within 1e-5 absolute (fp32 scores on the GPU, fp64 in the oracle); the
pooled-head flags identical (theta is placed in a gap of the oracle's entropies, at least 1e-4
from every head); block sets bit-exact except near-ties, accepted by the tie-tolerant rule of the
other selections: per row for per-row heads, over the flattened pool weights for a group."""
from dataclasses import replace

import numpy as np
import pytest

import oracle
from gen import CONFIGS, make_inputs
from helpers import dev_to_f64, log, to_dev, to_f64, topp_set_ok

pytestmark = pytest.mark.gpu


def _theta_in_gap(ent, frac=0.5, margin=1e-4):
    """A threshold midway between two neighbouring head entropies, at least `margin` from each:
    the usable gap nearest the `frac` quantile."""
    e = np.sort(ent.reshape(-1))
    k = int(round(frac * (len(e) - 1)))
    for i in sorted(range(len(e) - 1), key=lambda i: abs(i - k)):
        if e[i + 1] - e[i] > 2 * margin:
            return 0.5 * (e[i] + e[i + 1])
    raise AssertionError("no usable entropy gap")


def _check(w, rows_gpu, ent_gpu, pooled_gpu, S_ref, qs, p, theta, G):
    rows_ref, ent_ref, pooled_ref = oracle.select_eg(S_ref, p, qs, theta, G)
    B, H, nq, nkv = S_ref.shape
    eerr = float(np.abs(ent_gpu.reshape(B, H) - ent_ref).max())
    log(f"  entropy max-abs {eerr:.2e}; pooled heads {int(pooled_ref.sum())} of {B * H}")
    assert eerr <= 1e-5
    assert np.array_equal(pooled_gpu.reshape(B, H).astype(bool), pooled_ref)
    exact = tol = 0
    N = float(np.sum(qs))
    for b in range(B):
        for g0 in range(0, H, G):
            heads = list(range(g0, min(g0 + G, H)))
            members = [h for h in heads if pooled_ref[b, h]]
            for h in heads:
                if pooled_ref[b, h]:
                    continue
                for i in range(nq):
                    r = (b * H + h) * nq + i
                    g = rows_gpu[r]
                    assert len(g) < 2 or np.all(np.diff(g) > 0)
                    ok, ex = topp_set_ok(g, rows_ref[r], S_ref[b, h, i], p)
                    assert ok, (b, h, i)
                    exact += ex
                    tol += not ex
            if not members:
                continue
            m = len(members)
            W = np.concatenate([(S_ref[b, h] * np.asarray(qs, np.float64)[:, None] / (N * m))
                                .reshape(-1) for h in members])
            def flat(rows):
                out = []
                for k, h in enumerate(members):
                    for i in range(nq):
                        sel = np.asarray(rows[(b * H + h) * nq + i], np.int64)
                        assert len(sel) < 2 or np.all(np.diff(sel) > 0)
                        out.append((k * nq + i) * nkv + sel)
                return np.concatenate(out) if out else np.zeros(0, np.int64)
            ok, ex = topp_set_ok(flat(rows_gpu), flat(rows_ref), W, p)
            assert ok, (b, g0)
            exact += ex
            tol += not ex
    log(f"  sets: exact {exact}, tolerated near-ties {tol}")


def _run(w, G, p=None, frac=0.5, theta=None, seed=0, x=None, S_ref=None, margin=1e-4):
    """x (the workload's inputs) and S_ref (the oracle's row scores of them) may be passed in by
    a caller that already has them."""
    import torch
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    p = w.p if p is None else p
    x = make_inputs(w) if x is None else x
    hs = x["head_scale"]
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    qs = oracle.block_sizes(qb)
    if S_ref is None:
        Q, K = to_f64(x["q"]), to_f64(x["k"])
        S_ref = oracle.score_row(oracle.pool(Q, qb), oracle.pool(K, kb), hs.astype(np.float64))
        del Q, K
    if theta is None:
        theta = _theta_in_gap(oracle.head_entropy(S_ref, qs), frac, margin)
    log(f"eg {w.name} grid={w.grid} B={w.B} H={w.H} G={G} p={p} theta={theta:.6f}")
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart, dtype=w.dtype,
                                 head_scale=hs)
    q, k = to_dev(x["q"]), to_dev(x["k"])
    layer.pool(q, k)
    layer.score(0)
    layer.select_eg(p, theta, G)
    torch.cuda.synchronize()
    rp, ci = layer.csr_host()
    rows_gpu = oracle.csr_rows(rp, ci)
    assert np.array_equal(np.diff(rp), layer.counts.cpu().numpy())
    _check(w, rows_gpu, layer.head_entropy.cpu().numpy(), layer.head_pooled.cpu().numpy(),
           S_ref, qs, p, theta, G)
    return layer, rows_gpu


SMALL = replace(CONFIGS[2], grid=(9, 14, 26), H=6)


@pytest.mark.parametrize("G", [1, 2, 4, 6])
def test_eg_reduced(G):
    _run(SMALL, G, frac=0.7)


def test_eg_per_head_temperatures():
    # per-head softmax temperatures spread the head entropies
    _run(replace(CONFIGS[3], grid=(9, 14, 26), H=8), 3, p=0.9, frac=0.6)


def test_eg_batch2_ragged_groups():
    _run(replace(CONFIGS[2], grid=(5, 8, 16), H=5, B=2), 2, frac=0.4)


def test_eg_p_one_and_extreme_thresholds():
    import torch
    w = replace(CONFIGS[2], grid=(5, 8, 16), H=3)
    layer, rows = _run(w, 3, p=1.0)
    nkv = layer.plan.nkv
    assert all(len(r) == nkv for r in rows)
    # theta = -inf pools nothing: identical to the per-row selection
    _, rows_none = _run(w, 2, theta=-np.inf)
    layer.select(w.p)
    torch.cuda.synchronize()
    rp, ci = layer.csr_host()
    assert all(np.array_equal(a, b) for a, b in zip(rows_none, oracle.csr_rows(rp, ci)))
    # theta = +inf pools every head into one group
    _run(w, 3, theta=np.inf)


def test_eg_full_size_480p():
    _run(CONFIGS[2], 4)


def test_eg_rejects_bad_parameters():
    import torch
    import block_sparse_attention_bsa_amd as bsa
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    w = replace(CONFIGS[2], grid=(5, 8, 16), H=2)
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart)
    for p, theta, G in ((0.0, 0.5, 1), (1.5, 0.5, 1), (0.9, np.nan, 1), (0.9, 0.5, 0)):
        with pytest.raises(bsa.BsaError) as ei:
            layer.select_eg(p, theta, G)
        assert ei.value.code == bsa.BSA_EINVAL
    with pytest.raises(bsa.BsaError) as ei:
        bsa.bsa_select_eg(layer.plan, layer.S, 0.9, 0.5, 1, layer.row_ptr, layer.col_idx,
                          layer.col_cap, None, None, None, layer.ws_select,
                          layer.plan.ws_select - 1)
    assert ei.value.code == bsa.BSA_ECAPACITY
    torch.cuda.synchronize()
