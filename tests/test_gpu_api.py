"""The boundary's documented behaviour beyond parity (needs a device for the plan):

- size limits are rejected before anything is enqueued (32-bit CSR offsets);
- the binding refuses tensors whose shape, dtype, layout or device the kernels would misread;
- CSR entries outside [0, nkv) are skipped by the forward and the backward;
- NaN inputs propagate into the outputs they touch, and the selection stays a valid CSR;
- the backward is deterministic (no atomics): two calls give the same bits.
"""
import ctypes
from dataclasses import replace

import numpy as np
import pytest

import oracle
from gen import CONFIGS, make_inputs
from helpers import dev_to_f64, log, to_dev, to_f64

pytestmark = pytest.mark.gpu


def _plan_handle(B, H, grid, qpart, kvpart, d=128):
    import block_sparse_attention_bsa_amd as bsa
    return bsa.Plan(B, H, d, grid, qpart, kvpart, dtype="bf16")


def test_size_limits_rejected_before_any_launch():
    import block_sparse_attention_bsa_amd as bsa
    L = bsa.lib()
    # one-token blocks over 8192 tokens: H * nq * nkv = 64 * 8192^2 > 2^31 - 1
    plan = _plan_handle(1, 64, (8192, 1, 1), ("flat", 1), ("flat", 1))
    fake = 256  # never dereferenced: every check runs before anything is enqueued
    prm = bsa.SelectParams(0.9, bsa.BSA_POOL_ROW, bsa.BSA_MINK_NONE, 0)
    rc = L.bsa_select(plan.handle, fake, ctypes.byref(prm), fake, fake, 1 << 40, None, None,
                      fake, 1 << 40, None)
    assert rc == bsa.BSA_EUNSUPPORTED, L.bsa_last_error()
    assert b"2^31" in L.bsa_last_error()
    rc = L.bsa_attn_bwd(plan.handle, *([fake] * 12), 1 << 40, None)
    assert rc == bsa.BSA_EUNSUPPORTED, L.bsa_last_error()
    # per-token selection: 2048 kv blocks (its own limit), H * nq * nkv above 2^31 - 1
    plan2 = _plan_handle(1, 2048, (2048, 1, 1), ("flat", 1), ("flat", 1))
    rc = L.bsa_select_tokens(plan2.handle, fake, fake, 2, fake, fake, fake, 1 << 40, fake,
                             1 << 40, None)
    assert rc == bsa.BSA_EUNSUPPORTED, L.bsa_last_error()


def test_binding_rejects_misread_tensors():
    import torch
    from block_sparse_attention_bsa_amd import Plan
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    w = replace(CONFIGS[2], grid=(4, 8, 8), H=2)
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart)
    shp = (1, 2, 256, 128)
    good = torch.zeros(shp, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):  # [B, N, H, d] read as [B, H, N, d]
        layer.pool(good.transpose(1, 2).contiguous().view(1, 256, 2, 128), good)
    with pytest.raises(ValueError):  # a transposed view
        layer.pool(good.transpose(2, 3).contiguous().transpose(2, 3), good)
    with pytest.raises(TypeError):  # fp32 on a bf16 plan
        layer.pool(good.float(), good)
    with pytest.raises(ValueError):
        layer.pool(good.cpu(), good)
    with pytest.raises(TypeError):
        layer.attention(good, good, good, row_ptr=layer.row_ptr.long())
    with pytest.raises(ValueError):
        Plan(1, 3, 128, (4, 8, 8), w.qpart, w.kvpart, head_scale=np.ones(2, np.float32))


def test_out_of_range_csr_entries_are_skipped():
    # Rows listing bad indices (negative, nkv, huge) among good ones give the same O, LSE and
    # gradients as the rows with the bad entries removed.
    import torch
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    w = replace(CONFIGS[2], grid=(5, 8, 16), H=2)
    x = make_inputs(w, tensors=("q", "k", "v", "do"))
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    nkv = len(kb)
    rng = np.random.default_rng(8)
    good, bad = [], []
    for _ in range(w.H * len(qb)):
        sel = np.sort(rng.choice(nkv, size=int(rng.integers(1, nkv + 1)), replace=False))
        good.append(sel)
        junk = rng.choice([-1, nkv, nkv + 7, 1 << 30, -(1 << 30)], size=2)
        bad.append(np.concatenate([junk[:1], sel, junk[1:]]))
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart,
                                 head_scale=x["head_scale"])
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    outs = []
    for rows in (good, bad):
        rp, ci = oracle.to_csr(rows)
        rp_d, ci_d = torch.from_numpy(rp).cuda(), torch.from_numpy(ci).cuda()
        O, L = layer.attention(q, k, v, row_ptr=rp_d, col_idx=ci_d)
        O2, _ = layer.attention(q, k, v, row_ptr=rp_d, col_idx=ci_d, with_lse=False)
        dq, dk, dv = layer.backward(q, k, v, O, do, L, row_ptr=rp_d, col_idx=ci_d)
        torch.cuda.synchronize()
        outs.append([t.clone() for t in (O, L, O2, dq, dk, dv)])
    for name, a, b in zip(("O", "LSE", "O (no LSE)", "dQ", "dK", "dV"), *outs):
        assert torch.equal(a, b), f"{name} differs when bad CSR entries are present"
    log("out-of-range CSR entries skipped: forward, output-only forward and backward identical")


def test_nan_inputs_propagate_and_selection_stays_valid():
    import torch
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    w = replace(CONFIGS[2], grid=(5, 8, 16), H=2)
    x = make_inputs(w)
    qb, kb = oracle.partition(w.grid, w.qpart), oracle.partition(w.grid, w.kvpart)
    nq, nkv = len(qb), len(kb)
    qn = x["q"].copy()
    h0, I0 = 1, 3
    tok = int(qb[I0][0])
    qn[0, h0, tok, :] = 0x7FC0  # bf16 NaN in one query token
    vn = x["v"].copy()
    h1, J1 = 0, 2
    vn[0, h1, int(kb[J1][0]), 5] = 0x7FC0  # and in one value row
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart,
                                 head_scale=x["head_scale"])
    q, k, v = to_dev(qn), to_dev(x["k"]), to_dev(vn)
    O, L = layer.forward(q, k, v, w.p)
    torch.cuda.synchronize()
    rp, ci = layer.csr_host()
    rows = oracle.csr_rows(rp, ci)
    assert rp[0] == 0 and np.all(np.diff(rp) >= 0) and np.all(np.diff(rp) <= nkv)
    for r in rows:
        assert np.all((r >= 0) & (r < nkv)) and np.all(np.diff(r) > 0)
    Og = dev_to_f64(O)
    # the NaN query's row of pooled Q is NaN: its block's queries see NaN scores, unless the
    # block's row came out empty (it cannot: a NaN row keeps every block)
    r0 = h0 * nq + I0
    assert len(rows[r0]) > 0
    assert np.all(np.isnan(Og[0, h0, tok]))
    # every query of head h1 whose row selects J1 reads the NaN value row: NaN in channel 5
    for I in range(nq):
        sel = rows[h1 * nq + I]
        toks = qb[I]
        if J1 in sel.tolist():
            assert np.all(np.isnan(Og[0, h1, toks, 5]))
        elif not (h1 == h0 and I == I0):
            assert np.all(np.isfinite(Og[0, h1, toks]))
    # everything the NaNs cannot reach stays finite
    other = [h for h in range(w.H) if h not in (h0, h1)]
    for h in other:
        assert np.all(np.isfinite(Og[0, h]))
    log(f"NaN propagation: row {r0} keeps {len(rows[r0])}/{nkv} blocks")


def test_backward_is_deterministic():
    import torch
    from block_sparse_attention_bsa_amd.layer import BlockSparseAttention
    w = replace(CONFIGS[5], grid=(6, 9, 20), H=3, kvpart=("tile", (2, 3, 5)))
    x = make_inputs(w, tensors=("q", "k", "v", "do"))
    layer = BlockSparseAttention(w.B, w.H, w.d, w.grid, w.qpart, w.kvpart,
                                 head_scale=x["head_scale"])
    q, k, v, do = (to_dev(x[n]) for n in ("q", "k", "v", "do"))
    O, L = layer.forward(q, k, v, 0.5, mode="head")
    first = [t.clone() for t in layer.backward(q, k, v, O, do, L)]
    for _ in range(2):
        again = layer.backward(q, k, v, O, do, L)
        torch.cuda.synchronize()
        for name, a, b in zip(("dQ", "dK", "dV"), first, again):
            assert torch.equal(a, b), f"{name} differs between two identical backward calls"
    log("backward: three calls bit-identical")


def test_measurement_probes():
    """The copy probe copies exactly; the MFMA probe (peak loops and matrix/vector mixes) reports
    the FLOPs of its MFMAs and rejects bad arguments (the bench's measured ceilings come from
    these two)."""
    import torch
    import block_sparse_attention_bsa_amd as bsa
    src = torch.arange(1 << 20, dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    bsa.bsa_probe_copy(src, dst, src.numel() * 4)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
    sink = torch.zeros(4 * 256, dtype=torch.float32, device="cuda")
    for shape in range(7):  # the two peak loops and the five matrix/vector mixes
        f = bsa.bsa_probe_mfma(shape, 4, 3, sink)
        torch.cuda.synchronize()
        assert f == (0 if shape in (4, 6) else 4 * 4 * 3 * 8 * 2 * 32 * 32 * 16)
    assert bsa.lib().bsa_probe_mfma(0, 0, 3, sink.data_ptr(), None, None) == bsa.BSA_EINVAL
    assert bsa.lib().bsa_probe_mfma(7, 4, 3, sink.data_ptr(), None, None) == bsa.BSA_EINVAL
    assert bsa.lib().bsa_probe_copy(src.data_ptr(), dst.data_ptr(), 10, None) == bsa.BSA_EINVAL
