"""C-ABI boundary checks that need no GPU: the library loads, exports every declared symbol,
builds partitions identical to the oracle's, and rejects bad arguments before any device call."""
import ctypes
import os
import re

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
bsa = pytest.importorskip("block_sparse_attention_bsa_amd")


def _declared():
    with open(os.path.join(ROOT, "include", "bsa.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:int|const char\*)\s+(bsa_\w+)\s*\(", text, re.M)))


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bsa.LIB_PATH):
        pytest.fail("libbsa.so is not built (run __graft_entry__.build())")
    return bsa.lib()


def test_exports_every_declared_symbol(L):
    names = _declared()
    assert len(names) >= 12
    assert sorted(bsa.EXPORTED) == names
    for n in names:
        assert hasattr(L, n)


@pytest.mark.parametrize("grid,part", [
    ((4, 8, 8), ("flat", 32)), ((21, 30, 52), ("tile", (4, 4, 8))),
    ((33, 45, 80), ("tile", (4, 4, 8))), ((21, 45, 80), ("tile", (3, 45, 80))),
    ((21, 45, 80), ("tile", (21, 15, 5))), ((21, 45, 80), ("tile", (7, 9, 20))),
    ((5, 7, 9), ("tile", (2, 3, 4))), ((1, 2, 5), ("flat", 4)), ((3, 3, 3), ("flat", 100))])
def test_partition_build_matches_oracle(L, grid, part):
    perm, start = bsa.bsa_partition_build(grid, part)
    blocks = oracle.partition(grid, part)
    assert len(start) == len(blocks) + 1
    for j, b in enumerate(blocks):
        np.testing.assert_array_equal(perm[start[j]:start[j + 1]], b)


def _problem(**kw):
    base = dict(B=1, H=2, N=256, d=64, dtype=bsa.BSA_FP32, T=4, Hg=8, Wg=8)
    base.update(kw)
    pr = bsa.Problem(base["B"], base["H"], base["N"], base["d"], base["dtype"], base["T"],
                     base["Hg"], base["Wg"], bsa.make_partition(("flat", 32)),
                     bsa.make_partition(("tile", (1, 4, 8))))
    return pr


@pytest.mark.parametrize("kw,code", [
    (dict(N=255), bsa.BSA_EINVAL), (dict(B=0), bsa.BSA_EINVAL), (dict(dtype=7), bsa.BSA_EINVAL),
    (dict(d=96), bsa.BSA_EUNSUPPORTED), (dict(T=0, N=0), bsa.BSA_EINVAL)])
def test_plan_create_rejects_before_any_device_call(L, kw, code):
    pr = _problem(**kw)
    h = ctypes.c_void_p(None)
    rc = L.bsa_plan_create(ctypes.byref(pr), None, ctypes.byref(h))
    assert rc == code
    assert h.value is None
    assert L.bsa_last_error().decode()


def test_bad_partitions_rejected(L):
    pr = _problem()
    pr.qpart = bsa.Partition(bsa.BSA_PART_TILE, 0, 0, 4, 8)
    h = ctypes.c_void_p(None)
    assert L.bsa_plan_create(ctypes.byref(pr), None, ctypes.byref(h)) == bsa.BSA_EINVAL
    pr = _problem()
    pr.kvpart = bsa.Partition(5, 1, 1, 1, 1)
    assert L.bsa_plan_create(ctypes.byref(pr), None, ctypes.byref(h)) == bsa.BSA_EINVAL
    for bad in (np.nan, 0.0, -0.5, np.inf):
        hs = np.array([1.0, bad], np.float32)
        assert L.bsa_plan_create(ctypes.byref(_problem()), hs.ctypes.data,
                                 ctypes.byref(h)) == bsa.BSA_EINVAL


def test_null_arguments_rejected(L):
    P = None
    assert L.bsa_pool(P, 0, None, None, None) == bsa.BSA_EINVAL
    assert L.bsa_pool_qk(P, None, None, None, None, None) == bsa.BSA_EINVAL
    assert L.bsa_score(P, None, None, 0, None, None) == bsa.BSA_EINVAL
    assert L.bsa_calibrate_mass(P, None, None, None, None, 0, None) == bsa.BSA_EINVAL
    assert L.bsa_calibrate_mass_fwd(P, *([None] * 7), 0, None) == bsa.BSA_EINVAL
    prm = bsa.SelectParams(0.9, 0, 0, 0)
    assert L.bsa_select(P, None, ctypes.byref(prm), None, None, 0, None, None, None, 0,
                        None) == bsa.BSA_EINVAL
    eg = bsa.EgParams(0.9, 0.5, 2)
    assert L.bsa_select_eg(P, None, ctypes.byref(eg), None, None, 0, None, None, None, None, 0,
                           None) == bsa.BSA_EINVAL
    assert L.bsa_select_tokens(P, None, None, 2, None, None, None, 0, None, 0,
                               None) == bsa.BSA_EINVAL
    assert L.bsa_attn_fwd_tokens(P, *([None] * 6), 2, None, None, None, 0,
                                 None) == bsa.BSA_EINVAL
    assert L.bsa_tokens_ws(P, None) == bsa.BSA_EINVAL
    assert L.bsa_attn_fwd(P, None, None, None, None, None, None, None, None, 0,
                          None) == bsa.BSA_EINVAL
    assert L.bsa_attn_bwd(P, *([None] * 12), 0, None) == bsa.BSA_EINVAL
    assert L.bsa_plan_destroy(None) == bsa.BSA_EINVAL
    assert L.bsa_plan_info(None, None, None, None, None, None, None) == bsa.BSA_EINVAL
    assert L.bsa_plan_blocks(None, 0, None, None) == bsa.BSA_EINVAL


def test_partition_build_capacity_and_errors(L):
    part = bsa.make_partition(("tile", (4, 4, 8)))
    perm = np.empty(32760, np.int32)
    start = np.empty(11, np.int32)
    n = ctypes.c_int32(0)
    rc = L.bsa_partition_build(21, 30, 52, ctypes.byref(part), perm.ctypes.data,
                               start.ctypes.data, 10, ctypes.byref(n))
    assert rc == bsa.BSA_ECAPACITY and n.value == 336
    bad = bsa.make_partition(("flat", 0))
    assert L.bsa_partition_build(2, 2, 2, ctypes.byref(bad), perm.ctypes.data,
                                 start.ctypes.data, 10, ctypes.byref(n)) == bsa.BSA_EINVAL


def test_stale_library_is_refused(monkeypatch, L):
    """The in-tree library records the hash of the sources it was built from; a library built
    from other sources fails to load instead of running old kernels."""
    from block_sparse_attention_bsa_amd import build
    monkeypatch.setattr(bsa, "_lib", None)
    monkeypatch.setattr(build, "source_hash", lambda: "0" * 64)
    with pytest.raises(ImportError, match="other sources"):
        bsa.lib()
    monkeypatch.undo()
    assert bsa.lib() is not None
