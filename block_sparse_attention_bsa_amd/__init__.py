"""Python binding of the block-sparse attention library (libbsa.so, HIP for gfx950).

Argument marshalling only: every function here forwards device pointers and sizes to the C ABI
declared in include/bsa.h, and every step of the computation runs in the library's HIP kernels.
PyTorch is used for device memory and streams. There is no CPU fallback: if the library is missing
or a call fails, an exception is raised.

Names follow the C ABI: bsa_pool, bsa_score, bsa_calibrate_mass(_fwd), bsa_select(_eg), bsa_attn_fwd,
bsa_attn_bwd, bsa_partition_build; a Plan wraps bsa_plan_create / bsa_plan_info /
bsa_plan_blocks / bsa_plan_destroy.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "_lib", "libbsa.so")
_DEFAULT_LIB = LIB_PATH

BSA_OK, BSA_EINVAL, BSA_EUNSUPPORTED, BSA_ECAPACITY, BSA_EHIP = 0, -1, -2, -3, -4
BSA_PART_FLAT, BSA_PART_TILE = 0, 1
BSA_BF16, BSA_FP32 = 0, 1
BSA_NORM_ROW, BSA_NORM_HEAD = 0, 1
BSA_POOL_ROW, BSA_POOL_HEAD, BSA_POOL_LOCAL_TOPK = 0, 1, 2
BSA_MINK_NONE, BSA_MINK_FIXED, BSA_MINK_WEIGHTED_MEAN = 0, 1, 2

EXPORTED = ("bsa_partition_build", "bsa_plan_create", "bsa_plan_destroy", "bsa_plan_info",
            "bsa_plan_blocks", "bsa_pool", "bsa_pool_qk", "bsa_score", "bsa_calibrate_mass",
            "bsa_calibrate_mass_fwd", "bsa_select", "bsa_select_noalloc", "bsa_score_select",
            "bsa_select_eg",
            "bsa_tokens_ws",
            "bsa_select_tokens", "bsa_attn_fwd", "bsa_attn_fwd_tokens", "bsa_attn_bwd",
            "bsa_tokens_global_ws", "bsa_select_tokens_global", "bsa_attn_fwd_token_bits",
            "bsa_probe_mfma", "bsa_probe_copy",
            "bsa_last_error")


class BsaError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class Partition(ctypes.Structure):
    _fields_ = [("kind", ctypes.c_int32), ("flat", ctypes.c_int32), ("bt", ctypes.c_int32),
                ("bh", ctypes.c_int32), ("bw", ctypes.c_int32)]


class Problem(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("T", ctypes.c_int32),
                ("Hg", ctypes.c_int32), ("Wg", ctypes.c_int32), ("qpart", Partition),
                ("kvpart", Partition)]


class SelectParams(ctypes.Structure):
    _fields_ = [("p", ctypes.c_double), ("pool", ctypes.c_int32),
                ("min_k_mode", ctypes.c_int32), ("fixed_k", ctypes.c_int32)]


class EgParams(ctypes.Structure):
    _fields_ = [("p", ctypes.c_double), ("theta", ctypes.c_double),
                ("group_size", ctypes.c_int32)]


_lib = None


def lib():
    """Load libbsa.so (built in-tree by block_sparse_attention_bsa_amd.build). Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"libbsa.so not built at {LIB_PATH}; run __graft_entry__.build()")
    if LIB_PATH == _DEFAULT_LIB:
        # the in-tree library must have been built from the sources as they are now
        from . import build as _build
        stamp = _build.STAMP
        built = open(stamp).read().strip() if os.path.exists(stamp) else None
        if built != _build.source_hash():
            raise ImportError(f"{LIB_PATH} was built from other sources than csrc/ and include/ "
                              f"hold now; run __graft_entry__.build()")
    L = ctypes.CDLL(LIB_PATH)
    P, I32, I64, SZ, D = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t,
                          ctypes.c_double)
    sig = {
        "bsa_partition_build": [I32, I32, I32, ctypes.POINTER(Partition), P, P, I32,
                                ctypes.POINTER(I32)],
        "bsa_plan_create": [ctypes.POINTER(Problem), P, ctypes.POINTER(P)],
        "bsa_plan_destroy": [P],
        "bsa_plan_info": [P, ctypes.POINTER(I32), ctypes.POINTER(I32), ctypes.POINTER(SZ),
                          ctypes.POINTER(SZ), ctypes.POINTER(SZ), ctypes.POINTER(SZ)],
        "bsa_plan_blocks": [P, I32, P, P],
        "bsa_pool": [P, I32, P, P, P],
        "bsa_pool_qk": [P, P, P, P, P, P],
        "bsa_score": [P, P, P, I32, P, P],
        "bsa_calibrate_mass": [P, P, P, P, P, SZ, P],
        "bsa_calibrate_mass_fwd": [P, P, P, P, P, P, P, P, SZ, P],
        "bsa_select": [P, P, ctypes.POINTER(SelectParams), P, P, I64, P, P, P, SZ, P],
        "bsa_select_noalloc": [P, P, ctypes.POINTER(SelectParams), P, P, I64, P, P, P],
        "bsa_score_select": [P, P, P, ctypes.POINTER(SelectParams), P, P, P, I64, P, P, P, SZ,
                             P],
        "bsa_select_eg": [P, P, ctypes.POINTER(EgParams), P, P, I64, P, P, P, P, SZ, P],
        "bsa_tokens_ws": [P, ctypes.POINTER(SZ)],
        "bsa_select_tokens": [P, P, P, I32, P, P, P, I64, P, SZ, P],
        "bsa_attn_fwd_tokens": [P, P, P, P, P, P, P, I32, P, P, P, SZ, P],
        "bsa_attn_fwd": [P, P, P, P, P, P, P, P, P, SZ, P],
        "bsa_tokens_global_ws": [P, ctypes.POINTER(SZ)],
        "bsa_probe_mfma": [I32, I32, I32, P, ctypes.POINTER(D), P],
        "bsa_probe_copy": [P, P, SZ, P],
        "bsa_select_tokens_global": [P, P, P, D, P, P, P, I64, P, SZ, P],
        "bsa_attn_fwd_token_bits": [P, P, P, P, P, P, P, P, P, P, SZ, P],
        "bsa_attn_bwd": [P, P, P, P, P, P, P, P, P, P, P, P, P, SZ, P],
    }
    for name, args in sig.items():
        fn = getattr(L, name)
        fn.argtypes = args
        fn.restype = ctypes.c_int
    L.bsa_last_error.argtypes = []
    L.bsa_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(rc: int):
    if rc != BSA_OK:
        raise BsaError(rc, lib().bsa_last_error().decode())


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    if isinstance(x, np.ndarray):
        return x.ctypes.data
    raise TypeError(f"cannot pass {type(x)} as a pointer")


def _stream(stream) -> Optional[int]:
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def make_partition(spec) -> Partition:
    kind, arg = spec
    if kind == "flat":
        return Partition(BSA_PART_FLAT, int(arg), 0, 0, 0)
    bt, bh, bw = arg
    return Partition(BSA_PART_TILE, 0, int(bt), int(bh), int(bw))


def bsa_partition_build(grid: Sequence[int], part) -> Tuple[np.ndarray, np.ndarray]:
    """Host-only partition: (perm[N], blk_start[nblk + 1]) as int32 numpy arrays."""
    T, Hg, Wg = (int(v) for v in grid)
    N = T * Hg * Wg
    perm = np.empty(N, np.int32)
    nblk = ctypes.c_int32(0)
    prt = make_partition(part)
    start = np.empty(1, np.int32)
    rc = lib().bsa_partition_build(T, Hg, Wg, ctypes.byref(prt), perm.ctypes.data,
                                   start.ctypes.data, 0, ctypes.byref(nblk))
    if rc != BSA_ECAPACITY and rc != BSA_OK:
        _check(rc)
    start = np.empty(nblk.value + 1, np.int32)
    _check(lib().bsa_partition_build(T, Hg, Wg, ctypes.byref(prt), perm.ctypes.data,
                                     start.ctypes.data, nblk.value, ctypes.byref(nblk)))
    return perm, start


class Plan:
    """A bsa_plan: partitions and per-head scales of one attention shape, on the current device."""

    def __init__(self, B: int, H: int, d: int, grid: Sequence[int], qpart, kvpart,
                 dtype: str = "bf16", head_scale=None):
        T, Hg, Wg = (int(v) for v in grid)
        self.B, self.H, self.d, self.grid = int(B), int(H), int(d), (T, Hg, Wg)
        self.N = T * Hg * Wg
        self.dtype = dtype
        prob = Problem(self.B, self.H, self.N, self.d, BSA_BF16 if dtype == "bf16" else BSA_FP32,
                       T, Hg, Wg, make_partition(qpart), make_partition(kvpart))
        hs = None
        if head_scale is not None:
            hs = np.ascontiguousarray(np.asarray(head_scale, np.float32).reshape(-1))
            if hs.size != self.H:  # the C ABI reads exactly H host floats
                raise ValueError(f"head_scale has {hs.size} entries, expected H = {self.H}")
        self._hs = hs
        handle = ctypes.c_void_p(None)
        _check(lib().bsa_plan_create(ctypes.byref(prob), None if hs is None else hs.ctypes.data,
                                     ctypes.byref(handle)))
        self.handle = handle
        nq, nkv = ctypes.c_int32(0), ctypes.c_int32(0)
        wss, wsc, wsb, wsf = (ctypes.c_size_t(0) for _ in range(4))
        _check(lib().bsa_plan_info(handle, ctypes.byref(nq), ctypes.byref(nkv), ctypes.byref(wss),
                                   ctypes.byref(wsc), ctypes.byref(wsb), ctypes.byref(wsf)))
        self.nq, self.nkv = nq.value, nkv.value
        self.ws_select, self.ws_calib, self.ws_bwd = wss.value, wsc.value, wsb.value
        self.ws_fwd = wsf.value

    def blocks(self, which: int) -> Tuple[np.ndarray, np.ndarray]:
        nb = self.nq if which == 0 else self.nkv
        perm = np.empty(self.N, np.int32)
        start = np.empty(nb + 1, np.int32)
        _check(lib().bsa_plan_blocks(self.handle, which, perm.ctypes.data, start.ctypes.data))
        return perm, start

    def close(self):
        if getattr(self, "handle", None) is not None and self.handle.value:
            _check(lib().bsa_plan_destroy(self.handle))
            self.handle = ctypes.c_void_p(None)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def bsa_pool(plan: Plan, which: int, X, Xbar, stream=None):
    _check(lib().bsa_pool(plan.handle, which, _ptr(X), _ptr(Xbar), _stream(stream)))


def bsa_pool_qk(plan: Plan, Q, K, Qbar, Kbar, stream=None):
    _check(lib().bsa_pool_qk(plan.handle, _ptr(Q), _ptr(K), _ptr(Qbar), _ptr(Kbar),
                             _stream(stream)))


def bsa_score(plan: Plan, Qbar, Kbar, norm: int, S, stream=None):
    _check(lib().bsa_score(plan.handle, _ptr(Qbar), _ptr(Kbar), norm, _ptr(S), _stream(stream)))


def bsa_calibrate_mass(plan: Plan, Q, K, M, ws, ws_bytes: int, stream=None):
    _check(lib().bsa_calibrate_mass(plan.handle, _ptr(Q), _ptr(K), _ptr(M), _ptr(ws), ws_bytes,
                                    _stream(stream)))


def bsa_calibrate_mass_fwd(plan: Plan, Q, K, V, M, O, lse, ws, ws_bytes: int, stream=None):
    _check(lib().bsa_calibrate_mass_fwd(plan.handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(M), _ptr(O),
                                        _ptr(lse), _ptr(ws), ws_bytes, _stream(stream)))


def bsa_select(plan: Plan, S, p: float, pool: int, min_k_mode: int, fixed_k: int, row_ptr,
               col_idx, col_cap: int, counts, head_k, ws, ws_bytes: int, stream=None):
    prm = SelectParams(float(p), int(pool), int(min_k_mode), int(fixed_k))
    _check(lib().bsa_select(plan.handle, _ptr(S), ctypes.byref(prm), _ptr(row_ptr),
                            _ptr(col_idx), int(col_cap), _ptr(counts), _ptr(head_k), _ptr(ws),
                            ws_bytes, _stream(stream)))


def bsa_score_select(plan: Plan, Qbar, Kbar, p: float, min_k_mode: int, fixed_k: int, S,
                     row_ptr, col_idx, col_cap: int, counts, head_k, ws, ws_bytes: int,
                     stream=None):
    prm = SelectParams(float(p), BSA_POOL_ROW, int(min_k_mode), int(fixed_k))
    _check(lib().bsa_score_select(plan.handle, _ptr(Qbar), _ptr(Kbar), ctypes.byref(prm),
                                  _ptr(S), _ptr(row_ptr), _ptr(col_idx), int(col_cap),
                                  _ptr(counts), _ptr(head_k), _ptr(ws), ws_bytes,
                                  _stream(stream)))


def bsa_select_noalloc(plan: Plan, S, p: float, pool: int, min_k_mode: int, fixed_k: int,
                       row_ptr, col_idx, col_cap: int, counts, head_k, stream=None):
    prm = SelectParams(float(p), int(pool), int(min_k_mode), int(fixed_k))
    _check(lib().bsa_select_noalloc(plan.handle, _ptr(S), ctypes.byref(prm), _ptr(row_ptr),
                                    _ptr(col_idx), int(col_cap), _ptr(counts), _ptr(head_k),
                                    _stream(stream)))


def bsa_select_eg(plan: Plan, S, p: float, theta: float, group_size: int, row_ptr, col_idx,
                  col_cap: int, counts, head_entropy, head_pooled, ws, ws_bytes: int,
                  stream=None):
    prm = EgParams(float(p), float(theta), int(group_size))
    _check(lib().bsa_select_eg(plan.handle, _ptr(S), ctypes.byref(prm), _ptr(row_ptr),
                               _ptr(col_idx), int(col_cap), _ptr(counts), _ptr(head_entropy),
                               _ptr(head_pooled), _ptr(ws), ws_bytes, _stream(stream)))


def bsa_tokens_ws(plan: Plan) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().bsa_tokens_ws(plan.handle, ctypes.byref(n)))
    return int(n.value)


def bsa_select_tokens(plan: Plan, Q, Kbar, k: int, sel, row_ptr, col_idx, col_cap: int, ws,
                      ws_bytes: int, stream=None):
    _check(lib().bsa_select_tokens(plan.handle, _ptr(Q), _ptr(Kbar), int(k), _ptr(sel),
                                   _ptr(row_ptr), _ptr(col_idx), int(col_cap), _ptr(ws), ws_bytes,
                                   _stream(stream)))


def bsa_attn_fwd_tokens(plan: Plan, Q, K, V, row_ptr, col_idx, sel, k: int, O, lse, ws,
                        ws_bytes: int, stream=None):
    _check(lib().bsa_attn_fwd_tokens(plan.handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(row_ptr),
                                     _ptr(col_idx), _ptr(sel), int(k), _ptr(O), _ptr(lse),
                                     _ptr(ws), ws_bytes, _stream(stream)))


def bsa_tokens_global_ws(plan: Plan) -> int:
    n = ctypes.c_size_t(0)
    _check(lib().bsa_tokens_global_ws(plan.handle, ctypes.byref(n)))
    return int(n.value)


def bsa_select_tokens_global(plan: Plan, Q, Kbar, tau: float, tbits, row_ptr, col_idx,
                             col_cap: int, ws, ws_bytes: int, stream=None):
    _check(lib().bsa_select_tokens_global(plan.handle, _ptr(Q), _ptr(Kbar), float(tau),
                                          _ptr(tbits), _ptr(row_ptr), _ptr(col_idx),
                                          int(col_cap), _ptr(ws), ws_bytes, _stream(stream)))


def bsa_attn_fwd_token_bits(plan: Plan, Q, K, V, row_ptr, col_idx, tbits, O, lse, ws,
                            ws_bytes: int, stream=None):
    _check(lib().bsa_attn_fwd_token_bits(plan.handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(row_ptr),
                                         _ptr(col_idx), _ptr(tbits), _ptr(O), _ptr(lse),
                                         _ptr(ws), ws_bytes, _stream(stream)))


def bsa_probe_mfma(shape: int, workgroups: int, iters: int, sink, stream=None) -> float:
    """Enqueue the bf16 MFMA peak loop (shape 0: 32x32x16, 1: 16x16x32) or, at three
    workgroups per CU, one of the matrix/vector mixes (2: 16x16x32 MFMAs alone, 3: with 32
    exponentials per round, 4: the exponentials alone, 5: MFMAs with 32 FMAs, 6: the FMAs
    alone); returns the FLOPs of its MFMAs."""
    f = ctypes.c_double(0.0)
    _check(lib().bsa_probe_mfma(int(shape), int(workgroups), int(iters), _ptr(sink),
                                ctypes.byref(f), _stream(stream)))
    return f.value


def bsa_probe_copy(src, dst, nbytes: int, stream=None):
    _check(lib().bsa_probe_copy(_ptr(src), _ptr(dst), int(nbytes), _stream(stream)))


def bsa_attn_fwd(plan: Plan, Q, K, V, row_ptr, col_idx, O, lse, ws, ws_bytes: int, stream=None):
    _check(lib().bsa_attn_fwd(plan.handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(row_ptr),
                              _ptr(col_idx), _ptr(O), _ptr(lse), _ptr(ws), ws_bytes,
                              _stream(stream)))


def bsa_attn_bwd(plan: Plan, Q, K, V, O, dO, lse, row_ptr, col_idx, dQ, dK, dV, ws,
                 ws_bytes: int, stream=None):
    _check(lib().bsa_attn_bwd(plan.handle, _ptr(Q), _ptr(K), _ptr(V), _ptr(O), _ptr(dO),
                              _ptr(lse), _ptr(row_ptr), _ptr(col_idx), _ptr(dQ), _ptr(dK),
                              _ptr(dV), _ptr(ws), ws_bytes, _stream(stream)))
