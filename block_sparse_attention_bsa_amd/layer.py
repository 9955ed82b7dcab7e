"""One block-sparse attention layer call, built from the C-ABI entry points.

Allocates the block-level buffers, CSR and workspaces with PyTorch on the current device and
calls bsa_pool / bsa_score / bsa_select (or bsa_select_eg) / bsa_attn_fwd (and bsa_calibrate_mass,
bsa_attn_bwd) in order on one stream. No arithmetic happens here.
"""
from __future__ import annotations

from typing import Optional

import torch

from . import (BSA_MINK_NONE, BSA_NORM_HEAD, BSA_NORM_ROW, BSA_POOL_HEAD, BSA_POOL_ROW, Plan,
               bsa_attn_bwd, bsa_attn_fwd, bsa_calibrate_mass, bsa_calibrate_mass_fwd,
               bsa_attn_fwd_tokens, bsa_pool_qk, bsa_score, bsa_score_select, bsa_select,
               bsa_select_eg, bsa_select_tokens, bsa_tokens_ws, bsa_tokens_global_ws,
               bsa_select_tokens_global, bsa_attn_fwd_token_bits)


class BlockSparseAttention:
    def __init__(self, B, H, d, grid, qpart, kvpart, dtype="bf16", head_scale=None,
                 device="cuda"):
        self.plan = Plan(B, H, d, grid, qpart, kvpart, dtype=dtype, head_scale=head_scale)
        p = self.plan
        self.device = torch.device(device)
        f32 = dict(dtype=torch.float32, device=self.device)
        i32 = dict(dtype=torch.int32, device=self.device)
        self.rows = B * H * p.nq
        self.qbar = torch.empty((B, H, p.nq, d), **f32)
        self.kbar = torch.empty((B, H, p.nkv, d), **f32)
        self.S = torch.empty((B, H, p.nq, p.nkv), **f32)
        self.row_ptr = torch.empty(self.rows + 1, **i32)
        self.col_cap = self.rows * p.nkv
        self.col_idx = torch.empty(self.col_cap, **i32)
        self.counts = torch.empty(self.rows, **i32)
        self.head_k = torch.empty(B * H, **i32)
        self.head_entropy = torch.empty(B * H, **f32)
        self.head_pooled = torch.empty(B * H, **i32)
        self.ws_select = torch.empty(max(p.ws_select, 1), dtype=torch.uint8, device=self.device)
        self._ws_calib = None
        self._ws_bwd = None
        self._ws_fwd = None
        self._ws_tok = None
        self.tdtype = torch.bfloat16 if dtype == "bf16" else torch.float32
        self.shape = (B, H, p.N, d)

    # -- argument checks (the C ABI sees only pointers) -----------------------------------------
    def _act(self, name, t):
        """A [B, H, N, d] activation of the plan's dtype, contiguous, on the layer's device."""
        if t is None:
            return t
        if tuple(t.shape) != self.shape:
            raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {self.shape}")
        if t.dtype != self.tdtype:
            raise TypeError(f"{name}: dtype {t.dtype}, expected {self.tdtype}")
        if not t.is_contiguous():
            raise ValueError(f"{name}: must be contiguous ([B, H, N, d], d fastest)")
        if t.device != self._dev():
            raise ValueError(f"{name}: on {t.device}, the layer is on {self._dev()}")
        return t

    def _i32(self, name, t, n=None):
        if t is None:
            return t
        if t.dtype != torch.int32 or not t.is_contiguous() or t.device != self._dev():
            raise TypeError(f"{name}: must be a contiguous int32 tensor on {self._dev()}")
        if n is not None and t.numel() < n:
            raise ValueError(f"{name}: {t.numel()} entries, at least {n} needed")
        return t

    def _f32(self, name, t, shape):
        if t is None:
            return t
        if (tuple(t.shape) != tuple(shape) or t.dtype != torch.float32 or not t.is_contiguous()
                or t.device != self._dev()):
            raise TypeError(f"{name}: must be a contiguous float32 tensor of shape {tuple(shape)} "
                            f"on {self._dev()}")
        return t

    def _dev(self):
        return self.qbar.device

    # -- stages -----------------------------------------------------------------------------
    def pool(self, q, k, stream=None):
        self._act("q", q), self._act("k", k)
        bsa_pool_qk(self.plan, q, k, self.qbar, self.kbar, stream)

    def score(self, norm=BSA_NORM_ROW, stream=None):
        bsa_score(self.plan, self.qbar, self.kbar, norm, self.S, stream)
        return self.S

    def calibrate(self, q, k, stream=None):
        self._act("q", q), self._act("k", k)
        if self._ws_calib is None:
            self._ws_calib = torch.empty(self.plan.ws_calib, dtype=torch.uint8, device=self.device)
        bsa_calibrate_mass(self.plan, q, k, self.S, self._ws_calib, self.plan.ws_calib, stream)
        return self.S

    def calibrate_attention(self, q, k, v, out=None, lse=None, stream=None):
        """The dense step: exact block masses into self.S and the dense attention output."""
        if self._ws_calib is None:
            self._ws_calib = torch.empty(self.plan.ws_calib, dtype=torch.uint8, device=self.device)
        self._act("q", q), self._act("k", k), self._act("v", v)
        if out is None:
            out = torch.empty_like(q)
        self._act("out", out), self._f32("lse", lse, self.shape[:3])
        bsa_calibrate_mass_fwd(self.plan, q, k, v, self.S, out, lse, self._ws_calib,
                               self.plan.ws_calib, stream)
        return self.S, out

    def select(self, p, pool=BSA_POOL_ROW, min_k_mode=BSA_MINK_NONE, fixed_k=0, stream=None,
               scores=None):
        bsa_select(self.plan, self.S if scores is None else scores, p, pool, min_k_mode, fixed_k,
                   self.row_ptr, self.col_idx, self.col_cap, self.counts, self.head_k,
                   self.ws_select, self.plan.ws_select, stream)
        return self.row_ptr, self.col_idx

    def score_select(self, p, min_k_mode=BSA_MINK_NONE, fixed_k=0, stream=None, write_scores=None):
        """Scores and ROW-pool selection in one pass from the pooled Q and K (pool() first). The
        scores go to self.S only when asked (write_scores) or when a minimum count needs them."""
        if write_scores is None:
            write_scores = min_k_mode != BSA_MINK_NONE
        bsa_score_select(self.plan, self.qbar, self.kbar, p, min_k_mode, fixed_k,
                         self.S if write_scores else None, self.row_ptr, self.col_idx,
                         self.col_cap, self.counts, self.head_k, self.ws_select,
                         self.plan.ws_select, stream)
        return self.row_ptr, self.col_idx

    def select_eg(self, p, theta, group_size, stream=None, scores=None):
        """Entropy-routed selection from the row-normalised scores (score(BSA_NORM_ROW) first);
        fills head_entropy and head_pooled too."""
        bsa_select_eg(self.plan, self.S if scores is None else scores, p, theta, group_size,
                      self.row_ptr, self.col_idx, self.col_cap, self.counts, self.head_entropy,
                      self.head_pooled, self.ws_select, self.plan.ws_select, stream)
        return self.row_ptr, self.col_idx

    def select_tokens(self, q, k_best, stream=None):
        """Per-token Local + TopK from Q and the pooled K (pool() first): returns sel
        [B, H, N, 1 + min(k, nkv - 1)] and fills row_ptr / col_idx with each query block's
        union."""
        self._act("q", q)
        B, H, N = q.shape[:3]
        ns = 1 + min(int(k_best), self.plan.nkv - 1)
        sel = torch.empty((B, H, N, ns), dtype=torch.int32, device=self.device)
        n = bsa_tokens_ws(self.plan)
        if self._ws_tok is None or self._ws_tok.numel() < n:
            self._ws_tok = torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)
        bsa_select_tokens(self.plan, q, self.kbar, k_best, sel, self.row_ptr, self.col_idx,
                          self.col_cap, self._ws_tok, self._ws_tok.numel(), stream)
        return sel

    def attention_tokens(self, q, k, v, sel, k_best, out=None, lse=None, with_lse=True,
                         stream=None):
        """Attention of every token over its own blocks (sel from select_tokens)."""
        self._act("q", q), self._act("k", k), self._act("v", v)
        ns = 1 + min(int(k_best), self.plan.nkv - 1)
        self._i32("sel", sel, q.shape[0] * q.shape[1] * q.shape[2] * ns)
        if out is None:
            out = torch.empty_like(q)
        if lse is None and with_lse:
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=self.device)
        self._act("out", out), self._f32("lse", lse, self.shape[:3])
        if self._ws_fwd is None and self.plan.ws_fwd > 0:
            self._ws_fwd = torch.empty(self.plan.ws_fwd, dtype=torch.uint8, device=self.device)
        bsa_attn_fwd_tokens(self.plan, q, k, v, self.row_ptr, self.col_idx, sel, k_best, out,
                            lse, self._ws_fwd, self.plan.ws_fwd, stream)
        return out, lse

    def select_tokens_global(self, q, tau, stream=None):
        """Per-token head-global selection from Q and the pooled K (pool() first): returns the
        per-token block bitmaps [B, H, N, ceil(nkv / 32)] (int32 words) and fills row_ptr /
        col_idx with each query block's union."""
        self._act("q", q)
        B, H, N = q.shape[:3]
        nw = (self.plan.nkv + 31) // 32
        bits = torch.empty((B, H, N, nw), dtype=torch.int32, device=self.device)
        n = bsa_tokens_global_ws(self.plan)
        if getattr(self, "_ws_tg", None) is None or self._ws_tg.numel() < n:
            self._ws_tg = torch.empty(max(n, 1), dtype=torch.uint8, device=self.device)
        bsa_select_tokens_global(self.plan, q, self.kbar, tau, bits, self.row_ptr, self.col_idx,
                                 self.col_cap, self._ws_tg, self._ws_tg.numel(), stream)
        return bits

    def attention_token_bits(self, q, k, v, bits, out=None, lse=None, with_lse=True,
                             stream=None):
        """Attention of every token over the blocks of its bitmap (from select_tokens_global)."""
        self._act("q", q), self._act("k", k), self._act("v", v)
        nw = (self.plan.nkv + 31) // 32
        self._i32("bits", bits, q.shape[0] * q.shape[1] * q.shape[2] * nw)
        if out is None:
            out = torch.empty_like(q)
        if lse is None and with_lse:
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=self.device)
        self._act("out", out), self._f32("lse", lse, self.shape[:3])
        if self._ws_fwd is None and self.plan.ws_fwd > 0:
            self._ws_fwd = torch.empty(self.plan.ws_fwd, dtype=torch.uint8, device=self.device)
        bsa_attn_fwd_token_bits(self.plan, q, k, v, self.row_ptr, self.col_idx, bits, out, lse,
                                self._ws_fwd, self.plan.ws_fwd, stream)
        return out, lse

    def attention(self, q, k, v, row_ptr=None, col_idx=None, out=None, lse=None, stream=None,
                  with_lse=True):
        """O (and the LSE, unless with_lse is False: then the output-only kernel runs and the
        returned lse is None)."""
        self._act("q", q), self._act("k", k), self._act("v", v)
        self._i32("row_ptr", row_ptr, self.rows + 1), self._i32("col_idx", col_idx)
        if out is None:
            out = torch.empty_like(q)
        if lse is None and with_lse:
            lse = torch.empty(q.shape[:3], dtype=torch.float32, device=self.device)
        self._act("out", out), self._f32("lse", lse, self.shape[:3])
        if self._ws_fwd is None and self.plan.ws_fwd > 0:
            self._ws_fwd = torch.empty(self.plan.ws_fwd, dtype=torch.uint8, device=self.device)
        bsa_attn_fwd(self.plan, q, k, v, self.row_ptr if row_ptr is None else row_ptr,
                     self.col_idx if col_idx is None else col_idx, out, lse, self._ws_fwd,
                     self.plan.ws_fwd, stream)
        return out, lse

    def backward(self, q, k, v, o, do, lse, row_ptr=None, col_idx=None, stream=None):
        for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
            self._act(name, t)
        self._f32("lse", lse, self.shape[:3])
        self._i32("row_ptr", row_ptr, self.rows + 1), self._i32("col_idx", col_idx)
        if self._ws_bwd is None:
            self._ws_bwd = torch.empty(self.plan.ws_bwd, dtype=torch.uint8, device=self.device)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        bsa_attn_bwd(self.plan, q, k, v, o, do, lse, self.row_ptr if row_ptr is None else row_ptr,
                     self.col_idx if col_idx is None else col_idx, dq, dk, dv, self._ws_bwd,
                     self.plan.ws_bwd, stream)
        return dq, dk, dv

    # -- whole layer ---------------------------------------------------------------------------
    def forward(self, q, k, v, p, mode="row", min_k_mode=BSA_MINK_NONE, out=None, lse=None,
                stream=None, with_lse=True):
        """pool(Q), pool(K), score, select, sparse attention. mode: 'row' or 'head'."""
        self.pool(q, k, stream)
        self.score(BSA_NORM_HEAD if mode == "head" else BSA_NORM_ROW, stream)
        self.select(p, BSA_POOL_HEAD if mode == "head" else BSA_POOL_ROW, min_k_mode,
                    stream=stream)
        return self.attention(q, k, v, out=out, lse=lse, stream=stream, with_lse=with_lse)

    def csr_host(self):
        rp = self.row_ptr.cpu().numpy()
        return rp, self.col_idx[: int(rp[-1])].cpu().numpy()
