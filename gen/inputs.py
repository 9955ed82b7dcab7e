"""Seeded synthetic inputs, generated on the host.

Recipe (one per workload, seeded by ``SeedSequence(1000 * cid)`` spawned in the fixed order
Q, K, V, dO, T_h, Q-drift, K-drift, V-drift):

* tiny fp32 workload: Q, K, V iid N(0, 1) in fp32.
* video workloads: Q and K are, per (batch, head, channel), a 3D Gaussian-smoothed random field over
  the (T, Hg, Wg) token grid (sigma = 2 tokens, truncated at 4 sigma, half-sample reflect at the
  edges), renormalised to unit standard deviation, plus 0.5 * N(0, 1) noise; then a 3D rotary
  position embedding is applied (channels [0, 44) rotate with the frame index, [44, 86) with the
  row, [86, 128) with the column; adjacent channel pairs; base 10000; integer positions from 0).
  V and dO are iid N(0, 1). Everything is built in fp32 and rounded once to bf16 with
  round-to-nearest-even.
* calibrate-then-reuse workload: per-head temperature T_h ~ U[0.5, 2] gives the softmax scale
  1 / (sqrt(d) * T_h); later steps follow a random walk X_s = X_{s-1} + 0.05 * N(0, 1) on an fp32
  master copy, rounded to bf16 at every step.

The pages measure on VBench prompts with pretrained video models; those are not available, and
these tensors stand in for them at the models' attention shapes. Nothing here computes any part
of block-sparse attention.
"""
from __future__ import annotations

import numpy as np
import torch

from .configs import Workload

_STREAMS = ("q", "k", "v", "do", "temp", "dq_drift", "dk_drift", "dv_drift")


def _streams(cid: int) -> dict:
    ss = np.random.SeedSequence(1000 * cid)
    return dict(zip(_STREAMS, ss.spawn(len(_STREAMS))))


# ---------------------------------------------------------------------------------------------
# bf16 bit handling (round-to-nearest-even), shared by every consumer of the inputs
# ---------------------------------------------------------------------------------------------

def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest, ties to even) and return the raw 16-bit words."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32)


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bits).astype(np.float64)


# ---------------------------------------------------------------------------------------------
# Smooth 3D random field and rotary embedding (input synthesis only)
# ---------------------------------------------------------------------------------------------

def _reflect_index(n: int, radius: int) -> np.ndarray:
    """Half-sample symmetric extension of [0, n) by `radius` on each side."""
    i = np.arange(-radius, n + radius)
    period = 2 * n
    i = np.mod(i, period)
    return np.where(i >= n, period - 1 - i, i)


def _gauss_taps(sigma: float = 2.0, truncate: float = 4.0) -> np.ndarray:
    radius = int(truncate * sigma + 0.5)
    k = np.arange(-radius, radius + 1, dtype=np.float64)
    w = np.exp(-0.5 * (k / sigma) ** 2)
    return (w / w.sum()).astype(np.float32)


def _smooth_axis(x: torch.Tensor, axis: int, taps: np.ndarray) -> torch.Tensor:
    r = (len(taps) - 1) // 2
    n = x.shape[axis]
    idx = torch.from_numpy(_reflect_index(n, r))
    padded = x.index_select(axis, idx)
    out = torch.zeros_like(x)
    for k, wk in enumerate(taps):
        out.add_(padded.narrow(axis, k, n), alpha=float(wk))
    return out


def _smooth_field(rng: np.random.Generator, grid, d: int) -> np.ndarray:
    """One (T, Hg, Wg, d) block of independent per-channel smooth fields, unit std each."""
    T, Hg, Wg = grid
    z = torch.from_numpy(rng.standard_normal((T, Hg, Wg, d), dtype=np.float32))
    taps = _gauss_taps()
    for axis in range(3):
        z = _smooth_axis(z, axis, taps)
    std = z.reshape(-1, d).to(torch.float64).std(dim=0, unbiased=False).to(torch.float32)
    noise = torch.from_numpy(rng.standard_normal((T, Hg, Wg, d), dtype=np.float32))
    return (z / std).add_(noise, alpha=0.5).numpy()


def _rope_tables(grid, d: int):
    """cos/sin tables per token for the 3D rotary embedding, split 44/42/42 for d = 128."""
    T, Hg, Wg = grid
    if d == 128:
        seg = (44, 42, 42)
    else:  # generic split: as equal as possible, each even
        a = (d // 3) // 2 * 2
        seg = (d - 2 * a, a, a)
    tt, hh, ww = np.meshgrid(np.arange(T), np.arange(Hg), np.arange(Wg), indexing="ij")
    pos = [tt.reshape(-1), hh.reshape(-1), ww.reshape(-1)]
    cos = np.empty((T * Hg * Wg, d // 2), np.float64)
    sin = np.empty_like(cos)
    col = 0
    for axis, L in enumerate(seg):
        k = np.arange(L // 2, dtype=np.float64)
        theta = 10000.0 ** (-2.0 * k / L)
        ang = pos[axis][:, None].astype(np.float64) * theta[None, :]
        cos[:, col:col + L // 2] = np.cos(ang)
        sin[:, col:col + L // 2] = np.sin(ang)
        col += L // 2
    return cos.astype(np.float32), sin.astype(np.float32)


def _apply_rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray) -> np.ndarray:
    """x: (N, d) fp32; rotates adjacent pairs (2k, 2k+1)."""
    xt = torch.from_numpy(np.ascontiguousarray(x)).view(x.shape[0], -1, 2)
    c, s = torch.from_numpy(cos), torch.from_numpy(sin)
    x0, x1 = xt[..., 0], xt[..., 1]
    out = torch.stack((x0 * c - x1 * s, x0 * s + x1 * c), dim=-1)
    return out.reshape(x.shape).numpy()


# ---------------------------------------------------------------------------------------------
# Public generators
# ---------------------------------------------------------------------------------------------

def iid_normal(seed_seq, shape) -> np.ndarray:
    rng = np.random.default_rng(seed_seq)
    return rng.standard_normal(shape, dtype=np.float32)


def _smooth_tensor(seed_seq, w: Workload) -> np.ndarray:
    rng = np.random.default_rng(seed_seq)
    cos, sin = _rope_tables(w.grid, w.d)
    out = np.empty((w.B, w.H, w.N, w.d), np.float32)
    for b in range(w.B):
        for h in range(w.H):
            f = _smooth_field(rng, w.grid, w.d).reshape(w.N, w.d)
            out[b, h] = _apply_rope(f, cos, sin)
    return out


def make_inputs(w: Workload, tensors=("q", "k", "v"), grid_override=None, heads_override=None):
    """Inputs of workload `w` as a dict.

    Each tensor is [B, H, N, d]: raw bf16 words (uint16) for bf16 workloads, fp32 otherwise.
    Also returns 'head_scale' (fp32 [H]) and, for bf16 workloads, 'q32'/'k32'/'v32' fp32 masters
    when the workload drifts. `grid_override` / `heads_override` shrink a workload for fast tests
    while keeping its recipe.
    """
    if grid_override is not None or heads_override is not None:
        from dataclasses import replace
        w = replace(w, grid=tuple(grid_override or w.grid), H=int(heads_override or w.H))
    st = _streams(w.cid)
    out = {"workload": w}
    shape = (w.B, w.H, w.N, w.d)
    for name in tensors:
        if name in ("q", "k") and w.smooth:
            x = _smooth_tensor(st[name], w)
        else:
            x = iid_normal(st[name], shape)
        if w.dtype == "bf16":
            if w.drift_steps:
                out[name + "32"] = x
            out[name] = f32_to_bf16_bits(x)
        else:
            out[name] = x
    if w.temperature:
        rng = np.random.default_rng(st["temp"])
        temp = rng.uniform(0.5, 2.0, size=w.H)
        out["temperature"] = temp
        out["head_scale"] = (1.0 / (np.sqrt(w.d) * temp)).astype(np.float32)
    else:
        out["head_scale"] = np.full(w.H, 1.0 / np.sqrt(w.d), np.float32)
    return out


def drift_step(w: Workload, masters: dict, step: int):
    """Advance the fp32 masters by one random-walk step (step >= 1) and return bf16 words.

    X_s = X_{s-1} + scale * N(0, 1); each of Q, K, V uses its own stream, and step s draws from
    the stream's s-th spawned child so that any step can be regenerated on its own.
    """
    st = _streams(w.cid)
    res = {}
    for name, key in (("q", "dq_drift"), ("k", "dk_drift"), ("v", "dv_drift")):
        child = st[key].spawn(step)[step - 1]
        eps = np.random.default_rng(child).standard_normal(masters[name].shape, dtype=np.float32)
        masters[name] = masters[name] + np.float32(w.drift_scale) * eps
        res[name] = f32_to_bf16_bits(masters[name])
    return res
