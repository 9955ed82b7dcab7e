"""The five workloads: shapes, block partitions and selection thresholds.

Shapes follow the video DiT attention calls the pages discuss: Wan2.1-1.3B at 480p has a latent
token grid of 21 x 30 x 52, HunyuanVideo 720p 33 x 45 x 80, Wan2.1-14B at 720p 21 x 45 x 80.
Thresholds: top-p 0.9 for block-mean scoring, 0.99 retained mass for the calibrated selection
(LoSA abstract, scholarbro author page), tau = 0.25 for the head-global pool (VMoBA review,
"Assumptions & free parameters"). Block counts 48 (2D) and 60 (3D) for the cycled kv partitions
follow the VMoBA appendix excerpt quoted in the review's reference list; the 1D temporal block of
3 frames follows the same review's free-parameter list.

A partition is ("flat", s) for contiguous runs of s tokens in frame-major order, or
("tile", (bt, bh, bw)) for 3D tiles clipped at the grid edge.
"""
from dataclasses import dataclass, field
from typing import Optional, Tuple


@dataclass(frozen=True)
class Workload:
    cid: int
    name: str
    B: int
    H: int
    d: int
    dtype: str                      # "fp32" or "bf16"
    grid: Tuple[int, int, int]      # (T, Hg, Wg), frame-major token order
    qpart: tuple
    kvpart: tuple                   # for the cycled workload: the 3D member (layer 2 mod 3)
    p: float                        # top-p threshold (ROW), retained mass, or tau (HEAD)
    mode: str                       # "row", "calib", "hybrid", "head"
    kv_cycle: Optional[tuple] = None  # per-layer kv partitions, chosen by layer index mod 3
    drift_steps: int = 0
    drift_scale: float = 0.0
    temperature: bool = False       # per-head softmax temperature T_h ~ U[0.5, 2]
    backward: bool = False
    smooth: bool = False            # Q/K from a smooth 3D random field plus RoPE
    extras: dict = field(default_factory=dict)

    @property
    def N(self) -> int:
        T, Hg, Wg = self.grid
        return T * Hg * Wg


CONFIGS = {
    1: Workload(1, "tiny-fp32", B=1, H=2, d=64, dtype="fp32", grid=(4, 8, 8),
                qpart=("flat", 32), kvpart=("flat", 32), p=0.9, mode="row"),
    2: Workload(2, "wan2.1-1.3b-480p", B=1, H=12, d=128, dtype="bf16", grid=(21, 30, 52),
                qpart=("tile", (4, 4, 8)), kvpart=("tile", (4, 4, 8)), p=0.9, mode="row",
                smooth=True),
    3: Workload(3, "losa-calibrate-reuse-480p", B=1, H=12, d=128, dtype="bf16",
                grid=(21, 30, 52), qpart=("tile", (4, 4, 8)), kvpart=("tile", (4, 4, 8)),
                p=0.99, mode="calib", drift_steps=10, drift_scale=0.05, temperature=True,
                smooth=True),
    4: Workload(4, "hunyuanvideo-720p-hybrid", B=1, H=24, d=128, dtype="bf16",
                grid=(33, 45, 80), qpart=("tile", (4, 4, 8)), kvpart=("tile", (4, 4, 8)),
                p=0.9, mode="hybrid", smooth=True),
    5: Workload(5, "wan2.1-14b-720p-train", B=1, H=40, d=128, dtype="bf16", grid=(21, 45, 80),
                qpart=("tile", (4, 4, 8)), kvpart=("tile", (7, 9, 20)), p=0.25, mode="head",
                kv_cycle=(("tile", (3, 45, 80)), ("tile", (21, 15, 5)), ("tile", (7, 9, 20))),
                backward=True, smooth=True),
}


def kv_partition_for_layer(w: Workload, layer: int) -> tuple:
    """Layer-wise cyclic 1D/2D/3D kv partition (VMoBA review, "Core claim" and the
    editorial note on the fixed mod-3 schedule): layer l uses member l mod 3."""
    if w.kv_cycle is None:
        return w.kvpart
    return w.kv_cycle[layer % 3]
