"""Seeded synthetic inputs for the block-sparse attention workloads.

This package holds the workload descriptions (shapes, partitions, thresholds) and the seeded
input generators. It is shared by the tests, the benchmark and the oracle's callers, and it holds
none of the method's arithmetic: no pooling, scoring, selection or attention is computed here.
"""
from .configs import CONFIGS, Workload, kv_partition_for_layer  # noqa: F401
from .inputs import (  # noqa: F401
    bf16_bits_to_f64,
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    make_inputs,
    drift_step,
    iid_normal,
)
