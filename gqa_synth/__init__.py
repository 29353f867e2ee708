"""Seeded synthetic inputs for GQA decode: workload shapes and generators.

This package is shared by the GPU path's tests/benchmark and by the CPU oracle's
tests. It holds shapes, seeds and random draws only -- none of the attention
arithmetic (no logits, softmax or weighted sums live here).
"""
from .workloads import Workload, WORKLOADS, BENCH_DEFAULT, BENCH_PER_CONFIG, workload
from .generate import (
    draw_lengths,
    draw_key_scales,
    draw_block_table,
    make_inputs,
    DecodeInputs,
    make_latent_inputs,
    LatentInputs,
)

__all__ = [
    "Workload",
    "WORKLOADS",
    "BENCH_DEFAULT",
    "BENCH_PER_CONFIG",
    "workload",
    "draw_lengths",
    "draw_key_scales",
    "draw_block_table",
    "make_inputs",
    "DecodeInputs",
    "make_latent_inputs",
    "LatentInputs",
]
