"""Seeded synthetic inputs for the KV-selection hot path.

This package only draws and lays out input tensors: keys, values, window and
decode queries, per-layer uncertainty profiles, head-kind assignments, special
token sets and chunk boundaries.  It holds none of the selection or attention
arithmetic; the CPU oracle and the HIP library both consume the bit patterns it
produces (bf16 as uint16 words, fp32 as float32), so input rounding never enters
a parity comparison.
"""
from .configs import CONFIGS, Config, get_config
from .gen import (
    bf16_bits_to_f32,
    f32_to_bf16_bits,
    layer_inputs,
    segment_inputs,
    zigzag_profile,
    head_kinds,
    special_positions,
    chunk_ends,
    step_token,
    step_inputs,
    chunk_step_inputs,
    kept_pairs,
    rope_table,
    HEAD_GLOBAL,
    HEAD_LOCAL,
    HEAD_SPECIAL,
)

__all__ = [
    "CONFIGS", "Config", "get_config", "bf16_bits_to_f32", "f32_to_bf16_bits",
    "layer_inputs", "segment_inputs", "zigzag_profile", "head_kinds",
    "special_positions", "chunk_ends", "step_token", "step_inputs", "chunk_step_inputs", "kept_pairs", "rope_table", "HEAD_GLOBAL", "HEAD_LOCAL", "HEAD_SPECIAL",
]
