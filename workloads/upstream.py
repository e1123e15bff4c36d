"""Inputs of the upstream verify steps: the new rows' q / k / v before RoPE, and the LM head's
hidden states and output weight. Like the rest of this package it only draws numbers.

New rows are N(0, 1) in bfloat16 (the recipe of the cached keys and values). Hidden states are
N(0, 1) and the weight N(0, sigma^2) with sigma = 3 / sqrt(H), so that the logits have the
standard deviation 3 of the 8B logits recipe.
"""

from __future__ import annotations

import numpy as np

from .gen import Preset, _normal_bf16, bf16_bits

# RoPE bases of the model families the workloads are shaped after (Llama-3 8B, Qwen2.5)
ROPE_THETA = {"8b": 500000.0, "tiny": 10000.0, "7b": 1000000.0, "longtail": 500000.0, "262k": 1000000.0}


def make_new_rows(preset: Preset, k: int, seed: int, B: int | None = None) -> dict:
    """q [B][k+1][Hq][D], k_new and v_new [B][k+1][Hkv][D] (bf16 bits), PCG64 seed 9000 + seed."""
    B = preset.B if B is None else B
    rng = np.random.Generator(np.random.PCG64(9000 + seed))
    return dict(q=_normal_bf16(rng, (B, k + 1, preset.Hq, preset.D)),
                k_new=_normal_bf16(rng, (B, k + 1, preset.Hkv, preset.D)),
                v_new=_normal_bf16(rng, (B, k + 1, preset.Hkv, preset.D)))


def make_lm_head_inputs(R: int, H: int, V: int, seed: int) -> dict:
    """hidden [R][H] ~ N(0, 1), weight [V][H] ~ N(0, (3 / sqrt(H))^2), bf16 bits; PCG64 seed 9500 + seed."""
    rng = np.random.Generator(np.random.PCG64(9500 + seed))
    hidden = _normal_bf16(rng, (R, H))
    sigma = np.float32(3.0 / np.sqrt(H))
    weight = np.empty((V, H), dtype=np.uint16)
    step = max(1, (1 << 24) // H)
    for v0 in range(0, V, step):
        v1 = min(V, v0 + step)
        weight[v0:v1] = bf16_bits(rng.standard_normal((v1 - v0, H), dtype=np.float32) * sigma)
    return dict(hidden=hidden, weight=weight)
