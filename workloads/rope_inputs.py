"""Seeded inputs for the fused RoPE store: q, k, v rows, target rows,
positions and per-head norm weights.  Nothing here computes any part of the
rotation or the norm."""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .synth import float32_to_bf16_bits, normal_bf16

# typical model settings: Llama-style base 1e4 (and 5e5 for Llama 3), Qwen3 1e6
ROPE_BASES = (1e4, 5e5, 1e6)
NORM_EPS = 1e-6


@dataclass
class RopeInputs:
    q: np.ndarray          # bf16 bits [T, Hq, d]
    k: np.ndarray          # bf16 bits [T, Hkv, d]
    v: np.ndarray          # bf16 bits [T, Hkv, d]
    out_loc: np.ndarray    # int32 [T], distinct rows in [1, num_pool_rows)
    positions: np.ndarray  # int32 [T] in [0, max_position); includes 0 and max_position - 1
    q_weight: np.ndarray   # bf16 bits [d], values in [0.5, 1.5)
    k_weight: np.ndarray   # bf16 bits [d]
    max_position: int
    num_pool_rows: int


def rope_inputs(seed: int, num_tokens: int, num_qo_heads: int, num_kv_heads: int, head_dim: int = 128,
                num_pool_rows: int = 4096, max_position: int = 32768) -> RopeInputs:
    ss = np.random.SeedSequence(seed)
    c = ss.spawn(5)
    rng = np.random.Generator(np.random.PCG64(c[0]))
    T = num_tokens
    out_loc = (1 + rng.permutation(num_pool_rows - 1)[:T]).astype(np.int32)
    positions = rng.integers(0, max_position, size=T).astype(np.int32)
    if T >= 2:
        positions[0], positions[-1] = 0, max_position - 1
    w = float32_to_bf16_bits(rng.uniform(0.5, 1.5, size=(2, head_dim)).astype(np.float32))
    return RopeInputs(q=normal_bf16(c[1], (T, num_qo_heads, head_dim)), k=normal_bf16(c[2], (T, num_kv_heads, head_dim)),
                      v=normal_bf16(c[3], (T, num_kv_heads, head_dim)), out_loc=out_loc, positions=positions,
                      q_weight=w[0].copy(), k_weight=w[1].copy(), max_position=max_position,
                      num_pool_rows=num_pool_rows)
