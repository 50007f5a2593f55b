"""fp64 CPU oracle for rotary position embedding (+ optional per-head RMS
norm of q and k) fused into the K/V store.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this module.  The GPU library never calls it and
shares no code with it.

What it follows: "mini-sglang architecture deep dive" (tinymind.me),
§7.2 (the attention layer applies the optional q/k RMS norm, then RoPE to q and
k by position, before the backend stores K/V and attends) and §7.3 (RoPE with
rotary_dim equal to head_size and inverse frequencies base^(-2i/rotary_dim),
i = 0 .. rotary_dim/2 - 1, applied in place to q and k by position).

Readings where the pages are silent: the rotation pairs element j with element
j + d/2 (the "rotate half" layout; the pages call the library routine with its
default layout); the angles are exact (pos * theta_i in float64) rather than
taken from a float32 table; the RMS norm is x / sqrt(mean(x^2) + eps) * w per
head, and with the fused store its result is rotated without an intermediate
bf16 rounding.

Parity status: pinned by the tests (complex-exponential form of the rotation,
rotation invariants, torch's rms_norm in float64).  Not "parity unpinned".
"""
from __future__ import annotations

from typing import Dict, Optional, Tuple

import numpy as np

from .pagedkv_oracle import widen_bf16


def inv_freq(d: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/d), i = 0 .. d/2 - 1 (the section 7.3 frequencies)."""
    i = np.arange(d // 2, dtype=np.float64)
    return base ** (-2.0 * i / d)


def rope_rotate(x: np.ndarray, pos: int, base: float) -> np.ndarray:
    """Rotate each pair (x_j, x_{j+d/2}) of the last axis by the angle pos * theta_j."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = float(pos) * inv_freq(d, base)
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def rms_norm(x: np.ndarray, w: np.ndarray, eps: float) -> np.ndarray:
    """x / sqrt(mean(x^2) + eps) * w over the last axis."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x / np.sqrt(ms + eps) * np.asarray(w, dtype=np.float64)


def store_kv_rope(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, out_loc: np.ndarray,
                  positions: np.ndarray, base: float,
                  qk_norm: Optional[Tuple[np.ndarray, np.ndarray, float]] = None
                  ) -> Tuple[np.ndarray, Dict[int, Tuple[np.ndarray, np.ndarray]]]:
    """The fused step on T tokens, explicitly per token.

    Returns (q after norm and rotation, float64 [T, Hq, d]; the written pool
    rows {row: (K float64 [Hkv, d], V bf16 bits [Hkv, d])}, a later token
    winning when two write the same row)."""
    q = widen_bf16(q_bits)
    k = widen_bf16(k_bits)
    q_out = np.empty_like(q)
    rows: Dict[int, Tuple[np.ndarray, np.ndarray]] = {}
    for t in range(q.shape[0]):
        qt, kt = q[t], k[t]
        if qk_norm is not None:
            qw, kw, eps = qk_norm
            qt = rms_norm(qt, widen_bf16(qw), eps)
            kt = rms_norm(kt, widen_bf16(kw), eps)
        q_out[t] = rope_rotate(qt, int(positions[t]), base)
        rows[int(out_loc[t])] = (rope_rotate(kt, int(positions[t]), base), np.array(v_bits[t], dtype=np.uint16))
    return q_out, rows
