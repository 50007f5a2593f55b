"""Pins for the RoPE / qk-norm oracle (oracle/rope_oracle.py), none of which
re-types an oracle formula:

* the frequencies are the geometric sequence that starts at 1 and reaches
  1/base after d/2 steps (closed form, checked through ratios);
* the rotation equals multiplying z_j = x_j + i x_{j+d/2} by exp(i pos theta_j)
  in numpy complex arithmetic (a second formulation);
* rotation invariants: position 0 is the identity, pair norms are kept,
  rotations compose additively, and scores depend only on the position
  difference;
* RMS norm against torch.nn.functional.rms_norm in float64 (a library routine);
* the fused store on hand-built rows whose expected values are closed forms.
"""
from __future__ import annotations

import numpy as np
import torch

import oracle.rope_oracle as R
from workloads import float32_to_bf16_bits

D = 128


def _rng(seed=0):
    return np.random.default_rng(seed)


def pin_frequencies_geometric():
    for base in (1e4, 1e6, 5e5):
        f = R.inv_freq(D, base)
        assert f.shape == (D // 2,)
        assert f[0] == 1.0
        r = f[1:] / f[:-1]
        assert np.allclose(r, r[0], rtol=1e-13, atol=0)
        assert np.isclose(r[0] ** (D // 2), 1.0 / base, rtol=1e-11)


def pin_complex_form():
    rng = _rng(1)
    x = rng.normal(size=(3, D))
    for base in (1e4, 1e6):
        f = R.inv_freq(D, base)
        for pos in (0, 1, 7, 1000, 32767):
            z = (x[:, : D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * pos * f)
            want = np.concatenate([z.real, z.imag], axis=-1)
            assert np.allclose(R.rope_rotate(x, pos, base), want, rtol=0, atol=1e-12)


def pin_rotation_invariants():
    rng = _rng(2)
    q, k = rng.normal(size=D), rng.normal(size=D)
    base = 1e4
    assert np.array_equal(R.rope_rotate(q, 0, base), q)
    y = R.rope_rotate(q, 123, base)
    pair = lambda v: v[: D // 2] ** 2 + v[D // 2:] ** 2
    assert np.allclose(pair(y), pair(q), rtol=1e-12)
    assert np.allclose(R.rope_rotate(R.rope_rotate(q, 40, base), 2, base), R.rope_rotate(q, 42, base), atol=1e-12)
    s1 = R.rope_rotate(q, 50, base) @ R.rope_rotate(k, 20, base)
    s2 = R.rope_rotate(q, 1050, base) @ R.rope_rotate(k, 1020, base)
    assert np.isclose(s1, s2, rtol=1e-9, atol=1e-9)
    s3 = R.rope_rotate(q, 51, base) @ R.rope_rotate(k, 20, base)
    assert not np.isclose(s1, s3, rtol=1e-6)


def pin_rms_norm_library():
    rng = _rng(3)
    x = rng.normal(size=(5, D)) * 3.0
    w = rng.normal(size=D)
    for eps in (1e-6, 1e-2):
        want = torch.nn.functional.rms_norm(torch.from_numpy(x), (D,), torch.from_numpy(w), eps).numpy()
        assert np.allclose(R.rms_norm(x, w, eps), want, rtol=1e-12, atol=1e-12)


def _bits(a):
    return float32_to_bf16_bits(np.asarray(a, dtype=np.float32))


def pin_store_closed_forms():
    """Rows of equal values 2.0 have RMS 2, so with eps = 0 the norm turns them
    into the weights; position 0 leaves them unrotated, position p rotates the
    weights (complex form).  V rows are copied bit for bit; a later token wins a
    shared row."""
    rng = _rng(4)
    T, hq, hkv, base = 3, 2, 1, 1e4
    q = _bits(np.full((T, hq, D), 2.0))
    k = _bits(np.full((T, hkv, D), 2.0))
    v = _bits(rng.normal(size=(T, hkv, D)))
    qw = _bits(rng.uniform(0.5, 1.5, size=D))
    kw = _bits(rng.uniform(0.5, 1.5, size=D))
    out_loc = np.array([5, 9, 5], dtype=np.int32)
    positions = np.array([0, 17, 300], dtype=np.int32)
    q_out, rows = R.store_kv_rope(q, k, v, out_loc, positions, base, (qw, kw, 0.0))
    f = R.inv_freq(D, base)

    def rot(w_bits, pos):
        w = (w_bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
        z = (w[: D // 2] + 1j * w[D // 2:]) * np.exp(1j * pos * f)
        return np.concatenate([z.real, z.imag])

    for t in range(T):
        for h in range(hq):
            assert np.allclose(q_out[t, h], rot(qw, positions[t]), atol=1e-12)
    assert sorted(rows) == [5, 9]
    assert np.allclose(rows[9][0][0], rot(kw, 17), atol=1e-12)
    assert np.allclose(rows[5][0][0], rot(kw, 300), atol=1e-12)  # the later token won row 5
    assert np.array_equal(rows[5][1], v[2]) and np.array_equal(rows[9][1], v[1])
    # without the norm: the rotation of the raw rows
    q_out2, rows2 = R.store_kv_rope(q, k, v, out_loc, positions, base, None)
    z = (2.0 + 2.0j) * np.exp(1j * 17 * f)
    assert np.allclose(rows2[9][0][0], np.concatenate([z.real, z.imag]), atol=1e-12)


ALL_PINS = [pin_frequencies_geometric, pin_complex_form, pin_rotation_invariants, pin_rms_norm_library,
            pin_store_closed_forms]
