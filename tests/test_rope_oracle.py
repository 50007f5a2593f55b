"""CPU tests: the RoPE / qk-norm oracle against its pins, and the pins against
planted mistakes in that oracle."""
import numpy as np
import pytest

import oracle.rope_oracle as R
from tests import rope_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_rope_oracle_pin(pin):
    pin()


_orig_rotate = R.rope_rotate
_orig_norm = R.rms_norm
_orig_freq = R.inv_freq


def _rotate_sin_sign(x, pos, base):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = pos * R.inv_freq(d, base)
    x1, x2 = x[..., : d // 2], x[..., d // 2:]
    return np.concatenate([x1 * np.cos(a) + x2 * np.sin(a), x2 * np.cos(a) - x1 * np.sin(a)], axis=-1)


def _rotate_interleaved(x, pos, base):
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    a = pos * R.inv_freq(d, base)
    out = x.copy()
    out[..., 0::2] = x[..., 0::2] * np.cos(a) - x[..., 1::2] * np.sin(a)
    out[..., 1::2] = x[..., 1::2] * np.cos(a) + x[..., 0::2] * np.sin(a)
    return out


def _store_rotate_then_norm(q_bits, k_bits, v_bits, out_loc, positions, base, qk_norm=None):
    if qk_norm is None:
        return _orig_store(q_bits, k_bits, v_bits, out_loc, positions, base, None)
    qw, kw, eps = qk_norm
    q = R.widen_bf16(q_bits)
    k = R.widen_bf16(k_bits)
    q_out = np.empty_like(q)
    rows = {}
    for t in range(q.shape[0]):
        q_out[t] = _orig_norm(_orig_rotate(q[t], int(positions[t]), base), R.widen_bf16(qw), eps)
        rows[int(out_loc[t])] = (_orig_norm(_orig_rotate(k[t], int(positions[t]), base), R.widen_bf16(kw), eps),
                                 np.array(v_bits[t], dtype=np.uint16))
    return q_out, rows


_orig_store = R.store_kv_rope

MUTANTS = {
    "sin_sign": ("rope_rotate", _rotate_sin_sign),
    "interleaved_pairs": ("rope_rotate", _rotate_interleaved),
    "angle_off_by_one": ("rope_rotate", lambda x, pos, base: _orig_rotate(x, pos + 1, base)),
    "freq_half_exponent": ("inv_freq", lambda d, base: base ** (-np.arange(d // 2, dtype=np.float64) / d)),
    "freq_reversed": ("inv_freq", lambda d, base: _orig_freq(d, base)[::-1].copy()),
    "norm_sum_not_mean": ("rms_norm", lambda x, w, eps: np.asarray(x) / np.sqrt(np.sum(np.asarray(x) ** 2, -1, keepdims=True) + eps) * w),
    "norm_no_weight": ("rms_norm", lambda x, w, eps: _orig_norm(x, np.ones_like(np.asarray(w, dtype=np.float64)), eps)),
    "norm_eps_outside": ("rms_norm", lambda x, w, eps: np.asarray(x) / (np.sqrt(np.mean(np.asarray(x) ** 2, -1, keepdims=True)) + eps) * w),
    "rotate_then_norm": ("store_kv_rope", _store_rotate_then_norm),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_rope_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(R, attr, fn)
    failed = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(pin.__name__)
    assert failed, f"planted mistake {name} passed every pin"
