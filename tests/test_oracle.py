"""CPU tests: the fp64 oracle against its pins, and the pins against planted
mistakes in the oracle (so a plausible slip in it cannot pass unnoticed)."""
import numpy as np
import pytest

import oracle.pagedkv_oracle as O
from tests import oracle_pins as P


@pytest.mark.parametrize("pin", P.ALL_PINS, ids=lambda f: f.__name__)
def test_oracle_pin(pin):
    pin()


def _fails_some_pin():
    failed = []
    for pin in P.ALL_PINS:
        try:
            with np.errstate(all="ignore"):
                pin()
        except Exception:  # noqa: BLE001 - any failure of a pin counts
            failed.append(pin.__name__)
    return failed


def _store_first_wins(pool, k_new_bits, v_new_bits, out_loc):
    out = pool.copy()
    seen = set()
    for t in range(len(out_loc)):
        if int(out_loc[t]) in seen:
            continue
        seen.add(int(out_loc[t]))
        out.write_row(int(out_loc[t]), k_new_bits[t], v_new_bits[t])
    return out


_orig_gather = O.gather_rows
_orig_build = O.build_metadata

MUTANTS = {
    "gqa_modulo": ("kv_head_of", lambda h, group: h % group),
    "gqa_times": ("kv_head_of", lambda h, group: min(h * group, 0) if group > 1 else h),
    "causal_excludes_self": ("keys_visible", lambda c, t: c + t),
    "causal_one_past": ("keys_visible", lambda c, t: c + t + 2),
    "causal_ignores_prefix": ("keys_visible", lambda c, t: t + 1),
    "no_scale": ("scores", lambda q, K, scale: K @ q),
    "scale_squared": ("scores", lambda q, K, scale: (K @ q) * scale * scale),
    "softmax_no_shift": ("softmax", lambda s: np.exp(s) / np.sum(np.exp(s))),
    "softmax_by_max": ("softmax", lambda s: np.exp(s - s.max()) / np.max(np.exp(s - s.max()))),
    "mix_reversed": ("mix", lambda p, V: p @ V[::-1]),
    "mix_transposed_weights": ("mix", lambda p, V: p[::-1] @ V),
    "gather_shifted": ("gather_rows", lambda pt, r, n: [int(pt[r, j + 1]) for j in range(n)]),
    "gather_wrong_row": ("gather_rows", lambda pt, r, n: _orig_gather(pt, (r + 1) % pt.shape[0], n)),
    "pages_floor": ("pages_needed", lambda n, s: int(n) // int(s)),
    "store_first_wins": ("store_kv", _store_first_wins),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_planted_mistake(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(O, attr, fn)
    if attr == "store_kv":
        import oracle.run as R
        monkeypatch.setattr(R, "store_kv", fn)
    failed = _fails_some_pin()
    assert failed, f"planted mistake {name} passed every pin"
