"""CPU check that the attention bar can see a lost key tile at long context.

With N(0,1) inputs the outputs of a 16K-32K-key decode are small (|o| up to
about 0.06), so a kernel that drops one 32-key tile of a split, or counts one
twice, moves them by only a few 1e-3: inside the absolute bar (max-abs 2e-2,
mean-abs 2e-3).  The relative bounds of tests/parity_checks.py are meant to
close that gap.  Here, at the long-decode shape (64 query / 8 KV heads, head
dim 128, contexts drawn from the long-decode range), the fp64 oracle's own
output rounded to bf16 (what a correct kernel returns at best) must pass the
whole bar with a wide margin, while the oracle run with one 32-key tile
removed from, or repeated in, a request's page-table row at the start, middle
or end of the context must fail it.  Nothing here touches the GPU path.
"""
import numpy as np
import pytest

import oracle.pagedkv_oracle as O
from oracle.run import reference_step
from tests import parity_checks as P
from workloads import configs
from workloads.synth import bf16_bits_to_float32, float32_to_bf16_bits

TILE = 32


@pytest.fixture(scope="module")
def long_case():
    # two requests with contexts from the long-decode range; only the rows the
    # requests use are drawn, so a small pool holds them
    w = configs.long_decode(seed=77, batch=2, num_pool_rows=1 << 17)
    ref = reference_step(w)
    return w, ref


def as_bf16(x: np.ndarray) -> np.ndarray:
    """fp64 -> nearest bf16 (through float32), widened back to fp64."""
    return bf16_bits_to_float32(float32_to_bf16_bits(x.astype(np.float32))).astype(np.float64)


def tampered_output(w, ref, i, k0, mode):
    """Request i's decode output with keys [k0, k0 + 32) of its page-table row
    removed ("drop") or visited twice ("repeat")."""
    pt = ref["meta"]["page_table"].copy()
    r = int(w.table_idx[i])
    dl = int(w.device_len[i])
    row = pt[r, :dl].copy()
    if mode == "drop":
        rows = np.r_[row[:k0], row[k0 + TILE:]]
    else:
        rows = np.r_[row[:k0 + TILE], row[k0:k0 + TILE], row[k0 + TILE:]]
    wide = np.zeros((pt.shape[0], max(pt.shape[1], rows.size)), dtype=pt.dtype)
    wide[:, :pt.shape[1]] = pt
    wide[r, :rows.size] = rows
    return O.attend_token(ref["pool"], wide, r, rows.size, w.q[i], w.num_kv_heads, w.sm_scale)


def test_long_context_outputs_are_small(long_case):
    w, ref = long_case
    assert int(w.device_len.min()) > 16384
    top = max(np.abs(ref["out"][i]).max() for i in range(w.num_reqs))
    assert top < 0.1  # so an absolute bar of 2e-2 is 20% of the largest output or more


def test_correct_rounding_passes_with_margin(long_case):
    w, ref = long_case
    for i in range(w.num_reqs):
        want = ref["out"][i][None]
        stats = P.attention_error_stats(as_bf16(want), want)
        assert not P.bar_failures(stats)
        assert stats["rel_max"] <= P.REL_MAX_TOL / 4 and stats["row_rel_max"] <= P.ROW_REL_TOL / 4, stats


@pytest.mark.parametrize("mode", ["drop", "repeat"])
@pytest.mark.parametrize("where", ["first", "middle", "last"])
def test_lost_or_doubled_tile_fails_the_bar(long_case, mode, where):
    w, ref = long_case
    for i in range(w.num_reqs):
        dl = int(w.device_len[i])
        k0 = {"first": 0, "middle": TILE * ((dl // 2) // TILE), "last": TILE * ((dl - 1) // TILE) - TILE}[where]
        want = ref["out"][i][None]
        got = as_bf16(tampered_output(w, ref, i, k0, mode))[None]
        stats = P.attention_error_stats(got, want)
        # the absolute bar alone would accept it ...
        assert stats["max_abs"] <= P.MAX_ABS_TOL and stats["mean_abs"] <= P.MEAN_ABS_TOL, stats
        # ... both relative bounds do not
        assert stats["rel_max"] > P.REL_MAX_TOL and stats["row_rel_max"] > P.ROW_REL_TOL, stats
        assert P.bar_failures(stats)
