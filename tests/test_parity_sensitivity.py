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
or end of the context must fail it.  A second group of checks, at a wide
score spread, shows the same bar separating the kernels' fp32 score scaling
from a cheaper bf16 one.  Nothing here touches the GPU path.
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


# ---------------------------------------------------------------------------
# Wide score spread.  With q and K at 3 times N(0, 1) (scores with a standard
# deviation of about 9, so a row's softmax sits on a few keys), the bar must
# still hold for the arithmetic the kernels use, scores in fp32 scaled by
# scale * log2(e) in fp32 and exponentiated against the row max, probabilities
# rounded to bf16 for the PV product, and must fail the shortcut of folding
# scale * log2(e) into q before the QK^T product (q * scale rounded to bf16).
# The two are emulated here in numpy on the oracle's own gathered rows: this
# pins what the wide-score GPU parity cases can see.  Softmax as defined in the
# mini-sglang architecture deep dive, section 5.2 (FlashAttention).
# ---------------------------------------------------------------------------

WIDE = 3.0


def _round_bf16(x):
    return bf16_bits_to_float32(float32_to_bf16_bits(np.asarray(x, dtype=np.float32)))


def _emulated_row(q, K, V, scale, fold_scale_into_q):
    c = np.float32(scale * np.log2(np.e))
    q32, K32 = q.astype(np.float32), K.astype(np.float32)
    s = (_round_bf16(q32 * c) @ K32.T) if fold_scale_into_q else (q32 @ K32.T) * c
    p = _round_bf16(np.exp2(s - s.max())).astype(np.float64)
    return (p @ V) / p.sum()


@pytest.fixture(scope="module")
def wide_case():
    w = P.widen_scores(configs.small(2, seed=7), WIDE)
    return w, reference_step(w)


def _emulated_outputs(w, ref, fold):
    pt = ref["meta"]["page_table"]
    G = w.num_qo_heads // w.num_kv_heads
    got, want = [], []
    for i in range(w.num_reqs):
        if w.is_padding[i]:
            continue
        rows = O.gather_rows(pt, int(w.table_idx[i]), int(w.device_len[i]))
        K, V = ref["pool"].gather(rows)
        q = O.widen_bf16(w.q[i])  # decode: request i's one new token is token i
        got.append(as_bf16(np.stack([_emulated_row(q[h], K[:, h // G], V[:, h // G], w.sm_scale, fold)
                                     for h in range(w.num_qo_heads)])))
        want.append(ref["out"][i])
    return np.stack(got), np.stack(want)


def test_wide_scores_are_peaked(wide_case):
    w, ref = wide_case
    q = O.widen_bf16(w.q[0, 0])
    rows = O.gather_rows(ref["meta"]["page_table"], int(w.table_idx[0]), int(w.device_len[0]))
    K, _ = ref["pool"].gather(rows)
    s = K[:, 0, :] @ q * w.sm_scale
    assert s.std() > 6.0  # about 9: a few keys carry each row


def test_wide_scores_fp32_scaling_passes(wide_case):
    w, ref = wide_case
    stats = P.attention_error_stats(*_emulated_outputs(w, ref, fold=False))
    assert not P.bar_failures(stats), stats


def test_wide_scores_scale_folded_into_q_fails(wide_case):
    w, ref = wide_case
    stats = P.attention_error_stats(*_emulated_outputs(w, ref, fold=True))
    assert P.bar_failures(stats), stats
