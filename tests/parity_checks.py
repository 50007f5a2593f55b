"""Comparison helpers for the GPU parity tests: HIP path vs the fp64 oracle.

Bar (from the build's stated target): store, page table and metadata are
bit-exact; bf16 attention outputs widened to fp64 are within max-abs 2e-2 and
mean-abs 2e-3 of the unrounded fp64 oracle, over real (non-padding) tokens.
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.run import reference_step

MAX_ABS_TOL = 2e-2
MEAN_ABS_TOL = 2e-3


def sample_tokens(w, per_request: int = 12, seed: int = 0):
    """Chunk offsets to check per extend request: both ends, the edges of
    tiles of 16..256 tokens, random."""
    rng = np.random.default_rng(seed)
    out = {}
    for i in range(w.num_decode, w.num_reqs):
        ext = int(w.device_len[i] - w.cached_len[i])
        cand = {0, 1, ext - 1, ext - 2, ext // 2}
        cand |= {e + d for e in (16, 32, 64, 128, 256) for d in (-1, 0)}
        cand |= set(int(x) for x in rng.integers(0, ext, size=per_request))
        out[i] = sorted(t for t in cand if 0 <= t < ext)
    return out


def token_starts(w):
    ext = w.device_len.astype(np.int64) - w.cached_len
    return np.concatenate([[0], np.cumsum(ext)])


def check_metadata(ds, ref, w):
    m = ref["meta"]
    T = w.num_tokens
    got = lambda t, n: t[:n].cpu().numpy()
    assert np.array_equal(got(ds.meta.out_loc, T), m["out_loc"]), "out_loc"
    assert np.array_equal(got(ds.meta.positions, T), m["positions"]), "positions"
    assert np.array_equal(got(ds.meta.qo_indptr, w.num_reqs + 1), m["qo_indptr"]), "qo_indptr"
    assert np.array_equal(got(ds.meta.kv_indptr, w.num_reqs + 1), m["kv_indptr"]), "kv_indptr"
    assert np.array_equal(got(ds.meta.last_indices, w.num_reqs), m["last_indices"]), "last_indices"
    assert np.array_equal(ds.page_table.cpu().numpy(), m["page_table"]), "page_table"


def check_store(ds, ref, w, max_untouched: int = 20000, seed: int = 0):
    out_loc = ref["meta"]["out_loc"]
    real_tok = np.ones(w.num_tokens, dtype=bool)
    starts = token_starts(w)
    for i in np.nonzero(w.is_padding)[0]:
        real_tok[starts[i]:starts[i + 1]] = False
    rows = out_loc[real_tok]
    if rows.size:
        k, v = ds.pool_rows_bits(rows)
        assert np.array_equal(k, w.k_new[real_tok]), "stored K rows"
        assert np.array_equal(v, w.v_new[real_tok]), "stored V rows"
    # cached rows untouched
    rng = np.random.default_rng(seed)
    n = w.cached_rows.size
    pick = np.arange(n) if n <= max_untouched else np.sort(rng.choice(n, max_untouched, replace=False))
    if pick.size:
        k, v = ds.pool_rows_bits(w.cached_rows[pick])
        assert np.array_equal(k, w.k_cached[pick]) and np.array_equal(v, w.v_cached[pick]), "cached rows changed"
    # poison page untouched
    k, v = ds.pool_rows_bits(np.arange(w.poison_rows.start, w.poison_rows.stop))
    assert np.all(k == 0x7FC0) and np.all(v == 0x7FC0), "poison page written"


def check_attention(ds, ref_out: dict, w, label: str = ""):
    toks = sorted(ref_out)
    if not toks:
        return {}
    got = ds.output_f64(toks)
    want = np.stack([ref_out[t] for t in toks])
    assert np.all(np.isfinite(got)), f"{label}: non-finite output"
    diff = np.abs(got - want)
    stats = {"tokens": len(toks), "max_abs": float(diff.max()), "mean_abs": float(diff.mean()),
             "rel_max": float(diff.max() / max(np.abs(want).max(), 1e-30))}
    assert stats["max_abs"] <= MAX_ABS_TOL, f"{label}: max-abs {stats['max_abs']:.3e} > {MAX_ABS_TOL}"
    assert stats["mean_abs"] <= MEAN_ABS_TOL, f"{label}: mean-abs {stats['mean_abs']:.3e} > {MEAN_ABS_TOL}"
    return stats


def real_outputs_finite(ds, w):
    starts = token_starts(w)
    real = [np.arange(starts[i], starts[i + 1]) for i in range(w.num_reqs) if not w.is_padding[i]]
    if not real:
        return
    idx = torch.as_tensor(np.concatenate(real), device=ds.device)
    assert bool(torch.isfinite(ds.o[idx].float()).all()), "a real output is NaN/inf (poison read or unwritten row)"


def oracle_for(w, decode_requests=None, extend_tokens=None):
    reqs = []
    dec = range(w.num_decode) if decode_requests is None else decode_requests
    reqs += [i for i in dec if not w.is_padding[i]]
    tokens = {}
    if extend_tokens is None:
        reqs += list(range(w.num_decode, w.num_reqs))
    else:
        reqs += list(extend_tokens)
        tokens = extend_tokens
    return reference_step(w, requests=reqs, tokens=tokens)
