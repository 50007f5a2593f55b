"""The five synthetic workloads of the paged-KV attention step, and smaller
variants with the same structure.

Each builder draws integer lengths from the first child of
``SeedSequence(seed)`` (see ``synth.build_workload`` for the later stages), so
the full-size and reduced variants of one config share their recipe.  All
values are N(0,1) rounded to bf16; the softmax scale is 1/sqrt(head_dim).

Shapes are Qwen3-0.6B-like (16 query / 8 KV heads), Llama-3-8B-like (32/8) and
a 70B-like layer at TP=1 head counts (64/8), head_dim 128.
"""
from __future__ import annotations

import numpy as np

from .synth import RequestSpec, Workload, build_workload


def _length_rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed).spawn(1)[0]))


def tiny_decode(seed: int = 1001, batch: int = 4, lo: int = 64, hi: int = 256, num_pool_rows: int = 4096,
                page_order: str = "random") -> Workload:
    """Single-layer decode, 16 query / 8 KV heads, page_size 1, pool of 4096 rows.

    Context length L ~ U{lo..hi}; the step stores one new row per request, so
    cached_len = L and device_len = L + 1.
    """
    rng = _length_rng(seed)
    L = rng.integers(lo, hi + 1, size=batch)
    reqs = [RequestSpec(int(l), int(l) + 1) for l in L]
    return build_workload("tiny_decode", seed, reqs, num_qo_heads=16, num_kv_heads=8, head_dim=128,
                          page_size=1, num_pool_rows=num_pool_rows, num_decode=batch,
                          width=((hi + 1 + 31) // 32) * 32, page_order=page_order)


def serving_decode(seed: int = 1002, real: int = 200, padded_to: int = 256, lo: int = 512, hi: int = 4096,
                   page_order: str = "random",
                   num_pool_rows: int = 1 << 21, num_qo_heads: int = 32) -> Workload:
    """Llama-3-8B-like decode: 200 real requests padded with dummies to 256."""
    rng = _length_rng(seed)
    L = rng.integers(lo, hi + 1, size=real)
    reqs = [RequestSpec(int(l), int(l) + 1) for l in L]
    reqs += [RequestSpec(0, 1, padding=True) for _ in range(padded_to - real)]
    return build_workload("serving_decode", seed, reqs, num_qo_heads=num_qo_heads, num_kv_heads=8, head_dim=128,
                          page_size=1, num_pool_rows=num_pool_rows, num_decode=padded_to,
                          width=((hi + 1 + 31) // 32) * 32, page_order=page_order)


def extend_radix(seed: int = 1003, nreq: int = 8, prefix: int = 2048, tail_hi: int = 1024, chunk: int = 1024,
                 num_pool_rows: int = 1 << 20, page_order: str = "random") -> Workload:
    """Chunked prefill on a radix-shared prefix: every request's first `prefix`
    cached tokens are the same physical rows; private cached tail ~ U{0..tail_hi};
    `chunk` new tokens per request."""
    rng = _length_rng(seed)
    tails = rng.integers(0, tail_hi + 1, size=nreq)
    reqs = [RequestSpec(prefix + int(t), prefix + int(t) + chunk, shared_prefix=prefix) for t in tails]
    return build_workload("extend_radix", seed, reqs, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          page_size=1, num_pool_rows=num_pool_rows, num_decode=0,
                          width=((prefix + tail_hi + chunk + 31) // 32) * 32, page_order=page_order)


LONG_DECODE_POOL_ROWS = 36_621_056   # 150.0e9 bytes of K+V at 8 KV heads x 128 x bf16


def long_decode(seed: int = 1004, batch: int = 32, lo: int = 16384, hi: int = 32768,
                num_pool_rows: int = LONG_DECODE_POOL_ROWS, page_order: str = "random") -> Workload:
    """70B-like layer (64 query / 8 KV heads) decode over 16K-32K contexts in a
    ~150 GB pool; rows are scattered uniformly over the whole pool."""
    rng = _length_rng(seed)
    L = rng.integers(lo, hi + 1, size=batch)
    reqs = [RequestSpec(int(l), int(l) + 1) for l in L]
    return build_workload("long_decode", seed, reqs, num_qo_heads=64, num_kv_heads=8, head_dim=128,
                          page_size=1, num_pool_rows=num_pool_rows, num_decode=batch,
                          width=((hi + 1 + 31) // 32) * 32, page_order=page_order)


def mixed_page64(seed: int = 1005, ndec: int = 64, dec_lo: int = 1024, dec_hi: int = 8192, next_: int = 4,
                 pre_hi: int = 4096, new_tokens: int = 2048, num_pool_rows: int = 1 << 20,
                 page_size: int = 64, page_order: str = "random") -> Workload:
    """page_size 64 mixed batch: decode requests first, then extend requests of
    `new_tokens` on prefixes ~ U{0..pre_hi}; page-aligned random free pages."""
    rng = _length_rng(seed)
    L = rng.integers(dec_lo, dec_hi + 1, size=ndec)
    P = rng.integers(0, pre_hi + 1, size=next_)
    reqs = [RequestSpec(int(l), int(l) + 1) for l in L]
    reqs += [RequestSpec(int(p), int(p) + new_tokens) for p in P]
    width = ((max(dec_hi + 1, pre_hi + new_tokens) + 31) // 32) * 32
    return build_workload("mixed_page64", seed, reqs, num_qo_heads=32, num_kv_heads=8, head_dim=128,
                          page_size=page_size, num_pool_rows=num_pool_rows, num_decode=ndec, width=width,
                          page_order=page_order)


FULL = {
    1: tiny_decode,
    2: serving_decode,
    3: extend_radix,
    4: long_decode,
    5: mixed_page64,
}


def small(config: int, seed: int = 7) -> Workload:
    """A reduced variant of a config that the oracle finishes in seconds but
    that still spans several kernel tiles and ragged tails."""
    if config == 1:
        return tiny_decode(seed=seed)
    if config == 2:
        return serving_decode(seed=seed, real=24, padded_to=32, lo=1, hi=700, num_pool_rows=1 << 15)
    if config == 3:
        return extend_radix(seed=seed, nreq=3, prefix=96, tail_hi=70, chunk=83, num_pool_rows=1 << 13)
    if config == 4:
        return long_decode(seed=seed, batch=3, lo=1500, hi=2600, num_pool_rows=1 << 16)
    if config == 5:
        return mixed_page64(seed=seed, ndec=6, dec_lo=1, dec_hi=300, next_=3, pre_hi=200, new_tokens=150,
                            num_pool_rows=64 * 64)
    raise ValueError(config)
