#!/usr/bin/env python3
"""Benchmark of the paged-KV attention step on one MI355X.

One step = one pass of the whole path over one batch: build_attn_metadata,
kv_store, paged_decode_attn (split-K partial + merge) and paged_extend_attn,
on inputs already resident in HBM.  The default workload is the serving
decode batch (Llama-3-8B-like layer: 32 query / 8 KV heads, head_dim 128,
256 requests = 200 real + 56 padding, contexts U[512, 4096], page_size 1,
2^21-row pool).  `--config 1..5` selects another of the five workloads.

Prints ONE JSON line.  `value` is the whole step's algorithmic bytes (decode
K/V + page-table + q/o, store, metadata) per second for decode-dominated
workloads, or its extend flops per second for extend-dominated ones.
`roofline` covers the dominant call, timed with HIP events on the stream it
runs on; `cpu_baseline` times the fp64 oracle on the host.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "paged decode attn HBM GB/s (% peak); extend attn TFLOPS (% MFMA peak)"

WORKLOAD_TEXT = {
    1: "tiny_decode: 16 q / 8 kv heads, d 128, batch 4, ctx U[64,256], page_size 1, pool 4096 rows",
    2: "serving_decode: Llama-3-8B-like layer, 32 q / 8 kv heads, d 128, batch 256 (200 real + 56 dummy), "
       "ctx U[512,4096], page_size 1, pool 2^21 rows, fragmented rows",
    3: "extend_radix: 32 q / 8 kv heads, d 128, 8 requests sharing a 2048-row prefix, private tail U[0,1024], "
       "1024 new tokens each (8192), page_size 1, pool 2^20 rows",
    4: "long_decode: 70B-like layer, 64 q / 8 kv heads, d 128, batch 32, ctx U[16384,32768], page_size 1, "
       "~150 GB pool (36,621,056 rows), rows scattered over the pool",
    5: "mixed_page64: 32 q / 8 kv heads, d 128, page_size 64, 64 decode (ctx U[1024,8192]) + 4 extend "
       "(2048 new tokens on prefixes U[0,4096]), pool 2^20 rows",
}


def log(msg):
    print(f"[bench {time.strftime('%H:%M:%S')}] {msg}", file=sys.stderr, flush=True)


def cpu_baseline(w, kind: str, budget_s: float):
    """The fp64 oracle as it stands, single BLAS thread, on a bounded sample."""
    from threadpoolctl import threadpool_limits
    import oracle.pagedkv_oracle as O
    from oracle.run import initial_pool
    from paged_kv_attention_08_amd import perf_model as PM

    pool = initial_pool(w)
    real = [i for i in range(w.num_reqs) if not w.is_padding[i]]
    with threadpool_limits(limits=1):
        t0 = time.perf_counter()
        meta = O.build_metadata(w.page_table, w.table_idx, w.cached_len, w.device_len, w.alloc_rows, w.page_size)
        pool2 = O.store_kv(pool, w.k_new, w.v_new, meta["out_loc"])
        t_fixed = time.perf_counter() - t0
        done_reqs, done_tokens = [], {}
        t1 = time.perf_counter()
        if kind == "decode":
            for i in real:
                if i >= w.num_decode:
                    continue
                O.paged_attention(pool2, meta["page_table"], w.table_idx, w.cached_len, w.device_len, w.q,
                                  w.num_kv_heads, w.sm_scale, requests=[i])
                done_reqs.append(i)
                if time.perf_counter() - t1 > budget_s:
                    break
            elapsed = time.perf_counter() - t1 + t_fixed
            work = PM.decode_bytes(w.device_len[done_reqs], w.num_qo_heads, w.num_kv_heads, w.head_dim,
                                   w.page_size)
            value = work / elapsed / 1e9
            unit = "GB/s"
            sample = (f"metadata + store of the whole batch and decode attention of {len(done_reqs)} of "
                      f"{sum(1 for i in real if i < w.num_decode)} real decode requests")
        else:
            rng = np.random.default_rng(0)
            n_tok = 0
            flops = 0
            ext_reqs = [i for i in range(w.num_decode, w.num_reqs)]
            while time.perf_counter() - t1 < budget_s:
                i = int(rng.choice(ext_reqs))
                ext = int(w.device_len[i] - w.cached_len[i])
                t = int(rng.integers(0, ext))
                O.paged_attention(pool2, meta["page_table"], w.table_idx, w.cached_len, w.device_len, w.q,
                                  w.num_kv_heads, w.sm_scale, requests=[i], tokens={i: [t]})
                n_tok += 1
                flops += 4 * w.num_qo_heads * w.head_dim * (int(w.cached_len[i]) + t + 1)
            elapsed = time.perf_counter() - t1
            value = flops / elapsed / 1e12
            unit = "TFLOP/s"
            sample = f"extend attention of {n_tok} randomly drawn new tokens (all query heads each)"
    return {"value": value, "unit": unit, "cores": 1, "kind": "oracle", "sample": sample,
            "seconds": round(elapsed, 2)}


def graph_measurement(ds, w, args, stream):
    """The decode step (metadata, store, decode attention) replayed as one HIP
    graph captured for this batch size, against the same three calls issued
    eagerly; per-step latency from events around K back-to-back steps."""
    import torch
    import paged_kv_attention_08_amd as pkv

    side = torch.cuda.Stream()
    torch.cuda.synchronize()
    graph = pkv.DecodeGraph(ds.pool, ds.page_table, ds.batch, ds.alloc_rows, ds.q, ds.o, ds.k_new, ds.v_new,
                            ds.meta, ds.workspace, w.sm_scale, int(w.dummy_table_row), [w.num_reqs], side)
    try:
        def timed(fn):
            for _ in range(args.warmup):
                fn()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            side.synchronize()
            ev[0].record(side)
            for _ in range(args.steps):
                fn()
            ev[1].record(side)
            torch.cuda.synchronize()
            return ev[0].elapsed_time(ev[1]) / args.steps

        def eager():
            ds.metadata(side)
            ds.store(side)
            ds.decode(side)

        eager_ms = timed(eager)
        graph_ms = timed(lambda: graph.replay(w.num_reqs, stream=side))
    finally:
        graph.close()
    assert ds.status() == 0, f"device status {ds.status():#x}"
    return {"batch": w.num_reqs, "eager_step_ms": round(eager_ms, 4), "graph_step_ms": round(graph_ms, 4),
            "what": "build_attn_metadata + kv_store + paged_decode_attn, eager launches vs one graph replay"}


def alloc_measurement(ds, w, args, stream):
    """pkv_alloc_pages for the step's batch from a free list holding every
    page of the pool, then pkv_free_pages of the same pages: one pair per
    step, timed back to back."""
    import torch
    import paged_kv_attention_08_amd as pkv

    s = w.page_size
    npages = w.num_pool_rows // s
    fl = pkv.PageFreeList(npages, s, w.num_pool_rows)
    g = torch.Generator(device="cuda")
    g.manual_seed(5)
    fl.reset((torch.randperm(npages, device="cuda", generator=g, dtype=torch.int64) * s).to(torch.int32))
    c, d = w.cached_len.astype(np.int64), w.device_len.astype(np.int64)
    ok = (c >= 0) & (c <= d)
    n = int((((d + s - 1) // s) - ((c + s - 1) // s))[ok].sum())
    alloc = torch.empty(max(n, 1), dtype=torch.int32, device="cuda")
    status = torch.zeros(1, dtype=torch.int32, device="cuda")

    def pair():
        fl.alloc(ds.batch, alloc, status, stream)
        fl.free(alloc[:n], status, stream)

    for _ in range(args.warmup):
        pair()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        pair()
    ev[1].record(stream)
    torch.cuda.synchronize()
    assert int(status.item()) == 0, f"allocator status {int(status.item()):#x}"
    return {"pages_per_step": n, "free_list_pages": npages,
            "alloc_plus_free_ms": round(ev[0].elapsed_time(ev[1]) / args.steps, 4),
            "what": "pkv_alloc_pages + pkv_free_pages of the step's new pages (launch-latency bound)"}


def rope_measurement(ds, w, args, stream, PM):
    """kv_store_rope (RoPE with Qwen3-style per-head q/k RMS norm, base 1e6) on
    the step's tokens at their metadata positions and rows; timed on its own,
    after the step (it rotates q in place)."""
    import torch
    import paged_kv_attention_08_amd as pkv
    from workloads.rope_inputs import NORM_EPS, rope_inputs

    T = w.num_tokens
    max_pos = int(w.device_len.max()) + 1
    cache = torch.empty((max_pos, w.head_dim), dtype=torch.float32, device="cuda")
    pkv.rope_cos_sin_cache(cache, 1e6)
    inp = rope_inputs(7, 1, w.num_qo_heads, w.num_kv_heads, w.head_dim)  # only the norm weights are used
    from tests.gpu_harness import bf16_tensor
    norm = (bf16_tensor(inp.q_weight, "cuda"), bf16_tensor(inp.k_weight, "cuda"), NORM_EPS)
    out_loc, positions = ds.meta.out_loc[:T], ds.meta.positions[:T]

    def launch():
        pkv.kv_store_rope(ds.pool, ds.q, ds.k_new, ds.v_new, out_loc, positions, cache, qk_norm=norm,
                          status=ds.meta.status, stream=stream)

    for _ in range(args.warmup):
        launch()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ev[0].record(stream)
    for _ in range(args.steps):
        launch()
    ev[1].record(stream)
    torch.cuda.synchronize()
    assert ds.status() == 0, f"device status {ds.status():#x}"
    ms = ev[0].elapsed_time(ev[1]) / args.steps
    nbytes = PM.rope_store_bytes(T, w.num_qo_heads, w.num_kv_heads, w.head_dim)
    gbps = nbytes / (ms * 1e-3) / 1e9
    return {"tokens": T, "avg_launch_ms": round(ms, 4), "algorithmic_bytes_per_launch": nbytes,
            "achieved_gbps": round(gbps, 1), "roofline": {"bound": "hbm", "peak": PM.HBM_PEAK_GBPS,
                                                          "frac": round(gbps / PM.HBM_PEAK_GBPS, 4)},
            "what": "RoPE base 1e6 + per-head q/k RMS norm fused into the K/V store"}


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--settle-ms", type=float, default=300.0,
                    help="after the warm-up steps, untimed steps for at least this long (clock ramp)")
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--flush", action="store_true", help="flush L2/MALL before every step (outside the events)")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work for cpu_baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--layout", choices=["layer_first", "page_first", "row_interleaved"], default="layer_first",
                    help="physical order of a multi-layer KV cache whose layer 0 the step runs on")
    ap.add_argument("--layers", type=int, default=1, help="layers in that cache (1: a plain one-layer pool)")
    ap.add_argument("--page-order", choices=["random", "sequential"], default="random",
                    help="physical page order of the workload: a random order of the free pages (default, rows "
                         "scattered over the pool) or allocation order (a fresh pool's free list)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 1 GiB device copy (torch copy_) 5 times: the known-size reference "
                         "for scaling rocprofv3 FETCH_SIZE / WRITE_SIZE counters")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): this build has no multi-GPU path; "
              "the step shards by request or KV-head group with no exchange, so per-GPU throughput is the "
              "N=1 figure", file=sys.stderr)
        return 2

    import torch
    from workloads import configs
    from tests.gpu_harness import DeviceStep
    from paged_kv_attention_08_amd import perf_model as PM

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 1
    torch.cuda.set_device(0)
    if args.copy_calibration:
        nbytes = 1 << 30
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": nbytes, "copy_calibration_bytes_written": nbytes,
                          "launches": 5}), flush=True)
        return 0
    log(f"generating config {args.config}")
    w = configs.FULL[args.config](page_order=args.page_order)
    log(w.summary())
    pool = None
    if args.layers > 1 or args.layout != "layer_first":
        import paged_kv_attention_08_amd as pkv
        layout = {"layer_first": pkv.KVCacheTensors.LAYER_FIRST, "page_first": pkv.KVCacheTensors.PAGE_FIRST,
                  "row_interleaved": pkv.KVCacheTensors.ROW_INTERLEAVED}[args.layout]
        cache = pkv.KVCacheTensors(args.layers, w.num_pool_rows, w.num_kv_heads, w.head_dim, w.page_size, layout)
        pool = cache.layer(0)
    ds = DeviceStep(w, pool=pool)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    flush_buf = torch.empty(1 << 28, dtype=torch.float32, device="cuda") if args.flush else None

    has_decode = w.num_decode > 0
    has_extend = w.num_decode < w.num_reqs

    def step(marks):
        """One pass of the path.  `marks` maps a position to an event recorded
        there: 0..3 before metadata, store, decode and extend, 4 after the last
        call."""
        def mark(j):
            e = marks.get(j)
            if e is not None:
                e.record(stream)
        mark(0)
        ds.metadata()
        mark(1)
        ds.store()
        mark(2)
        if has_decode:
            ds.decode()
        mark(3)
        if has_extend:
            ds.extend()
        mark(4)

    log(f"warmup {args.warmup} steps, then {args.settle_ms} ms of steps for the clocks to settle")
    for _ in range(args.warmup):
        step({})
    torch.cuda.synchronize()
    # Under a fresh load the GPU runs at lower clocks for its first ~100 ms
    # (extend on the shared-prefix batch: 460 us per call over steps 5..25,
    # 394 us after 200 steps); untimed steps until the clocks have settled.
    settle_steps = 0
    t_settle = time.perf_counter()
    while (time.perf_counter() - t_settle) * 1e3 < args.settle_ms:
        for _ in range(8):
            step({})
        torch.cuda.synchronize()
        settle_steps += 8
    assert ds.status() == 0, f"device status {ds.status():#x}"

    # Per-call breakdown: an event before every call.  Each recorded event adds
    # a few microseconds to the stream, so the step time comes from a second
    # pass below with events around the dominant call only.
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(5)] for _ in range(args.steps)]
    log(f"breakdown over {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush_buf is not None:
            flush_buf.fill_(float(k))
        step({j: events[k][j] for j in range(5)})
    torch.cuda.synchronize()
    breakdown_wall_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    parts = np.array([[events[k][j].elapsed_time(events[k][j + 1]) for j in range(4)] for k in range(args.steps)])
    mean_ms = parts.mean(axis=0)  # metadata, store, decode, extend
    step_ms = float(parts.sum(axis=1).mean())
    decode_dominant = has_decode and (not has_extend or mean_ms[2] >= mean_ms[3])

    # Timed pass: K steps, events only around the dominant call (its launch
    # duration for the roofline), wall clock for the step.
    pos = (2, 3) if decode_dominant else (3, 4)
    pairs = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(args.steps):
        if flush_buf is not None:
            flush_buf.fill_(float(k))
        step({pos[0]: pairs[k][0], pos[1]: pairs[k][1]})
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    assert ds.status() == 0, f"device status {ds.status():#x}"
    dominant_ms = float(np.mean([pairs[k][0].elapsed_time(pairs[k][1]) for k in range(args.steps)]))
    dominant_in_breakdown_ms = float(mean_ms[2 if decode_dominant else 3])
    mean_ms[2 if decode_dominant else 3] = dominant_ms
    wall_ms = wall * 1e3 / args.steps
    ms_per_step = step_ms if args.flush else wall_ms

    real = ~w.is_padding
    dec_mask = np.zeros(w.num_reqs, dtype=bool)
    dec_mask[:w.num_decode] = True
    dec_bytes = PM.decode_bytes(w.device_len[dec_mask & real], w.num_qo_heads, w.num_kv_heads, w.head_dim,
                                w.page_size)
    st_bytes = PM.store_bytes(int((w.device_len[real] - w.cached_len[real]).sum()), w.num_kv_heads, w.head_dim)
    md_bytes = PM.metadata_bytes(w.num_reqs, w.num_tokens)
    ext_flops = PM.extend_flops(w.cached_len[~dec_mask], w.device_len[~dec_mask], w.num_qo_heads, w.head_dim)

    decode_gbps = dec_bytes / (mean_ms[2] * 1e-3) / 1e9 if has_decode else None
    extend_tflops = ext_flops / (mean_ms[3] * 1e-3) / 1e12 if has_extend else None
    store_gbps = st_bytes / (mean_ms[1] * 1e-3) / 1e9
    from paged_kv_attention_08_amd import profiling
    call = "paged_decode_attn" if decode_dominant else "paged_extend_attn"
    measured = profiling.traffic_for(call, args.config)  # None unless taken on the current kernel sources
    traffic = None if measured is None else round(measured["traffic_bytes"])
    if decode_dominant:
        value = (dec_bytes + st_bytes + md_bytes) / (ms_per_step * 1e-3) / 1e9
        unit = "GB/s"
        roof = {"bound": "hbm", "achieved": round(decode_gbps, 1), "peak": PM.HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(decode_gbps / PM.HBM_PEAK_GBPS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "kernel": "paged_decode_attn (decode_kernel + decode_merge_kernel)",
                "algorithmic_bytes_per_launch": dec_bytes, "avg_launch_ms": round(float(mean_ms[2]), 4),
                "profile": None if measured is None else measured["summary"]}
    else:
        value = ext_flops / (ms_per_step * 1e-3) / 1e12
        unit = "TFLOP/s"
        roof = {"bound": "mfma", "achieved": round(extend_tflops, 1), "peak": PM.BF16_DENSE_PEAK_TFLOPS,
                "unit": "TFLOP/s", "frac": round(extend_tflops / PM.BF16_DENSE_PEAK_TFLOPS, 4), "traffic": traffic,
                "traffic_unit": "HBM bytes per launch (rocprofv3 FETCH_SIZE + WRITE_SIZE, copy-calibrated)",
                "kernel": "paged_extend_attn (extend_kernel)", "algorithmic_flops_per_launch": ext_flops,
                "avg_launch_ms": round(float(mean_ms[3]), 4),
                "profile": None if measured is None else measured["summary"]}

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": unit, "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "settle_steps": settle_steps, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": WORKLOAD_TEXT[args.config], "config_index": args.config,
                   "global_batch": w.num_reqs, "new_tokens": w.num_tokens, "parallelism": "single GPU",
                   "l2_mall_flush_between_steps": bool(args.flush), "page_order": args.page_order,
                   "kv_cache": f"{args.layers} layer(s), {args.layout}, step on layer 0"},
        "breakdown_ms": {"metadata": round(float(mean_ms[0]), 4), "kv_store": round(float(mean_ms[1]), 4),
                         "decode": round(float(mean_ms[2]), 4), "extend": round(float(mean_ms[3]), 4),
                         "wall_per_step": round(wall_ms, 4), "events_per_step": round(step_ms, 4),
                         "wall_per_step_with_breakdown_events": round(breakdown_wall_ms, 4),
                         "dominant_call_in_breakdown_pass": round(dominant_in_breakdown_ms, 4)},
        "decode_gbps": None if decode_gbps is None else round(decode_gbps, 1),
        "decode_frac_hbm": None if decode_gbps is None else round(decode_gbps / PM.HBM_PEAK_GBPS, 4),
        "extend_tflops": None if extend_tflops is None else round(extend_tflops, 1),
        "extend_frac_mfma": None if extend_tflops is None else round(extend_tflops / PM.BF16_DENSE_PEAK_TFLOPS, 4),
        "store_gbps": round(store_gbps, 1),
        "roofline": roof,
    }
    out["next_rows"] = {}
    if has_decode and not has_extend:
        out["next_rows"]["decode_graph"] = graph_measurement(ds, w, args, stream)
    out["next_rows"]["page_alloc"] = alloc_measurement(ds, w, args, stream)
    out["next_rows"]["kv_store_rope"] = rope_measurement(ds, w, args, stream, PM)
    ds.free()
    if not args.no_cpu_baseline:
        log("cpu baseline (fp64 oracle)")
        out["cpu_baseline"] = cpu_baseline(w, "decode" if decode_dominant else "extend", args.cpu_budget)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
