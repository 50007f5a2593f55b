"""Summaries of rocprofv3 output for the paged-KV kernels.

    python -m paged_kv_attention_08_amd.profiling summarize \\
        --name decode_serving_b256 --kernels decode_kernel,decode_merge_kernel \\
        --trace DIR --fetch DIR --write DIR --copy-fetch DIR --copy-write DIR \\
        --algorithmic-bytes N --command "..." --out profiles/<name>.md

reads the CSV files rocprofv3 wrote (--output-format csv), writes a short
text summary (kernel times, HBM traffic) and records the traffic figure in
profiles/traffic.json together with a hash of the kernel sources, so that the
benchmark reports it only while the kernels are unchanged.

HBM traffic: rocprofv3's FETCH_SIZE and WRITE_SIZE (KiB per dispatch) are
scaled by what the same counters read for a plain device copy of known size
(1 GiB read, 1 GiB written) in a run of their own.
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
from collections import defaultdict

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "traffic.json")
KERNEL_SOURCES = {
    "paged_decode_attn": ["decode.hip", "common.hpp", "kernels.hpp"],
    "paged_extend_attn": ["extend.hip", "common.hpp", "kernels.hpp"],
    "kv_store": ["kv_store.hip", "common.hpp", "kernels.hpp"],
}


def source_hash(call: str) -> str:
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[call]:
        with open(os.path.join(PKG, "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def _csv(d: str, suffix: str) -> str:
    hits = glob.glob(os.path.join(d, "**", f"*{suffix}"), recursive=True)
    if not hits:
        raise FileNotFoundError(f"no *{suffix} under {d}")
    return hits[0]


def kernel_stats(trace_dir: str):
    rows = list(csv.DictReader(open(_csv(trace_dir, "kernel_stats.csv"))))
    return [(r["Name"], int(r["Calls"]), float(r["AverageNs"]), float(r["Percentage"])) for r in rows]


def counter_means(pmc_dir: str, counter: str):
    acc = defaultdict(list)
    for r in csv.DictReader(open(_csv(pmc_dir, "counter_collection.csv"))):
        if r["Counter_Name"] == counter:
            acc[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return {k: sum(v) / len(v) for k, v in acc.items()}


def _pick(table: dict, key: str) -> float:
    vals = [v for k, v in table.items() if key in k]
    if not vals:
        raise KeyError(key)
    return vals[0]


def algorithmic_bytes(call: str, config: int) -> int:
    """Bytes one launch of `call` must move on workload `config` (perf_model):
    decode K/V rows, page-table entries, q and o of the real decode requests;
    extend q, o, every distinct K/V row it sees (new rows included) and its
    page-table entries; store new rows in and out."""
    import numpy as np
    from workloads import configs
    from . import perf_model as PM
    w = configs.FULL[config]()
    dec = np.zeros(w.num_reqs, dtype=bool)
    dec[:w.num_decode] = True
    real = ~w.is_padding
    if call == "paged_decode_attn":
        return PM.decode_bytes(w.device_len[dec & real], w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size)
    if call == "paged_extend_attn":
        m = ~dec
        return PM.extend_unique_bytes(w.page_table, w.table_idx[m], w.cached_len[m], w.device_len[m],
                                      w.num_qo_heads, w.num_kv_heads, w.head_dim, w.page_size)
    return PM.store_bytes(int((w.device_len[real] - w.cached_len[real]).sum()), w.num_kv_heads, w.head_dim)


def summarize(args) -> dict:
    kernels = args.kernels.split(",")
    if args.algorithmic_bytes is None:
        args.algorithmic_bytes = float(algorithmic_bytes(args.call, args.config))
    stats = kernel_stats(args.trace)
    fetch = counter_means(args.fetch, "FETCH_SIZE")
    write = counter_means(args.write, "WRITE_SIZE")
    copy_fetch = _pick(counter_means(args.copy_fetch, "FETCH_SIZE"), args.copy_kernel)
    copy_write = _pick(counter_means(args.copy_write, "WRITE_SIZE"), args.copy_kernel)
    fetch_scale = (1 << 30) / (copy_fetch * 1024.0)
    write_scale = (1 << 30) / (copy_write * 1024.0)
    lines = [f"# {args.name}", "", f"Command: `{args.command}`", "",
             "| kernel | calls | average us | % of GPU time |", "|---|---|---|---|"]
    total_ns = 0.0
    for name, calls, avg, pct in stats:
        short = name.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
        if any(k in name for k in kernels) or "pkv::" in name or "reduce" in name.lower():
            lines.append(f"| {short} | {calls} | {avg / 1e3:.2f} | {pct:.2f} |")
        if any(k in name for k in kernels):
            total_ns += avg
    fetch_b = sum(_pick(fetch, k) for k in kernels) * 1024 * fetch_scale
    write_b = sum(_pick(write, k) for k in kernels) * 1024 * write_scale
    traffic = fetch_b + write_b
    lines += ["", f"Dominant call `{args.call}` = {' + '.join(kernels)}: average {total_ns / 1e3:.2f} us per launch "
              "(sum of the kernels' averages).", "",
              f"HBM traffic per launch (rocprofv3 FETCH_SIZE / WRITE_SIZE, each in its own run, scaled by a 1 GiB "
              f"device copy that read {copy_fetch:.0f} KiB and wrote {copy_write:.0f} KiB: factors "
              f"{fetch_scale:.3f} and {write_scale:.3f}):", "",
              f"- read {fetch_b / 1e9:.4f} GB, written {write_b / 1e9:.4f} GB, total {traffic / 1e9:.4f} GB",
              f"- algorithmic bytes {args.algorithmic_bytes / 1e9:.4f} GB -> traffic / algorithmic = "
              f"{traffic / args.algorithmic_bytes:.3f}" if args.algorithmic_bytes else "",
              f"- kernel-source hash {source_hash(args.call)}"]
    for d in args.extra or []:
        rows = defaultdict(lambda: defaultdict(list))
        for r in csv.DictReader(open(_csv(d, "counter_collection.csv"))):
            if any(k in r["Kernel_Name"] for k in kernels):
                rows[r["Counter_Name"]][r["Kernel_Name"]].append(float(r["Counter_Value"]))
        lines += ["", f"Counters (mean per dispatch, `{os.path.basename(d.rstrip('/'))}` pass):", ""]
        for cn in sorted(rows):
            for kn, v in rows[cn].items():
                short = kn.replace("(anonymous namespace)::", "").split("(")[0].replace("void ", "")
                lines.append(f"- {short} {cn}: {sum(v) / len(v):.0f}")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in rows and "GRBM_GUI_ACTIVE" in rows:
            busy = sum(sum(v) / len(v) for v in rows["SQ_VALU_MFMA_BUSY_CYCLES"].values())
            act = sum(sum(v) / len(v) for v in rows["GRBM_GUI_ACTIVE"].values())
            lines.append(f"- MFMA busy / (1024 SIMDs x active cycles per XCD (GRBM_GUI_ACTIVE / 8)) = "
                         f"{busy / (1024 * act / 8):.3f}")
        if "TCP_UTCL1_TRANSLATION_MISS_sum" in rows:
            miss = sum(sum(v) / len(v) for v in rows["TCP_UTCL1_TRANSLATION_MISS_sum"].values())
            hit = sum(sum(v) / len(v) for v in rows["TCP_UTCL1_TRANSLATION_HIT_sum"].values())
            lines.append(f"- UTCL1 translation miss rate {miss / (miss + hit):.3f}")
    with open(args.out, "w") as f:
        f.write("\n".join(l for l in lines if l is not None) + "\n")
    rec = {"source_hash": source_hash(args.call), "config": args.config, "fetch_bytes": fetch_b,
           "write_bytes": write_b, "traffic_bytes": traffic, "fetch_scale": fetch_scale, "write_scale": write_scale,
           "avg_launch_us": total_ns / 1e3, "summary": os.path.relpath(args.out, ROOT)}
    data = {}
    if os.path.exists(TRAFFIC_JSON):
        data = json.load(open(TRAFFIC_JSON))
    data.setdefault(args.call, {})[str(args.config)] = rec
    with open(TRAFFIC_JSON, "w") as f:
        json.dump(data, f, indent=1, sort_keys=True)
    return rec


def traffic_for(call: str, config: int):
    """Measured HBM bytes per launch of `call` on `config`, or None if the
    counters were taken on different kernel sources (or never)."""
    if not os.path.exists(TRAFFIC_JSON):
        return None
    rec = json.load(open(TRAFFIC_JSON)).get(call, {}).get(str(config))
    if not rec or rec.get("source_hash") != source_hash(call):
        return None
    return rec


def main(argv=None):
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    s = sub.add_parser("summarize")
    s.add_argument("--name", required=True)
    s.add_argument("--call", required=True, choices=sorted(KERNEL_SOURCES))
    s.add_argument("--config", type=int, required=True)
    s.add_argument("--kernels", required=True, help="comma-separated kernel name fragments")
    s.add_argument("--trace", required=True)
    s.add_argument("--fetch", required=True)
    s.add_argument("--write", required=True)
    s.add_argument("--copy-fetch", required=True)
    s.add_argument("--copy-write", required=True)
    s.add_argument("--copy-kernel", default="copyBuffer")
    s.add_argument("--algorithmic-bytes", type=float, default=None,
                   help="default: computed for --call on workload --config")
    s.add_argument("--command", required=True)
    s.add_argument("--extra", action="append", help="directory of another counter pass to list")
    s.add_argument("--out", required=True)
    args = ap.parse_args(argv)
    print(json.dumps(summarize(args), indent=1))


if __name__ == "__main__":
    main()
