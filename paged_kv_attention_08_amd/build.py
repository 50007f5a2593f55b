"""Build libpagedkv.so (gfx950) in-tree with hipcc.

    python -m paged_kv_attention_08_amd.build            # build
    python -m paged_kv_attention_08_amd.build --asm DIR  # also dump device assembly

Every source is compiled for gfx950 only.  Packed fp32 instructions are
disabled on the device side (`-Xclang -target-feature -Xclang -packed-fp32-ops`);
the host pass prints a harmless warning that it does not know the feature.
"""
from __future__ import annotations

import argparse
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libpagedkv.so")
SOURCES = ["api.hip", "kv_store.hip", "rope.hip", "graph.hip", "alloc.hip", "metadata.hip", "decode.hip", "extend.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = ["-O3", "-std=c++17", f"--offload-arch={ARCH}", "-fPIC", "-Wall", "-Wno-unused-function",
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         "-I", os.path.join(ROOT, "include")]


def _run(cmd):
    p = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(l for l in p.stdout.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"command failed ({p.returncode}): {' '.join(cmd)}\n{out}")
    return out


def build(verbose: bool = False, asm_dir: str | None = None) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]

    def compile_one(i):
        src = os.path.join(CSRC, SOURCES[i])
        return _run([HIPCC, *FLAGS, "-c", src, "-o", objs[i]])

    with ThreadPoolExecutor(max_workers=min(8, len(SOURCES))) as ex:
        outs = list(ex.map(compile_one, range(len(SOURCES))))
    if verbose:
        for o in outs:
            if o.strip():
                print(o)
    tmp = LIB + ".tmp"
    _run([HIPCC, *FLAGS, "-shared", "-o", tmp, *objs])
    os.replace(tmp, LIB)
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        for s in SOURCES:
            _run([HIPCC, *FLAGS, "-S", "--cuda-device-only", os.path.join(CSRC, s), "-o",
                  os.path.join(asm_dir, s.replace(".hip", ".s"))])
    return LIB


def main(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--asm", default=None, help="directory for device assembly dumps")
    ap.add_argument("-v", action="store_true")
    args = ap.parse_args(argv)
    print(build(verbose=args.v, asm_dir=args.asm))


if __name__ == "__main__":
    sys.exit(main())
