"""Build libmqa_int8.so in-tree with hipcc for gfx950.

Usage: python -m mqa_attention_int8_amd.build   (or __graft_entry__.build())
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libmqa_int8.so")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")
ARCH = "gfx950"

SOURCES = ["api.cpp", "prefix_cache.cpp", "quantize.hip", "decode.hip", "prefill.hip", "kv_transfer.hip"]
# Measurement kernels of the benchmark, in a library of their own.
CEILINGS_LIB = os.path.join(PKG, "libmqa_ceilings.so")
CEILINGS_SOURCES = ["ceilings.hip"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-mcode-object-version=5",
    # keep hipcc from forming packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-Wno-unused-function",
]


def hipcc() -> str:
    p = os.path.join(ROCM, "bin", "hipcc")
    return p if os.path.exists(p) else (shutil.which("hipcc") or "hipcc")


def build(verbose: bool = False, jobs: int = 4) -> str:
    """Compile and link libmqa_int8.so and libmqa_ceilings.so; returns the
    attention library's path."""
    _link(SOURCES, LIB, verbose, jobs)
    _link(CEILINGS_SOURCES, CEILINGS_LIB, verbose, jobs)
    return LIB


def _link(sources, lib_path: str, verbose: bool, jobs: int) -> None:
    out_dir = os.path.join(PKG, "_objs")
    os.makedirs(out_dir, exist_ok=True)
    procs, objs = [], []
    for src in sources:
        obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
        lang = ["-x", "hip"] if src.endswith(".hip") else []
        cmd = [hipcc(), *HIPCC_FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
        objs.append(obj)
        while len([p for _, p in procs if p.poll() is None]) >= jobs:
            procs[0][1].wait()
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        text = out.decode(errors="replace")
        if p.returncode != 0:
            failed.append((src, text))
        elif verbose and text.strip():
            print(text)
    if failed:
        for src, text in failed:
            sys.stderr.write(f"--- {src} ---\n{text}\n")
        raise RuntimeError("hipcc failed for: " + ", ".join(s for s, _ in failed))
    tmp = lib_path + ".tmp"
    cmd = [hipcc(), f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs,
           f"-L{ROCM}/lib", "-lamdhip64", "-Wl,--no-undefined"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, lib_path)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
