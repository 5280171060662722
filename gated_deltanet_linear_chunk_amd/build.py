"""Build libgdn.so (the HIP kernels + C ABI) in-tree for gfx950 with hipcc.

python -m gated_deltanet_linear_chunk_amd.build [--jobs N]

Objects go to _build/ at the repository root; the shared library lands next
to this file, where the Python binding loads it from.  The same call builds
libgdn_probe.so (csrc/probe/: the matrix-core rate probe the benchmark
reports against), which the library does not use.
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
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libgdn.so")
PROBE_LIB = os.path.join(PKG, "libgdn_probe.so")
PROBE_SOURCES = ["probe/mfma_peak.hip"]

SOURCES = ["api.cpp", "split_plan.cpp", "gate_conv.hip", "chunk_f32.hip", "chunk_prep.hip", "chunk_bf16.hip",
           "compose.hip", "decode.hip", "gated_norm.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
FLAGS = [
    "-O3",
    "-std=c++17",
    "-fPIC",
    "--offload-arch=" + ARCH,
    # keep the compiler from emitting packed fp32 arithmetic
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE,
    "-I", CSRC,
    "-Wall",
    "-Wno-unused-function",
]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src.replace("/", "_"))[0] + ".o")
    lang = ["-x", "hip"] if src.endswith(".cpp") else []
    cmd = [HIPCC] + FLAGS + lang + ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("compile failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    noise = "is not a recognized feature for this target"
    msgs = [l for l in (r.stderr or "").splitlines() if noise not in l and "warnings generated" not in l]
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def _link(objs, lib: str) -> None:
    tmp = lib + ".tmp%d" % os.getpid()
    cmd = [HIPCC, "-shared", "-fPIC", "--offload-arch=" + ARCH, "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed: %s\n%s\n%s" % (" ".join(cmd), r.stdout, r.stderr))
    os.replace(tmp, lib)


def build(jobs: int = 4) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with ThreadPoolExecutor(max_workers=max(1, jobs)) as ex:
        objs = list(ex.map(_compile, SOURCES + PROBE_SOURCES))
    _link(objs[: len(SOURCES)], LIB)
    _link(objs[len(SOURCES):], PROBE_LIB)
    return LIB


if __name__ == "__main__":
    ap = argparse.ArgumentParser()
    ap.add_argument("--jobs", type=int, default=4)
    args = ap.parse_args()
    print(build(args.jobs))
