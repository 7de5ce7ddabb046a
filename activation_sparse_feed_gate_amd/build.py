"""Build the gfx950 HIP library ``libtw.so`` in-tree with hipcc.

Every HIP source is compiled for gfx950 only, with the packed-fp32 target
feature switched off (the compiler then never emits packed fp32 add/mul/fma),
and linked into one shared library exporting the C ABI of ``include/tw.h``.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD_DIR = os.path.join(ROOT, "_build")
LIBRARY = os.path.join(HERE, "libtw.so")
PEAK_PROBE = os.path.join(HERE, "peak_probe")  # achievable-peak program (csrc/peak_probe.hip)

SOURCES = ["gate_twell.hip", "pack_dense.hip", "sparse_updown.hip", "dense_ffn.hip", "hybrid.hip",
           "tw_api.cpp"]

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-Wall",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", INCLUDE, "-I", CSRC,
]


def build(verbose: bool = False) -> str:
    """Compile all sources (in parallel) and link ``libtw.so``; returns its path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    procs = []
    objs = []
    for src in SOURCES:
        obj = os.path.join(BUILD_DIR, src + ".o")
        objs.append(obj)
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        cmd = [HIPCC, *FLAGS, *lang, "-c", os.path.join(CSRC, src), "-o", obj]
        if verbose:
            print(" ".join(cmd), flush=True)
        procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
    failed = []
    for src, p in procs:
        out, _ = p.communicate()
        if out and (verbose or p.returncode):
            sys.stderr.write(out.decode(errors="replace"))
        if p.returncode:
            failed.append(src)
    if failed:
        raise RuntimeError(f"hipcc failed for {failed}")
    tmp = LIBRARY + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, LIBRARY)
    return LIBRARY


def build_peak_probe(verbose: bool = False) -> str:
    """Compile the standalone achievable-peak program (a measurement tool,
    not part of the library: built only on request, with
    ``python -m activation_sparse_feed_gate_amd.build --peak-probe``);
    returns its path."""
    cmd = [HIPCC, *FLAGS, os.path.join(CSRC, "peak_probe.hip"), "-o", PEAK_PROBE]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    return PEAK_PROBE


if __name__ == "__main__":
    if "--peak-probe" in sys.argv:
        print(build_peak_probe(verbose="-v" in sys.argv))
    else:
        print(build(verbose="-v" in sys.argv))
