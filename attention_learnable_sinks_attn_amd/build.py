"""Builds libattn_sink.so (HIP, gfx950 only) in the package directory.

Usage: ``python -m attention_learnable_sinks_attn_amd.build`` (also called by
``__graft_entry__.build()``). Each source is compiled to an object in parallel, then linked.
"""
from __future__ import annotations

import concurrent.futures
import os
import shutil
import subprocess
import sys

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG_DIR)
CSRC = os.path.join(PKG_DIR, "csrc")
INCLUDE = os.path.join(ROOT, "include")
LIB_PATH = os.path.join(PKG_DIR, "libattn_sink.so")
# The benchmark's matrix-core throughput probe, a library of its own (the attention path never loads it).
PROBE_LIB_PATH = os.path.join(PKG_DIR, "libattn_sink_probe.so")
PROBE_SOURCES = ("probe.hip",)
BUILD_DIR = os.path.join(ROOT, "_build")
SOURCES = ("fwd.hip", "bwd.hip", "decode.hip", "api.hip")
ARCH = "gfx950"


def hipcc() -> str:
    cand = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    return cand


def compile_flags():
    return ["--offload-arch=" + ARCH, "-O3", "-std=c++17", "-fPIC",
            # no packed fp32 (v_pk_*_f32) code generation
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-I", INCLUDE, "-I", CSRC]


def _run(cmd):
    proc = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
    out = "\n".join(line for line in proc.stdout.splitlines()
                    if "is not a recognized feature for this target" not in line)
    if proc.returncode != 0:
        raise RuntimeError("command failed (%d): %s\n%s" % (proc.returncode, " ".join(cmd), out))
    return out


def build_library(verbose: bool = False) -> str:
    os.makedirs(BUILD_DIR, exist_ok=True)
    cc = hipcc()
    jobs = []
    for src in SOURCES + PROBE_SOURCES:
        obj = os.path.join(BUILD_DIR, src.replace(".hip", ".o"))
        jobs.append([cc, *compile_flags(), "-c", os.path.join(CSRC, src), "-o", obj])
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(jobs)) as ex:
        for out in ex.map(_run, jobs):
            if verbose and out.strip():
                print(out)
    for path, srcs in ((LIB_PATH, SOURCES), (PROBE_LIB_PATH, PROBE_SOURCES)):
        objs = [os.path.join(BUILD_DIR, src.replace(".hip", ".o")) for src in srcs]
        tmp = path + ".tmp"
        _run([cc, "--offload-arch=" + ARCH, "-shared", "-fPIC", "-o", tmp, *objs])
        os.replace(tmp, path)
        if verbose:
            print("built", path)
    return LIB_PATH


if __name__ == "__main__":
    build_library(verbose="-v" in sys.argv)
