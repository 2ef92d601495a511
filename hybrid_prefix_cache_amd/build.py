"""Build libkda.so (HIP kernels + C ABI) for gfx950 with hipcc, in-tree.

Usage: python hybrid_prefix_cache_amd/build.py   (run as a file: importing the
package first would bind the symbols of a possibly stale libkda.so)
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libkda.so")
# peak probes for the benchmark's roofline denominators (not part of libkda)
PROBE_SRC = "kda_probe.hip"
PROBE_LIB = os.path.join(HERE, "libkda_probe.so")
SOURCES = ["kda_api.cpp", "kda_prefill.hip", "kda_decode.hip", "kda_copy.hip", "kda_ckpt_int8.hip", "kda_conv.hip",
           "kda_index.cpp", "kda_noalloc.hip"]
ARCH = os.environ.get("KDA_OFFLOAD_ARCH", "gfx950")
FLAGS = ["-O3", "-fPIC", "-std=c++17", f"--offload-arch={ARCH}",
         # no packed fp32 instructions (v_pk_*_f32) in device code
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
         # matrix-core results in ordinary VGPRs: otherwise the prep kernels
         # copy ~150 accumulator values per pair out of AGPRs one at a time
         "-mllvm", "-amdgpu-mfma-vgpr-form",
         "-Wall", "-Wno-unused-function", "-I", os.path.join(HERE, "..", "include")]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = ["hipcc", f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(SOURCES) + 1)) as ex:
        objs = list(ex.map(_compile, SOURCES + [PROBE_SRC]))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
