"""Compile tests/host/abi_consumer.c (plain C99) against include/kda.h and the
in-tree libkda.so; used by the CPU link check and the GPU run."""
import os
import subprocess

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "host", "abi_consumer.c")
LIBDIR = os.path.join(ROOT, "hybrid_prefix_cache_amd")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def build(out_path: str) -> str:
    cmd = ["gcc", "-std=c99", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROCM, "include"), "-I", os.path.join(ROOT, "include"), SRC,
           "-L", LIBDIR, "-lkda", f"-Wl,-rpath,{LIBDIR}",
           "-L", os.path.join(ROCM, "lib"), "-lamdhip64", f"-Wl,-rpath,{os.path.join(ROCM, 'lib')}",
           "-lm", "-o", out_path]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("abi_consumer build failed:\n" + r.stderr)
    return out_path
