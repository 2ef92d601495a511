"""Build libkda_san.so: libkda with AddressSanitizer and UndefinedBehaviorSanitizer
on the host code (argument validation, metadata tables, window planning, the
prefix index); device code is built as usual.  For CPU test runs only:

    python hybrid_prefix_cache_amd/build_sanitized.py
    KDA_LIBRARY=hybrid_prefix_cache_amd/libkda_san.so \\
    LD_PRELOAD=$(/opt/rocm/llvm/bin/clang++ -print-file-name=libclang_rt.asan-x86_64.so) \\
    ASAN_OPTIONS=detect_leaks=0 UBSAN_OPTIONS=halt_on_error=1:print_stacktrace=1 \\
    python -m pytest tests -m "not gpu" -q

(the Python interpreter is not instrumented, so the sanitizer runtime is
preloaded; leak detection is off because the interpreter keeps its objects
alive at exit).
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, HERE)
import build as B  # noqa: E402

BUILD = os.path.join(HERE, "_build_san")
LIB = os.path.join(HERE, "libkda_san.so")
# each sanitizer flag applies to the host compilation only
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]


def _compile(src: str) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = ["hipcc", *B.FLAGS, *HOST_SAN, "-c", os.path.join(B.CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr}")
    return obj


def build() -> str:
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, len(B.SOURCES))) as ex:
        objs = list(ex.map(_compile, B.SOURCES))
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    cmd = [os.path.join(rocm, "llvm", "bin", "clang++"), "-shared", "-fPIC", "-shared-libsan",
           "-fsanitize=address,undefined", *objs, f"-L{rocm}/lib", "-lamdhip64",
           f"-Wl,-rpath,{rocm}/lib", "-o", LIB + ".tmp"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr}")
    os.replace(LIB + ".tmp", LIB)
    return LIB


if __name__ == "__main__":
    print(build())
