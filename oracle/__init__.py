"""fp64 CPU oracle for the KDA gated delta-rule recurrence.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package.  The product path
(``hybrid_prefix_cache_amd``) never imports, links or calls it, and the two share
no code.

``kda_oracle.c`` is the plain token-by-token definition of the recurrence (see its
header for the passages it follows); ``exact.py`` re-states the same definition and
its unrolled closed form over exact rationals for brute-force pins on tiny inputs.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import tempfile

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_oracle.c")
LIB_PATH = os.path.join(_HERE, "libkda_oracle.so")

F32, BF16, F64 = 0, 1, 2
_DT = {np.dtype(np.float32): F32, np.dtype(np.uint16): BF16, np.dtype(np.float64): F64}


def build(mutant: int = 0, out_path: str | None = None) -> str:
    """Compile the oracle with gcc (-O3, OpenMP).  ``mutant`` plants one of the
    deliberate mistakes listed in kda_oracle.c (0 = the real oracle)."""
    out = out_path or (LIB_PATH if mutant == 0 else
                       os.path.join(tempfile.mkdtemp(prefix="kda_mut"), f"libm{mutant}.so"))
    cmd = ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-std=c11",
           f"-DKDA_ORACLE_MUTANT={int(mutant)}", _SRC, "-o", out + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(out + ".tmp", out)
    return out


_libs: dict = {}


def load(path: str | None = None):
    path = path or LIB_PATH
    if path in _libs:
        return _libs[path]
    if not os.path.exists(path):
        if path == LIB_PATH:
            build()
        else:
            raise FileNotFoundError(path)
    lib = ctypes.CDLL(path)
    P = ctypes.c_void_p
    lib.kda_oracle_run.restype = ctypes.c_int
    lib.kda_oracle_run.argtypes = [
        ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P,
        ctypes.c_int32, ctypes.c_int32, P, P, P, P, P, P, P, P, P, P, P, P,
        ctypes.c_int32, ctypes.c_int32]
    lib.kda_oracle_mutant.restype = ctypes.c_int
    _libs[path] = lib
    return lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def run(q, k, v, g, beta, cu_seqlens, *, start_pos=None, s0=None, ckpt_cu=None,
        ckpt_pos=None, heads=None, gate_is_alpha=False, want_o=True, want_final=True,
        threads=0, lib_path=None):
    """Run the recurrence for every (sequence, selected head).

    q, k, g: [T, H, dk]; v: [T, H, dv]; beta: [T, H] -- all the same dtype
    (float32, float64, or uint16 holding bf16 bits).  ``g`` is log(alpha) unless
    ``gate_is_alpha``.  ``s0``: [num_seqs, n_sel, dk, dv] float64 or None (zero).
    Returns dict(o=[T, n_sel, dv], s_final=[num_seqs, n_sel, dk, dv],
    ckpts=[num_ckpts, n_sel, dk, dv]) in float64.
    """
    lib = load(lib_path)
    arrs = [np.ascontiguousarray(x) for x in (q, k, v, g, beta)]
    dt = arrs[0].dtype
    if any(a.dtype != dt for a in arrs) or dt not in _DT:
        raise TypeError("q, k, v, g, beta must share one dtype (float32, float64, uint16=bf16)")
    q, k, v, g, beta = arrs
    T, H, dk = q.shape
    dv = v.shape[2]
    if k.shape != (T, H, dk) or g.shape != (T, H, dk) or v.shape[:2] != (T, H) or beta.shape != (T, H):
        raise ValueError("shape mismatch")
    cu = np.ascontiguousarray(cu_seqlens, dtype=np.int64)
    ns = len(cu) - 1
    if cu[-1] != T:
        raise ValueError("cu_seqlens[-1] must equal T")
    sp = None if start_pos is None else np.ascontiguousarray(start_pos, dtype=np.int64)
    hs = None if heads is None else np.ascontiguousarray(heads, dtype=np.int32)
    n_sel = H if hs is None else len(hs)
    if s0 is not None:
        s0 = np.ascontiguousarray(s0, dtype=np.float64)
        if s0.shape != (ns, n_sel, dk, dv):
            raise ValueError(f"s0 must be {(ns, n_sel, dk, dv)}")
    o = np.empty((T, n_sel, dv), np.float64) if want_o else None
    sf = np.empty((ns, n_sel, dk, dv), np.float64) if want_final else None
    ccu = cpos = cout = None
    if ckpt_cu is not None:
        ccu = np.ascontiguousarray(ckpt_cu, dtype=np.int32)
        cpos = np.ascontiguousarray(ckpt_pos, dtype=np.int64)
        cout = np.empty((int(ccu[-1]), n_sel, dk, dv), np.float64)
    rc = lib.kda_oracle_run(H, dk, dv, ns, _ptr(cu), _ptr(sp), _DT[dt], int(bool(gate_is_alpha)),
                            _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(s0), _ptr(o),
                            _ptr(sf), _ptr(ccu), _ptr(cpos), _ptr(cout), _ptr(hs), n_sel,
                            int(threads))
    if rc != 0:
        raise ValueError(f"kda_oracle_run rejected its arguments (code {rc})")
    return {"o": o, "s_final": sf, "ckpts": cout}
