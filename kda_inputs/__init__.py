"""Seeded synthetic inputs for the KDA recurrence (test and bench infrastructure).

This module is shared by the oracle side and the HIP side: it only produces the
inputs both consume, and holds none of the method's arithmetic.  The random
source is the Philox4x32-10 counter-based generator (Salmon et al., SC'11)
implemented in ``kda_gen.c``; every element is a pure function of
(seed, stream, element index).

Distributions follow the workloads the pages' hot path is measured on
(32 heads, d = 128, contexts up to 1M tokens):

* q, k: i.i.d. N(0, 1) per channel, then L2-normalised per (token, head);
* v: N(0, 1);
* beta: sigmoid(N(0, 1)), one per (token, head);
* g = log(alpha): U(-0.05, 0) per channel;

all rounded once (round-to-nearest-even) to the stored dtype.  bf16 tensors are
numpy ``uint16`` arrays holding the bit patterns.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "kda_gen.c")
LIB_PATH = os.path.join(_HERE, "libkdagen.so")

F32, BF16, F64 = 0, 1, 2
NORMAL, UNIT_NORMAL, UNIFORM, SIGMOID_NORMAL = 0, 1, 2, 3
DTYPES = {"f32": (F32, np.float32), "bf16": (BF16, np.uint16), "f64": (F64, np.float64)}

# stream ids (low 8 bits) per tensor; bits 8.. carry the sequence / request id
TID_Q, TID_K, TID_V, TID_G, TID_BETA, TID_STATE, TID_PLAN = 1, 2, 3, 4, 5, 6, 7
TID_CONV_X, TID_CONV_W, TID_TOKENS = 8, 9, 10


def build() -> str:
    cmd = ["gcc", "-O3", "-fPIC", "-shared", "-fopenmp", "-std=c11", _SRC,
           "-o", LIB_PATH + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(LIB_PATH + ".tmp", LIB_PATH)
    return LIB_PATH


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            build()
        L = ctypes.CDLL(LIB_PATH)
        P, u64, u32, i64, i32, dbl = (ctypes.c_void_p, ctypes.c_uint64, ctypes.c_uint32,
                                      ctypes.c_int64, ctypes.c_int32, ctypes.c_double)
        L.kdagen_fill.restype = ctypes.c_int
        L.kdagen_fill.argtypes = [u64, u32, ctypes.c_int, dbl, dbl, dbl, i64, i64, i32, i32,
                                  ctypes.c_int, P, ctypes.c_int]
        L.kdagen_uniform.restype = ctypes.c_int
        L.kdagen_uniform.argtypes = [u64, u32, u64, i64, P]
        L.kdagen_normal.restype = ctypes.c_int
        L.kdagen_normal.argtypes = [u64, u32, u64, i64, P]
        L.kdagen_philox4x32_10.restype = None
        L.kdagen_philox4x32_10.argtypes = [P, P, P]
        L.kdagen_bf16_rne.restype = ctypes.c_uint16
        L.kdagen_bf16_rne.argtypes = [dbl]
        _lib = L
    return _lib


def philox4x32_10(ctr, key):
    c = np.ascontiguousarray(ctr, dtype=np.uint32)
    k = np.ascontiguousarray(key, dtype=np.uint32)
    out = np.zeros(4, np.uint32)
    lib().kdagen_philox4x32_10(c.ctypes.data, k.ctypes.data, out.ctypes.data)
    return out


def bf16_rne(x: float) -> int:
    return int(lib().kdagen_bf16_rne(float(x)))


def stream_id(tensor_id: int, seq_id: int = 0) -> int:
    return ((int(seq_id) & 0xFFFFFF) << 8) | (tensor_id & 0xFF)


def fill(seed, stream, kind, t0, nt, H, D, dtype="bf16", scale=1.0, lo=0.0, hi=1.0,
         out=None, threads=0):
    """Rows [t0, t0+nt) of a logical [T, H, D] tensor; returns [nt, H, D]."""
    code, npdt = DTYPES[dtype]
    if out is None:
        out = np.empty((nt, H, D), npdt)
    assert out.dtype == npdt and out.size == nt * H * D and out.flags.c_contiguous
    rc = lib().kdagen_fill(seed, stream, kind, scale, lo, hi, t0, nt, H, D, code,
                           out.ctypes.data, threads)
    if rc != 0:
        raise ValueError(f"kdagen_fill failed ({rc})")
    return out


def uniforms(seed, stream, first, n):
    out = np.empty(n, np.float64)
    lib().kdagen_uniform(seed, stream, first, n, out.ctypes.data)
    return out


def normals(seed, stream, first, n):
    out = np.empty(n, np.float64)
    lib().kdagen_normal(seed, stream, first, n, out.ctypes.data)
    return out


def kda_tokens(seed, H, D, t0, nt, dtype="bf16", seq_id=0, threads=0,
               g_lo=-0.05, g_hi=0.0):
    """q, k, v, g(=log alpha), beta for rows [t0, t0+nt) of one token stream."""
    sid = lambda t: stream_id(t, seq_id)  # noqa: E731
    return {
        "q": fill(seed, sid(TID_Q), UNIT_NORMAL, t0, nt, H, D, dtype, threads=threads),
        "k": fill(seed, sid(TID_K), UNIT_NORMAL, t0, nt, H, D, dtype, threads=threads),
        "v": fill(seed, sid(TID_V), NORMAL, t0, nt, H, D, dtype, threads=threads),
        "g": fill(seed, sid(TID_G), UNIFORM, t0, nt, H, D, dtype, lo=g_lo, hi=g_hi,
                  threads=threads),
        "beta": fill(seed, sid(TID_BETA), SIGMOID_NORMAL, t0, nt, H, 1, dtype,
                     threads=threads).reshape(nt, H),
    }


def random_states(seed, n, H, D, seq_id=0, threads=0):
    """n x H initial states, i.i.d. N(0, 1/D) fp32 -> float32 [n, H, D, D]."""
    st = fill(seed, stream_id(TID_STATE, seq_id), NORMAL, 0, n * H, D, D, "f32",
              scale=1.0 / np.sqrt(D), threads=threads)
    return st.reshape(n, H, D, D)


def conv_inputs(seed, T, C, dtype="bf16", threads=0):
    """Pre-convolution activations (one of the q, k, v projections): N(0, 1),
    [T, C] in the stored dtype."""
    H = next(h for h in range(1, C + 1) if C % h == 0 and C // h <= 1024)  # rows of <= 1024
    return fill(seed, stream_id(TID_CONV_X), NORMAL, 0, T, H, C // H, dtype,
                threads=threads).reshape(T, C)


def conv_weights(seed, C, W):
    """Short-convolution taps, N(0, 1/W) fp32 -> float32 [C, W]."""
    return fill(seed, stream_id(TID_CONV_W), NORMAL, 0, C, 1, W, "f32",
                scale=1.0 / np.sqrt(W)).reshape(C, W)


def token_ids(seed, n, vocab=163_840, seq_id=0):
    """n token ids, uniform over [0, vocab) (int32), for prefix-index workloads."""
    u = uniforms(seed, stream_id(TID_TOKENS, seq_id), 0, n)
    return np.minimum((u * vocab).astype(np.int64), vocab - 1).astype(np.int32)


from .workloads import *  # noqa: E402,F401,F403
