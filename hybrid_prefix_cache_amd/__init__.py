"""Python binding of libkda (KDA gated delta-rule recurrence on MI355X / gfx950).

Argument marshalling only: every step of the recurrence runs in the HIP kernels
of ``libkda.so``; this module turns torch tensors / numpy arrays into pointers,
sizes and the current HIP stream, calls the C ABI declared in ``include/kda.h``
under the same names, and raises ``KdaError`` on a non-zero status.  There is no
CPU fallback: importing fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
# torch first: it ships its own HIP runtime under the same soname as the one
# libkda.so is linked against, and the first one loaded serves the whole
# process.  Loading libkda first would pair torch with a runtime of another
# ROCm release (kernel launches then fail with "no ROCm-capable device").
import torch  # noqa: F401  (device memory and streams)

_HERE = os.path.dirname(os.path.abspath(__file__))
# KDA_LIBRARY selects another build of the same library (the sanitizer build
# of build_sanitized.py for CPU test runs)
LIB_PATH = os.environ.get("KDA_LIBRARY") or os.path.join(_HERE, "libkda.so")

KDA_OK, KDA_ERR_NULL, KDA_ERR_SHAPE, KDA_ERR_DTYPE = 0, 1, 2, 3
KDA_ERR_PAGE_RANGE, KDA_ERR_PAGE_ALIAS, KDA_ERR_CKPT_ALIGN, KDA_ERR_CKPT_RANGE = 4, 5, 6, 7
KDA_ERR_SEQ, KDA_ERR_WORKSPACE, KDA_ERR_HIP, KDA_ERR_POOL = 8, 9, 10, 11
KDA_ERR_PINNED, KDA_ERR_NOT_FOUND = 12, 13
STATUS_NAMES = {0: "KDA_OK", 1: "KDA_ERR_NULL", 2: "KDA_ERR_SHAPE", 3: "KDA_ERR_DTYPE",
                4: "KDA_ERR_PAGE_RANGE", 5: "KDA_ERR_PAGE_ALIAS", 6: "KDA_ERR_CKPT_ALIGN",
                7: "KDA_ERR_CKPT_RANGE", 8: "KDA_ERR_SEQ", 9: "KDA_ERR_WORKSPACE",
                10: "KDA_ERR_HIP", 11: "KDA_ERR_POOL", 12: "KDA_ERR_PINNED",
                13: "KDA_ERR_NOT_FOUND"}
KDA_F32, KDA_BF16 = 0, 1
HASH_BLOCK = 512
CHUNK = 64

EXPORTS = ("kda_version", "kda_last_error", "kda_pool_check", "kda_state_offset",
           "kda_prefill_workspace_bytes", "kda_prefill_workspace_min_bytes", "kda_prefill_chunked",
           "kda_prefill_chunked_noalloc", "kda_decode_step", "kda_decode_verify",
           "kda_checkpoint_write", "kda_checkpoint_restore", "kda_ckpt_int8_head_bytes",
           "kda_checkpoint_write_int8", "kda_checkpoint_restore_int8",
           "kda_conv_workspace_bytes", "kda_short_conv", "kda_short_conv_update", "kda_profile_enable", "kda_profile_read",
           "kda_xxh64", "kda_chain_hashes", "kda_ckpt_plan", "kda_index_create",
           "kda_index_destroy", "kda_index_register_pages", "kda_index_register_ckpt",
           "kda_index_mark_ready", "kda_index_lookup", "kda_index_release", "kda_index_evict_page",
           "kda_index_evict_ckpt", "kda_index_stats")


class KdaError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


class kda_pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("page_bytes", ctypes.c_int64),
                ("num_pages", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("d_k", ctypes.c_int32), ("d_v", ctypes.c_int32)]


class kda_conv_pool(ctypes.Structure):
    _fields_ = [("base", ctypes.c_void_p), ("page_bytes", ctypes.c_int64),
                ("num_pages", ctypes.c_int32), ("channels", ctypes.c_int32),
                ("width", ctypes.c_int32), ("dtype", ctypes.c_int32)]


class kda_hit(ctypes.Structure):
    _fields_ = [("boundary", ctypes.c_int64), ("mla_tokens", ctypes.c_int64),
                ("num_pages", ctypes.c_int32), ("pad", ctypes.c_int32),
                ("pin_handle", ctypes.c_int64)]


class kda_kernel_stat(ctypes.Structure):
    _fields_ = [("name", ctypes.c_char * 48), ("launches", ctypes.c_int64),
                ("total_ms", ctypes.c_double)]


if not os.path.exists(LIB_PATH):
    raise ImportError(f"libkda.so is not built ({LIB_PATH}); run "
                      "`python hybrid_prefix_cache_amd/build.py` (hipcc, gfx950)")
_lib = ctypes.CDLL(LIB_PATH)

_P, _i32, _i64, _sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
_PP = ctypes.POINTER(kda_pool)
_sig = {
    "kda_version": (_i32, []),
    "kda_last_error": (ctypes.c_char_p, []),
    "kda_pool_check": (ctypes.c_int, [_PP]),
    "kda_state_offset": (_i64, [_PP, _i32, _i32]),
    "kda_prefill_workspace_bytes": (_sz, [_PP, _i64, _i32, _i32, ctypes.c_int]),
    "kda_prefill_workspace_min_bytes": (_sz, [_PP, _i32, _i32, ctypes.c_int]),
    "kda_prefill_chunked": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int,
                                           _i32, _P, _P, _P, _P, _P, _P, _P, _i32, _i32, _P, _sz,
                                           _P]),
    "kda_prefill_chunked_noalloc": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, ctypes.c_int, _P,
                                                    ctypes.c_int, _i32, _P, _P, _P, _P, _P, _P, _P,
                                                    _i32, _i32, _P]),
    "kda_decode_step": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int,
                                       _i32, _P, _P, _P]),
    "kda_decode_verify": (ctypes.c_int, [_PP, _P, _P, _P, _P, _P, ctypes.c_int, _P, ctypes.c_int,
                                         _i32, _i32, _P, _P, _P]),
    "kda_checkpoint_write": (ctypes.c_int, [_PP, _P, _P, _i32, _P]),
    "kda_checkpoint_restore": (ctypes.c_int, [_PP, _P, _P, _i32, _P]),
    "kda_ckpt_int8_head_bytes": (ctypes.c_int64, [_i32, _i32]),
    "kda_checkpoint_write_int8": (ctypes.c_int, [_PP, _P, _PP, _P, _i32, _P]),
    "kda_checkpoint_restore_int8": (ctypes.c_int, [_PP, _P, _PP, _P, _i32, _P]),
    "kda_conv_workspace_bytes": (_i64, [_i32, _i32]),
    "kda_short_conv": (ctypes.c_int, [ctypes.POINTER(kda_conv_pool), _P, _P, _P, ctypes.c_int, _i32,
                                      _P, _P, _P, _P, _P, _P, _P, _i32, _P, _sz, _P]),
    "kda_short_conv_update": (ctypes.c_int, [ctypes.POINTER(kda_conv_pool), _P, _P, _P, ctypes.c_int,
                                             _i32, _P, _P, _P]),
    "kda_xxh64": (ctypes.c_uint64, [_P, _i64, ctypes.c_uint64]),
    "kda_chain_hashes": (_i64, [_P, _i64, _i32, ctypes.c_uint64, _P, _i64]),
    "kda_ckpt_plan": (_i64, [_i64, _i64, _i32]),
    "kda_index_create": (_P, [_i32, _i32, _i32, ctypes.c_uint64]),
    "kda_index_destroy": (None, [_P]),
    "kda_index_register_pages": (ctypes.c_int, [_P, _P, _i64, _P, _i32, _i64, _P]),
    "kda_index_register_ckpt": (ctypes.c_int, [_P, _P, _i64, _i32, _i32, _i32, _i64, _P]),
    "kda_index_mark_ready": (ctypes.c_int, [_P, _i64]),
    "kda_index_lookup": (ctypes.c_int, [_P, _P, _i64, _i32, _P, _i32, _P,
                                        ctypes.POINTER(kda_hit)]),
    "kda_index_release": (ctypes.c_int, [_P, _i64]),
    "kda_index_evict_page": (ctypes.c_int, [_P, _i32]),
    "kda_index_evict_ckpt": (ctypes.c_int, [_P, _i32, _i32, _P]),
    "kda_index_stats": (ctypes.c_int, [_P, _P, _P, _P]),
    "kda_profile_enable": (ctypes.c_int, [_i32]),
    "kda_profile_read": (_i32, [ctypes.POINTER(kda_kernel_stat), _i32, _i32]),
}
for _name, (_res, _args) in _sig.items():
    _f = getattr(_lib, _name)
    _f.restype = _res
    _f.argtypes = _args


# ---------------------------------------------------------------------------
# marshalling helpers
# ---------------------------------------------------------------------------
def _dptr(x):
    """Device pointer of a CUDA/HIP torch tensor (must be contiguous), an int,
    or None."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not x.is_cuda:
        raise ValueError("expected a device tensor")
    if not x.is_contiguous():
        raise ValueError("device tensors must be contiguous")
    return x.data_ptr()


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return KDA_BF16
    if t.dtype == torch.float32:
        return KDA_F32
    raise ValueError(f"unsupported dtype {t.dtype} (bfloat16 or float32)")


class _HostArr:
    """Keeps a contiguous numpy copy alive while its pointer is in use."""

    def __init__(self, x, dtype):
        self.a = None if x is None else np.ascontiguousarray(np.asarray(x), dtype=dtype)

    @property
    def ptr(self):
        return None if self.a is None else self.a.ctypes.data_as(ctypes.c_void_p)


def _need_len(name, arr, n):
    """Raise ValueError unless the host array `arr` (a _HostArr, possibly None)
    holds exactly n entries: the C side reads n entries through its pointer."""
    if arr.a is not None and (arr.a.ndim != 1 or len(arr.a) != n):
        raise ValueError(f"{name} must hold {n} entries (got shape {arr.a.shape})")


def _seq_meta_lengths(ns, sp, si, so, ccu, cpos, cpg):
    """Length checks of the per-sequence and checkpoint host arrays shared by
    kda_prefill_chunked and kda_short_conv."""
    for name, arr in (("start_pos", sp), ("state_in_page", si), ("state_out_page", so)):
        _need_len(name, arr, ns)
    if ccu.a is None:
        if cpos.a is not None or cpg.a is not None:
            raise ValueError("ckpt_pos / ckpt_page given without ckpt_cu")
        return
    _need_len("ckpt_cu", ccu, ns + 1)
    nck = int(ccu.a[-1]) if ns >= 0 else 0
    if nck > 0 and (cpos.a is None or cpg.a is None):
        raise ValueError("ckpt_pos and ckpt_page are required when ckpt_cu is given")
    if nck < 0:
        raise ValueError("ckpt_cu[-1] must be non-negative")
    for name, arr in (("ckpt_pos", cpos), ("ckpt_page", cpg)):
        if arr.a is not None and (arr.a.ndim != 1 or len(arr.a) < nck):
            raise ValueError(f"{name} must hold ckpt_cu[-1] = {nck} entries (got shape {arr.a.shape})")


def _stream(stream):
    if stream is None:
        import torch
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, int):
        return ctypes.c_void_p(stream)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(status: int):
    if status != KDA_OK:
        raise KdaError(status, kda_last_error())


def make_pool(base, page_bytes: int, num_pages: int, num_heads: int, d_k: int, d_v: int | None = None):
    """Pool descriptor over caller-owned device memory (a torch tensor or a raw
    device pointer)."""
    return kda_pool(_dptr(base), int(page_bytes), int(num_pages), int(num_heads), int(d_k),
                    int(d_k if d_v is None else d_v))


def make_conv_pool(base, page_bytes: int, num_pages: int, channels: int, width: int, dtype: int):
    """Conv-window pool descriptor over caller-owned device memory."""
    return kda_conv_pool(_dptr(base), int(page_bytes), int(num_pages), int(channels), int(width),
                         int(dtype))


# ---------------------------------------------------------------------------
# the C ABI under the same names
# ---------------------------------------------------------------------------
def kda_version() -> int:
    return int(_lib.kda_version())


def kda_last_error() -> str:
    return _lib.kda_last_error().decode()


def kda_pool_check(pool: kda_pool) -> int:
    return int(_lib.kda_pool_check(ctypes.byref(pool)))


def kda_state_offset(pool: kda_pool, page: int, head: int) -> int:
    return int(_lib.kda_state_offset(ctypes.byref(pool), page, head))


def kda_prefill_workspace_bytes(pool: kda_pool, total_tokens: int, num_seqs: int, num_ckpts: int,
                                in_dtype: int) -> int:
    return int(_lib.kda_prefill_workspace_bytes(ctypes.byref(pool), total_tokens, num_seqs,
                                                num_ckpts, in_dtype))


def kda_prefill_workspace_min_bytes(pool: kda_pool, num_seqs: int, num_ckpts: int,
                                    in_dtype: int) -> int:
    return int(_lib.kda_prefill_workspace_min_bytes(ctypes.byref(pool), num_seqs, num_ckpts,
                                                    in_dtype))


def kda_prefill_chunked(pool, q, k, v, g, beta, o, cu_seqlens, *, start_pos=None,
                        state_in_page=None, state_out_page=None, ckpt_cu=None, ckpt_pos=None,
                        ckpt_page=None, workspace=None, workspace_bytes=None, chunk_size=CHUNK,
                        hash_block=HASH_BLOCK, in_dtype=None, out_dtype=None, stream=None):
    """q, k, g: [T, H, d_k]; v, o: [T, H, d_v]; beta: [T, H] (device tensors).
    Host metadata as sequences / numpy arrays (see include/kda.h).  The
    workspace is a device tensor (uint8) of at least kda_prefill_workspace_bytes."""
    cu = _HostArr(cu_seqlens, np.int64)
    ns = len(cu.a) - 1
    sp = _HostArr(start_pos, np.int64)
    si = _HostArr(state_in_page, np.int32)
    so = _HostArr(state_out_page, np.int32)
    ccu = _HostArr(ckpt_cu, np.int32)
    cpos = _HostArr(ckpt_pos, np.int64)
    cpg = _HostArr(ckpt_page, np.int32)
    _seq_meta_lengths(ns, sp, si, so, ccu, cpos, cpg)
    ind = _dtype_code(q) if in_dtype is None else in_dtype
    outd = _dtype_code(o) if out_dtype is None else out_dtype
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else (
            workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0)
    st = _lib.kda_prefill_chunked(ctypes.byref(pool), _dptr(q), _dptr(k), _dptr(v), _dptr(g),
                                  _dptr(beta), ind, _dptr(o), outd, ns, cu.ptr, sp.ptr, si.ptr,
                                  so.ptr, ccu.ptr, cpos.ptr, cpg.ptr, chunk_size, hash_block,
                                  _dptr(workspace), workspace_bytes, _stream(stream))
    _check(st)


def kda_prefill_chunked_noalloc(pool, q, k, v, g, beta, o, cu_seqlens, *, start_pos=None,
                                state_in_page=None, state_out_page=None, ckpt_cu=None,
                                ckpt_pos=None, ckpt_page=None, chunk_size=CHUNK,
                                hash_block=HASH_BLOCK, in_dtype=None, out_dtype=None, stream=None):
    """kda_prefill_chunked on the library's static device scratch (no workspace
    argument; see include/kda.h)."""
    cu = _HostArr(cu_seqlens, np.int64)
    ns = len(cu.a) - 1
    sp = _HostArr(start_pos, np.int64)
    si = _HostArr(state_in_page, np.int32)
    so = _HostArr(state_out_page, np.int32)
    ccu = _HostArr(ckpt_cu, np.int32)
    cpos = _HostArr(ckpt_pos, np.int64)
    cpg = _HostArr(ckpt_page, np.int32)
    _seq_meta_lengths(ns, sp, si, so, ccu, cpos, cpg)
    ind = _dtype_code(q) if in_dtype is None else in_dtype
    outd = _dtype_code(o) if out_dtype is None else out_dtype
    st = _lib.kda_prefill_chunked_noalloc(ctypes.byref(pool), _dptr(q), _dptr(k), _dptr(v),
                                          _dptr(g), _dptr(beta), ind, _dptr(o), outd, ns, cu.ptr,
                                          sp.ptr, si.ptr, so.ptr, ccu.ptr, cpos.ptr, cpg.ptr,
                                          chunk_size, hash_block, _stream(stream))
    _check(st)


def kda_decode_step(pool, q, k, v, g, beta, o, page_in, page_out, *, n=None, in_dtype=None,
                    out_dtype=None, stream=None):
    """q, k, g: [n, H, d_k]; v, o: [n, H, d_v]; beta: [n, H]; page_in/page_out:
    int32 device tensors [n]."""
    n = int(page_in.numel()) if n is None else n
    ind = _dtype_code(q) if in_dtype is None else in_dtype
    outd = _dtype_code(o) if out_dtype is None else out_dtype
    st = _lib.kda_decode_step(ctypes.byref(pool), _dptr(q), _dptr(k), _dptr(v), _dptr(g),
                              _dptr(beta), ind, _dptr(o), outd, n, _dptr(page_in),
                              _dptr(page_out), _stream(stream))
    _check(st)


def kda_decode_verify(pool, q, k, v, g, beta, o, tokens, page_in, page_out, *, n=None,
                      in_dtype=None, out_dtype=None, stream=None):
    """`tokens` consecutive tokens per request, every intermediate state kept.
    q, k, g: [n*tokens, H, d_k]; v, o: [n*tokens, H, d_v]; beta: [n*tokens, H];
    page_in: int32 device [n]; page_out: int32 device [n*tokens]."""
    n = int(page_in.numel()) if n is None else n
    ind = _dtype_code(q) if in_dtype is None else in_dtype
    outd = _dtype_code(o) if out_dtype is None else out_dtype
    st = _lib.kda_decode_verify(ctypes.byref(pool), _dptr(q), _dptr(k), _dptr(v), _dptr(g),
                                _dptr(beta), ind, _dptr(o), outd, n, int(tokens), _dptr(page_in),
                                _dptr(page_out), _stream(stream))
    _check(st)


def kda_checkpoint_write(pool, src_active, dst_ckpt, *, stream=None):
    s, d = _HostArr(src_active, np.int32), _HostArr(dst_ckpt, np.int32)
    _need_len("dst_ckpt", d, len(s.a))
    _check(_lib.kda_checkpoint_write(ctypes.byref(pool), s.ptr, d.ptr, len(s.a), _stream(stream)))


def kda_checkpoint_restore(pool, src_ckpt, dst_active, *, stream=None):
    s, d = _HostArr(src_ckpt, np.int32), _HostArr(dst_active, np.int32)
    _need_len("dst_active", d, len(s.a))
    _check(_lib.kda_checkpoint_restore(ctypes.byref(pool), s.ptr, d.ptr, len(s.a), _stream(stream)))


def kda_ckpt_int8_head_bytes(d_k: int, d_v: int) -> int:
    """Bytes of one head in a compressed (int8) checkpoint page; -1 if unsupported."""
    return int(_lib.kda_ckpt_int8_head_bytes(d_k, d_v))


def kda_checkpoint_write_int8(pool, src_active, qpool, dst_qckpt, *, stream=None):
    s, d = _HostArr(src_active, np.int32), _HostArr(dst_qckpt, np.int32)
    _need_len("dst_qckpt", d, len(s.a))
    _check(_lib.kda_checkpoint_write_int8(ctypes.byref(pool), s.ptr, ctypes.byref(qpool), d.ptr,
                                          len(s.a), _stream(stream)))


def kda_checkpoint_restore_int8(qpool, src_qckpt, pool, dst_active, *, stream=None):
    s, d = _HostArr(src_qckpt, np.int32), _HostArr(dst_active, np.int32)
    _need_len("dst_active", d, len(s.a))
    _check(_lib.kda_checkpoint_restore_int8(ctypes.byref(qpool), s.ptr, ctypes.byref(pool), d.ptr,
                                            len(s.a), _stream(stream)))


def kda_conv_workspace_bytes(num_seqs: int, num_ckpts: int) -> int:
    return int(_lib.kda_conv_workspace_bytes(num_seqs, num_ckpts))


def kda_short_conv(cpool, x, w, y, cu_seqlens, *, start_pos=None, state_in_page=None,
                   state_out_page=None, ckpt_cu=None, ckpt_pos=None, ckpt_page=None,
                   hash_block=HASH_BLOCK, workspace=None, workspace_bytes=None, out_dtype=None,
                   stream=None):
    """x, y: [T, C] device tensors (x in the pool's dtype); w: [C, W] fp32 device
    tensor; host metadata as for kda_prefill_chunked.  The workspace is a device
    uint8 tensor of at least kda_conv_workspace_bytes."""
    cu = _HostArr(cu_seqlens, np.int64)
    ns = len(cu.a) - 1
    sp = _HostArr(start_pos, np.int64)
    si = _HostArr(state_in_page, np.int32)
    so = _HostArr(state_out_page, np.int32)
    ccu = _HostArr(ckpt_cu, np.int32)
    cpos = _HostArr(ckpt_pos, np.int64)
    cpg = _HostArr(ckpt_page, np.int32)
    _seq_meta_lengths(ns, sp, si, so, ccu, cpos, cpg)
    outd = _dtype_code(y) if out_dtype is None else out_dtype
    if workspace_bytes is None:
        workspace_bytes = 0 if workspace is None else (
            workspace.numel() * workspace.element_size() if hasattr(workspace, "numel") else 0)
    st = _lib.kda_short_conv(ctypes.byref(cpool), _dptr(x), _dptr(w), _dptr(y), outd, ns, cu.ptr,
                             sp.ptr, si.ptr, so.ptr, ccu.ptr, cpos.ptr, cpg.ptr, hash_block,
                             _dptr(workspace), workspace_bytes, _stream(stream))
    _check(st)


def kda_short_conv_update(cpool, x, w, y, page_in, page_out, *, n=None, out_dtype=None,
                          stream=None):
    """One token per request: x, y [n, C] device tensors, w [C, W] fp32 device
    tensor, page_in / page_out int32 device tensors [n]."""
    n = int(page_in.numel()) if n is None else n
    outd = _dtype_code(y) if out_dtype is None else out_dtype
    st = _lib.kda_short_conv_update(ctypes.byref(cpool), _dptr(x), _dptr(w), _dptr(y), outd, n,
                                    _dptr(page_in), _dptr(page_out), _stream(stream))
    _check(st)


# ---- host prefix index (include/kda_index.h) --------------------------------
def _tok(tokens):
    return _HostArr(tokens, np.int32)


def kda_xxh64(data: bytes, seed: int = 0) -> int:
    buf = ctypes.create_string_buffer(bytes(data), len(data))
    return int(_lib.kda_xxh64(buf, len(data), seed))


def kda_chain_hashes(tokens, hash_block: int = HASH_BLOCK, seed: int = 0) -> np.ndarray:
    t = _tok(tokens)
    n = 0 if t.a is None else t.a.size
    out = np.zeros(max(n // hash_block, 1), np.uint64)
    got = _lib.kda_chain_hashes(t.ptr, n, hash_block, seed, out.ctypes.data, n // hash_block)
    if got < 0:
        raise ValueError("kda_chain_hashes: bad arguments")
    return out[:got]


def kda_ckpt_plan(start: int, length: int, hash_block: int = HASH_BLOCK) -> int:
    return int(_lib.kda_ckpt_plan(start, length, hash_block))


class PrefixIndex:
    """Handle of a kda_index (pointer plus the shape the marshalling needs)."""

    def __init__(self, ptr, hash_block, physical_block, num_groups):
        self.ptr, self.hash_block, self.physical_block = ptr, hash_block, physical_block
        self.num_groups = num_groups

    def __del__(self, _destroy=_lib.kda_index_destroy):
        if getattr(self, "ptr", None):
            _destroy(self.ptr)
            self.ptr = None


def kda_index_create(hash_block: int = HASH_BLOCK, physical_block: int = 6144,
                     num_groups: int = 1, namespace_seed: int = 0) -> PrefixIndex:
    p = _lib.kda_index_create(hash_block, physical_block, num_groups, namespace_seed)
    if not p:
        raise KdaError(KDA_ERR_SHAPE, kda_last_error())
    return PrefixIndex(p, hash_block, physical_block, num_groups)


def kda_index_destroy(idx: PrefixIndex):
    idx.__del__()


def kda_index_register_pages(idx: PrefixIndex, tokens, pages, step: int = 0) -> np.ndarray:
    t, pg = _tok(tokens), _HostArr(pages, np.int32)
    n = 0 if t.a is None else t.a.size
    npg = 0 if pg.a is None else pg.a.size
    taken = np.zeros(max(npg, 1), np.int32)
    _check(_lib.kda_index_register_pages(idx.ptr, t.ptr, n, pg.ptr, npg, step, taken.ctypes.data))
    return taken[:npg]


def kda_index_register_ckpt(idx: PrefixIndex, tokens, pos: int, group: int, page: int,
                            durable: bool = False, step: int = 0) -> bool:
    t = _tok(tokens)
    taken = ctypes.c_int32(0)
    _check(_lib.kda_index_register_ckpt(idx.ptr, t.ptr, pos, group, page, int(durable), step,
                                        ctypes.byref(taken)))
    return bool(taken.value)


def kda_index_mark_ready(idx: PrefixIndex, step: int):
    _check(_lib.kda_index_mark_ready(idx.ptr, step))


def kda_index_lookup(idx: PrefixIndex, tokens, pin: bool = False, max_pages=None) -> dict:
    t = _tok(tokens)
    n = 0 if t.a is None else t.a.size
    if max_pages is None:
        max_pages = n // idx.physical_block + 1
    pages = np.zeros(max(max_pages, 1), np.int32)
    ck = np.zeros(idx.num_groups, np.int32)
    hit = kda_hit()
    _check(_lib.kda_index_lookup(idx.ptr, t.ptr, n, int(pin), pages.ctypes.data, max_pages,
                                 ck.ctypes.data, ctypes.byref(hit)))
    return {"boundary": hit.boundary, "mla_tokens": hit.mla_tokens,
            "pages": pages[:hit.num_pages].tolist(), "ckpt_pages": ck.tolist(),
            "pin_handle": hit.pin_handle}


def kda_index_release(idx: PrefixIndex, pin_handle: int):
    _check(_lib.kda_index_release(idx.ptr, pin_handle))


def kda_index_evict_page(idx: PrefixIndex, page: int):
    _check(_lib.kda_index_evict_page(idx.ptr, page))


def kda_index_evict_ckpt(idx: PrefixIndex, group: int, page: int) -> list:
    freed = np.zeros(idx.num_groups, np.int32)
    _check(_lib.kda_index_evict_ckpt(idx.ptr, group, page, freed.ctypes.data))
    return freed.tolist()


def kda_index_stats(idx: PrefixIndex):
    a, b, c = ctypes.c_int64(), ctypes.c_int64(), ctypes.c_int64()
    _check(_lib.kda_index_stats(idx.ptr, ctypes.byref(a), ctypes.byref(b), ctypes.byref(c)))
    return a.value, b.value, c.value


def kda_profile_enable(on: bool = True):
    _check(_lib.kda_profile_enable(1 if on else 0))


def kda_profile_read(reset: bool = True) -> dict:
    """{kernel name: (launches, total_ms)} since the last reset (synchronises
    the recorded events)."""
    n = _lib.kda_profile_read(None, 0, 0)
    arr = (kda_kernel_stat * max(1, n))()
    got = _lib.kda_profile_read(arr, n, 1 if reset else 0)
    return {arr[i].name.decode(): (int(arr[i].launches), float(arr[i].total_ms)) for i in range(got)}


def raw_call(name: str, *args):
    """Direct access to an exported symbol (for ABI tests)."""
    return getattr(_lib, name)(*args)
