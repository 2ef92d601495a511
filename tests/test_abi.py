"""C-ABI checks that need no GPU: the library loads, exports every function
include/kda.h declares, computes pool offsets, and rejects bad arguments with
the documented status before touching the device (all-or-nothing).

Device pointers below are fake aligned integers: every call here fails
validation, so none of them is ever dereferenced.
"""
import ctypes
import os
import re

import numpy as np
import pytest

import hybrid_prefix_cache_amd as K

INC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include")
HDRS = [os.path.join(INC, f) for f in sorted(os.listdir(INC)) if f.endswith(".h")]
FAKE = 1 << 20  # 256-byte aligned, never dereferenced
MiB2 = 2 << 20


def declared_functions():
    """Every function any include/*.h declares (type names are not followed by '(')."""
    names = set()
    for h in HDRS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(kda_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_exports_every_declared_symbol():
    names = declared_functions()
    assert set(names) >= {"kda_prefill_chunked", "kda_decode_step", "kda_checkpoint_write",
                          "kda_checkpoint_restore", "kda_short_conv", "kda_index_lookup"}
    lib = ctypes.CDLL(K.LIB_PATH)
    missing = [n for n in names if not hasattr(lib, n)]
    assert not missing, f"not exported: {missing}"
    assert set(names) == set(K.EXPORTS)


def test_probe_library_exports_and_rejects():
    """libkda_probe.so (the benchmark's peak probes, not part of the API) loads,
    exports its three probes, and rejects bad sizes before any launch."""
    lib = ctypes.CDLL(os.path.join(os.path.dirname(K.LIB_PATH), "libkda_probe.so"))
    for n in ("kda_probe_mfma_bf16", "kda_probe_copy", "kda_probe_fill"):
        assert hasattr(lib, n), n
    lib.kda_probe_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.kda_probe_fill.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_uint32, ctypes.c_void_p]
    lib.kda_probe_mfma_bf16.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_void_p]
    assert lib.kda_probe_copy(FAKE, FAKE, 4096 + 16, None) != 0      # not whole 4 KiB pieces
    assert lib.kda_probe_copy(FAKE + 8, FAKE, 4096, None) != 0       # misaligned
    assert lib.kda_probe_fill(FAKE, 0, 0, None) != 0
    assert lib.kda_probe_mfma_bf16(FAKE, 0, 10, None) != 0


def pool(**kw):
    d = dict(base=FAKE, page_bytes=MiB2, num_pages=16, num_heads=32, d_k=128)
    d.update(kw)
    return K.make_pool(**d)


@pytest.mark.parametrize("kw,status", [
    ({}, K.KDA_OK),
    (dict(base=0), K.KDA_ERR_POOL),
    (dict(base=FAKE + 16), K.KDA_ERR_POOL),
    (dict(d_k=96), K.KDA_ERR_SHAPE),
    (dict(d_k=128, d_v=64), K.KDA_ERR_SHAPE),
    (dict(page_bytes=MiB2 - 256), K.KDA_ERR_POOL),   # smaller than 32 heads x 64 KiB
    (dict(page_bytes=MiB2 + 8), K.KDA_ERR_POOL),     # not a multiple of 256
    (dict(page_bytes=MiB2 + 4096), K.KDA_OK),
    (dict(num_pages=0), K.KDA_ERR_POOL),
    (dict(num_heads=0), K.KDA_ERR_POOL),
])
def test_pool_check(kw, status):
    assert K.kda_pool_check(pool(**kw)) == status
    if status != K.KDA_OK:
        assert K.kda_last_error() != ""
    else:
        assert K.kda_last_error() == ""


def test_pool_check_null():
    assert K.raw_call("kda_pool_check", None) == K.KDA_ERR_NULL


def test_state_offset_layout():
    # heads stored contiguously inside a page; pages of a fixed byte size
    p = pool(page_bytes=MiB2 + 4096, num_pages=8, num_heads=32, d_k=128)
    for page in (0, 1, 7):
        for head in (0, 1, 31):
            assert K.kda_state_offset(p, page, head) == page * (MiB2 + 4096) + head * 128 * 128 * 4
    assert K.kda_state_offset(p, 8, 0) == -1
    assert K.kda_state_offset(p, 0, 32) == -1
    assert K.kda_state_offset(p, -1, 0) == -1
    p64 = pool(num_heads=1, d_k=64, page_bytes=16384, num_pages=4)
    assert K.kda_state_offset(p64, 3, 0) == 3 * 16384


def test_workspace_bytes():
    p = pool()
    a = K.kda_prefill_workspace_bytes(p, 8192, 1, 3, K.KDA_BF16)
    b = K.kda_prefill_workspace_bytes(p, 8192, 1, 3, K.KDA_F32)
    assert a > 0 and b > a
    # per (chunk, head): 3 x [64][128] + 2 x [64][64] elements + fp32 gamma, 256-aligned
    blk = ((3 * 64 * 128 + 2 * 64 * 64) * 2 + 4 * 128 + 255) // 256 * 256
    assert a >= 64 * 32 * blk  # one window of 64 chunks
    assert K.kda_prefill_workspace_bytes(p, 8192, 2, 3, K.KDA_BF16) >= a
    # the workspace holds one window (2048 (chunk, head) blocks), not the
    # whole call: a 1M-token call needs no more than an 8K one
    big = K.kda_prefill_workspace_bytes(p, 1 << 20, 1, 170, K.KDA_BF16)
    assert big <= a + 4096 and big < 1 << 30
    assert K.kda_prefill_workspace_bytes(p, 64, 1, 0, K.KDA_BF16) < a // 16  # short calls stay small
    assert K.kda_prefill_workspace_bytes(p, -1, 1, 0, K.KDA_BF16) == 0
    assert K.kda_prefill_workspace_bytes(p, 10, 1, 0, 7) == 0


def _prefill_status(p=None, T=1024, **kw):
    """Call kda_prefill_chunked with fake device pointers; returns the status."""
    p = p or pool()
    args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE, cu_seqlens=[0, T],
                in_dtype=K.KDA_BF16, out_dtype=K.KDA_BF16, workspace=FAKE,
                workspace_bytes=1 << 40, stream=0)
    args.update(kw)
    try:
        K.kda_prefill_chunked(p, **args)
    except K.KdaError as e:
        assert K.kda_last_error() != ""
        return e.status
    return K.KDA_OK


@pytest.mark.parametrize("kw,status", [
    (dict(chunk_size=32), K.KDA_ERR_SHAPE),
    (dict(hash_block=500), K.KDA_ERR_SHAPE),
    (dict(hash_block=0), K.KDA_ERR_SHAPE),
    (dict(in_dtype=5), K.KDA_ERR_DTYPE),
    (dict(out_dtype=-1), K.KDA_ERR_DTYPE),
    (dict(cu_seqlens=[1, 1024]), K.KDA_ERR_SEQ),
    (dict(cu_seqlens=[0, 512, 256]), K.KDA_ERR_SEQ),
    (dict(start_pos=[100]), K.KDA_ERR_SEQ),
    (dict(start_pos=[-64]), K.KDA_ERR_SEQ),
    (dict(start_pos=[(1 << 62) + 64]), K.KDA_ERR_SEQ),   # past the largest accepted position
    (dict(q=0), K.KDA_ERR_NULL),
    (dict(o=0), K.KDA_ERR_NULL),
    (dict(q=FAKE + 8), K.KDA_ERR_SHAPE),
    (dict(ckpt_cu=[0, 1], ckpt_pos=[500], ckpt_page=[3]), K.KDA_ERR_CKPT_ALIGN),
    (dict(ckpt_cu=[0, 1], ckpt_pos=[1536], ckpt_page=[3]), K.KDA_ERR_CKPT_RANGE),
    (dict(ckpt_cu=[0, 2], ckpt_pos=[1024, 512], ckpt_page=[3, 4]), K.KDA_ERR_CKPT_RANGE),
    (dict(ckpt_cu=[0, 1], ckpt_pos=[0], ckpt_page=[3]), K.KDA_ERR_CKPT_RANGE),
    (dict(start_pos=[512], ckpt_cu=[0, 1], ckpt_pos=[512], ckpt_page=[3]), K.KDA_ERR_CKPT_RANGE),
    (dict(ckpt_cu=[0, 1], ckpt_pos=[512], ckpt_page=[16]), K.KDA_ERR_PAGE_RANGE),
    (dict(state_in_page=[16]), K.KDA_ERR_PAGE_RANGE),
    (dict(state_out_page=[-2]), K.KDA_ERR_PAGE_RANGE),
    (dict(ckpt_cu=[0, 2], ckpt_pos=[512, 1024], ckpt_page=[3, 3]), K.KDA_ERR_PAGE_ALIAS),
    (dict(state_out_page=[3], ckpt_cu=[0, 1], ckpt_pos=[512], ckpt_page=[3]), K.KDA_ERR_PAGE_ALIAS),
    (dict(state_in_page=[3], ckpt_cu=[0, 1], ckpt_pos=[512], ckpt_page=[3]), K.KDA_ERR_PAGE_ALIAS),
    (dict(cu_seqlens=[0, 512, 1024], state_in_page=[2, -1], state_out_page=[-1, 2]), K.KDA_ERR_PAGE_ALIAS),
    (dict(cu_seqlens=[0, 512, 1024], state_out_page=[5, 5]), K.KDA_ERR_PAGE_ALIAS),
    (dict(cu_seqlens=[0, 512, 1024], state_in_page=[5, 5], state_out_page=[5, -1]), K.KDA_ERR_PAGE_ALIAS),
    (dict(workspace=0), K.KDA_ERR_WORKSPACE),
    (dict(workspace=FAKE + 64), K.KDA_ERR_WORKSPACE),
    (dict(workspace_bytes=1024), K.KDA_ERR_WORKSPACE),
])
def test_prefill_validation(kw, status):
    assert _prefill_status(**kw) == status


def test_prefill_rejects_bad_pool_and_accepts_empty_batch():
    assert _prefill_status(p=pool(d_k=32)) == K.KDA_ERR_SHAPE
    # zero sequences: nothing to do, nothing enqueued
    st = K.raw_call("kda_prefill_chunked", ctypes.byref(pool()), None, None, None, None, None,
                    K.KDA_BF16, None, K.KDA_BF16, 0, None, None, None, None, None, None, None,
                    64, 512, None, 0, None)
    assert st == K.KDA_OK


def test_workspace_bound_matches_check():
    """The preferred size (kda_prefill_workspace_bytes) covers the smallest one
    (kda_prefill_workspace_min_bytes: one chunk per window); one byte less than
    the smallest is rejected by the call's validation (varlen, partial chunks)."""
    p = pool()
    cu = [0, 100, 100, 1000, 1100]
    pref = K.kda_prefill_workspace_bytes(p, 1100, 4, 0, K.KDA_BF16)
    least = K.kda_prefill_workspace_min_bytes(p, 4, 0, K.KDA_BF16)
    assert 0 < least <= pref
    # one window of one chunk: 32 heads of (chunk, head) blocks, plus two
    # carried states of 32 heads
    blk = ((3 * 64 * 128 + 2 * 64 * 64) * 2 + 4 * 128 + 255) // 256 * 256
    assert least >= 32 * blk + 2 * 32 * 65536
    chunks = sum((b - a + 63) // 64 for a, b in zip(cu[:-1], cu[1:]))
    assert pref >= least + (chunks - 1) * 32 * blk  # the whole call fits one window
    assert _prefill_status(p=p, cu_seqlens=cu, workspace_bytes=least - 1) == K.KDA_ERR_WORKSPACE
    assert K.kda_prefill_workspace_min_bytes(p, -1, 0, K.KDA_BF16) == 0


def test_conv_update_validation():
    """kda_short_conv_update rejects bad arguments before touching the device."""
    cp = K.make_conv_pool(FAKE, 3 * 12288 * 2, 8, 12288, 4, K.KDA_BF16)
    base = dict(cpool=cp, x=FAKE, w=FAKE, y=FAKE + 4096, page_in=FAKE, page_out=FAKE, n=4,
                out_dtype=K.KDA_BF16, stream=0)
    for kw, status in ((dict(x=0), K.KDA_ERR_NULL), (dict(page_out=0), K.KDA_ERR_NULL),
                       (dict(y=FAKE + 8), K.KDA_ERR_SHAPE), (dict(y=FAKE), K.KDA_ERR_SHAPE),
                       (dict(n=-1), K.KDA_ERR_SHAPE), (dict(out_dtype=4), K.KDA_ERR_DTYPE)):
        a = dict(base)
        a.update(kw)
        c = a.pop("cpool")
        with pytest.raises(K.KdaError) as e:
            K.kda_short_conv_update(c, a.pop("x"), a.pop("w"), a.pop("y"), a.pop("page_in"),
                                    a.pop("page_out"), **a)
        assert e.value.status == status, kw
    bad = K.make_conv_pool(FAKE, 256, 8, 12288, 4, K.KDA_BF16)  # pages smaller than a window
    with pytest.raises(K.KdaError) as e:
        K.kda_short_conv_update(bad, FAKE, FAKE, FAKE + 4096, FAKE, FAKE, n=4, out_dtype=K.KDA_BF16,
                                stream=0)
    assert e.value.status == K.KDA_ERR_POOL
    # n = 0: nothing to do
    K.kda_short_conv_update(cp, FAKE, FAKE, FAKE + 4096, FAKE, FAKE, n=0, out_dtype=K.KDA_BF16,
                            stream=0)


def test_noalloc_rejects_calls_above_the_static_scratch():
    """kda_prefill_chunked_noalloc rejects, before any device access, a call
    whose tables and one-chunk window exceed its static scratch (512 heads:
    two carried states alone are 64 MiB), and passes invalid calls to the
    full validation."""
    p = pool(num_heads=512, page_bytes=512 * 65536)
    need = K.kda_prefill_workspace_min_bytes(p, 1, 0, K.KDA_BF16)
    assert need > 64 << 20
    for kw, status in ((dict(), K.KDA_ERR_WORKSPACE), (dict(in_dtype=9), K.KDA_ERR_DTYPE)):
        args = dict(q=FAKE, k=FAKE, v=FAKE, g=FAKE, beta=FAKE, o=FAKE, in_dtype=K.KDA_BF16,
                    out_dtype=K.KDA_BF16, stream=0)
        args.update(kw)
        with pytest.raises(K.KdaError) as e:
            K.kda_prefill_chunked_noalloc(p, cu_seqlens=[0, 1024], **args)
        assert e.value.status == status
        assert "static scratch" in K.kda_last_error() or status != K.KDA_ERR_WORKSPACE
    with pytest.raises(K.KdaError) as e:
        K.kda_prefill_chunked_noalloc(pool(), FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, [0, 1024],
                                      chunk_size=32, in_dtype=K.KDA_BF16, out_dtype=K.KDA_BF16,
                                      stream=0)
    assert e.value.status == K.KDA_ERR_SHAPE


@pytest.mark.parametrize("fn", ["kda_checkpoint_write", "kda_checkpoint_restore"])
@pytest.mark.parametrize("src,dst,status", [
    ([1, 2], [3, 16], K.KDA_ERR_PAGE_RANGE),
    ([-1], [3], K.KDA_ERR_PAGE_RANGE),
    ([1, 2], [3, 3], K.KDA_ERR_PAGE_ALIAS),
    ([1, 2], [2, 4], K.KDA_ERR_PAGE_ALIAS),
    ([5], [5], K.KDA_ERR_PAGE_ALIAS),
])
def test_copy_validation(fn, src, dst, status):
    with pytest.raises(K.KdaError) as ei:
        getattr(K, fn)(pool(), src, dst, stream=0)
    assert ei.value.status == status


def test_copy_empty_is_noop():
    K.kda_checkpoint_write(pool(), [], [], stream=0)


def test_decode_validation():
    p = pool()
    st = K.raw_call("kda_decode_step", ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, K.KDA_BF16,
                    FAKE, K.KDA_BF16, -1, FAKE, FAKE, None)
    assert st == K.KDA_ERR_SHAPE
    st = K.raw_call("kda_decode_step", ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, K.KDA_BF16,
                    FAKE, K.KDA_BF16, 4, None, FAKE, None)
    assert st == K.KDA_ERR_NULL
    st = K.raw_call("kda_decode_step", ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, 3,
                    FAKE, K.KDA_BF16, 4, FAKE, FAKE, None)
    assert st == K.KDA_ERR_DTYPE
    st = K.raw_call("kda_decode_step", ctypes.byref(p), None, None, None, None, None, K.KDA_BF16,
                    None, K.KDA_BF16, 0, None, None, None)
    assert st == K.KDA_OK  # n = 0: nothing to do


def test_version():
    assert K.kda_version() >> 16 >= 1


# ---- int8 compressed checkpoints -------------------------------------------
QFAKE = 1 << 30  # a second fake region, disjoint from the pool's
QPAGE = 32 * (128 * 128 + 4 * 128)  # 540,672 bytes: 32 heads at d = 128


def qpool(**kw):
    d = dict(base=QFAKE, page_bytes=QPAGE, num_pages=8, num_heads=32, d_k=128)
    d.update(kw)
    return K.make_pool(**d)


def test_int8_head_bytes():
    assert K.kda_ckpt_int8_head_bytes(128, 128) == 128 * 128 + 4 * 128
    assert K.kda_ckpt_int8_head_bytes(64, 64) == 64 * 64 + 4 * 64
    assert K.kda_ckpt_int8_head_bytes(96, 96) == -1
    assert K.kda_ckpt_int8_head_bytes(128, 64) == -1


@pytest.mark.parametrize("direction", ["write", "restore"])
@pytest.mark.parametrize("qkw,src,dst,status", [
    (dict(num_heads=16), [0], [0], K.KDA_ERR_SHAPE),
    (dict(d_k=64), [0], [0], K.KDA_ERR_SHAPE),
    (dict(page_bytes=QPAGE - 256), [0], [0], K.KDA_ERR_POOL),
    (dict(page_bytes=QPAGE + 8), [0], [0], K.KDA_ERR_POOL),
    (dict(base=0), [0], [0], K.KDA_ERR_POOL),
    (dict(base=FAKE + 4 * MiB2), [0], [0], K.KDA_ERR_PAGE_ALIAS),  # overlaps the pool
    (dict(), [0, 1], [2, 2], K.KDA_ERR_PAGE_ALIAS),
    (dict(), [-1], [0], K.KDA_ERR_PAGE_RANGE),
])
def test_int8_validation(direction, qkw, src, dst, status):
    with pytest.raises(K.KdaError) as ei:
        if direction == "write":
            K.kda_checkpoint_write_int8(pool(), src, qpool(**qkw), dst, stream=0)
        else:
            K.kda_checkpoint_restore_int8(qpool(**qkw), src, pool(), dst, stream=0)
    assert ei.value.status == status


def test_int8_page_ranges_follow_direction():
    # write: sources index the pool (16 pages), destinations the qpool (8 pages)
    with pytest.raises(K.KdaError) as ei:
        K.kda_checkpoint_write_int8(pool(), [15], qpool(), [8], stream=0)
    assert ei.value.status == K.KDA_ERR_PAGE_RANGE
    # restore: sources index the qpool, destinations the pool
    with pytest.raises(K.KdaError) as ei:
        K.kda_checkpoint_restore_int8(qpool(), [8], pool(), [15], stream=0)
    assert ei.value.status == K.KDA_ERR_PAGE_RANGE
    K.kda_checkpoint_write_int8(pool(), [], qpool(), [], stream=0)  # empty: nothing enqueued


def test_verify_validation():
    p = pool()
    call = lambda n, tok, pin=FAKE, pout=FAKE: K.raw_call(  # noqa: E731
        "kda_decode_verify", ctypes.byref(p), FAKE, FAKE, FAKE, FAKE, FAKE, K.KDA_BF16, FAKE,
        K.KDA_BF16, n, tok, pin, pout, None)
    assert call(4, 0) == K.KDA_ERR_SHAPE
    assert call(4, 65) == K.KDA_ERR_SHAPE
    assert call(-1, 2) == K.KDA_ERR_SHAPE
    assert call(4, 2, pout=None) == K.KDA_ERR_NULL
    assert call(0, 2, None, None) == K.KDA_OK  # no requests: nothing to do


def cpool(**kw):
    d = dict(base=FAKE, page_bytes=4096, num_pages=16, channels=512, width=4, dtype=K.KDA_BF16)
    d.update(kw)
    return K.make_conv_pool(d["base"], d["page_bytes"], d["num_pages"], d["channels"], d["width"],
                            d["dtype"])


def _conv_status(cp=None, T=1024, **kw):
    cp = cp or cpool()
    args = dict(x=FAKE, w=FAKE, y=FAKE + MiB2, cu_seqlens=[0, T], out_dtype=K.KDA_BF16,
                workspace=FAKE, workspace_bytes=1 << 40, stream=0)
    args.update(kw)
    x, w, y = args.pop("x"), args.pop("w"), args.pop("y")
    try:
        K.kda_short_conv(cp, x, w, y, **args)
    except K.KdaError as e:
        assert K.kda_last_error() != ""
        return e.status
    return K.KDA_OK


def test_conv_workspace_bytes():
    assert K.kda_conv_workspace_bytes(-1, 0) == -1
    a, b = K.kda_conv_workspace_bytes(4, 0), K.kda_conv_workspace_bytes(4, 100)
    assert 0 < a < b and a % 256 == 0 and b % 256 == 0


@pytest.mark.parametrize("pkw,status", [
    (dict(width=1), K.KDA_ERR_SHAPE),
    (dict(width=5), K.KDA_ERR_SHAPE),
    (dict(channels=0), K.KDA_ERR_SHAPE),
    (dict(channels=12), K.KDA_ERR_SHAPE),                     # bf16 needs a multiple of 8
    (dict(channels=6, dtype=K.KDA_F32), K.KDA_ERR_SHAPE),     # fp32 needs a multiple of 4
    (dict(dtype=3), K.KDA_ERR_DTYPE),
    (dict(base=0), K.KDA_ERR_POOL),
    (dict(base=FAKE + 16), K.KDA_ERR_POOL),
    (dict(num_pages=0), K.KDA_ERR_POOL),
    (dict(page_bytes=2816), K.KDA_ERR_POOL),                  # 3 * 512 * 2 = 3072 needed
    (dict(page_bytes=3100), K.KDA_ERR_POOL),                  # not a multiple of 256
])
def test_conv_pool_validation(pkw, status):
    assert _conv_status(cp=cpool(**pkw)) == status


@pytest.mark.parametrize("kw,status", [
    (dict(out_dtype=9), K.KDA_ERR_DTYPE),
    (dict(hash_block=100), K.KDA_ERR_SHAPE),
    (dict(x=0), K.KDA_ERR_NULL),
    (dict(w=0), K.KDA_ERR_NULL),
    (dict(y=FAKE + 8), K.KDA_ERR_SHAPE),
    (dict(y=FAKE), K.KDA_ERR_SHAPE),                          # y aliases x
    (dict(cu_seqlens=[2, 10]), K.KDA_ERR_SEQ),
    (dict(cu_seqlens=[0, 10, 5]), K.KDA_ERR_SEQ),
    (dict(start_pos=[-1]), K.KDA_ERR_SEQ),
    (dict(start_pos=[(1 << 62) + 1]), K.KDA_ERR_SEQ),
    (dict(state_in_page=[16]), K.KDA_ERR_PAGE_RANGE),
    (dict(state_out_page=[-3]), K.KDA_ERR_PAGE_RANGE),
    (dict(state_in_page=[2], state_out_page=[2]), K.KDA_ERR_PAGE_ALIAS),
    (dict(cu_seqlens=[0, 5, 9], state_out_page=[4, 4]), K.KDA_ERR_PAGE_ALIAS),
    (dict(ckpt_cu=[0, 1], ckpt_pos=[500], ckpt_page=[3]), K.KDA_ERR_CKPT_ALIGN),
    (dict(ckpt_cu=[0, 1], ckpt_pos=[1536], ckpt_page=[3]), K.KDA_ERR_CKPT_RANGE),
    (dict(start_pos=[512], ckpt_cu=[0, 1], ckpt_pos=[512], ckpt_page=[3]), K.KDA_ERR_CKPT_RANGE),
    (dict(ckpt_cu=[0, 2], ckpt_pos=[1024, 512], ckpt_page=[3, 4]), K.KDA_ERR_CKPT_RANGE),
    (dict(ckpt_cu=[0, 1], ckpt_pos=[512], ckpt_page=[99]), K.KDA_ERR_PAGE_RANGE),
    (dict(state_in_page=[3], ckpt_cu=[0, 1], ckpt_pos=[512], ckpt_page=[3]), K.KDA_ERR_PAGE_ALIAS),
    (dict(state_out_page=[3], ckpt_cu=[0, 1], ckpt_pos=[512], ckpt_page=[3]), K.KDA_ERR_PAGE_ALIAS),
    (dict(workspace=0), K.KDA_ERR_WORKSPACE),
    (dict(workspace=FAKE + 32), K.KDA_ERR_WORKSPACE),
    (dict(workspace_bytes=16), K.KDA_ERR_WORKSPACE),
])
def test_conv_validation(kw, status):
    assert _conv_status(**kw) == status


def test_conv_accepts_checkpoints_past_start_and_empty_batch():
    # a start inside a block: the checkpoint at the next boundary is in range
    assert _conv_status(start_pos=[700], ckpt_cu=[0, 1], ckpt_pos=[1024], ckpt_page=[3],
                        workspace=0) == K.KDA_ERR_WORKSPACE  # everything before the workspace passed
    st = K.raw_call("kda_short_conv", ctypes.byref(cpool()), None, ctypes.c_void_p(FAKE), None,
                    K.KDA_BF16, 0, None, None, None, None, None, None, None, 512, None, 0, None)
    assert st == K.KDA_OK
    # empty sequences without output pages enqueue nothing
    assert _conv_status(T=0, x=0, y=0) == K.KDA_OK


@pytest.mark.parametrize("kw", [
    dict(cu_seqlens=[0, 512, 1024], start_pos=[0]),
    dict(cu_seqlens=[0, 512, 1024], state_in_page=[1]),
    dict(cu_seqlens=[0, 512, 1024], state_out_page=[1, 2, 3]),
    dict(ckpt_cu=[0], ckpt_pos=[512], ckpt_page=[3]),
    dict(ckpt_cu=[0, 2], ckpt_pos=[512], ckpt_page=[3, 4]),
    dict(ckpt_cu=[0, 2], ckpt_pos=[512, 1024], ckpt_page=[3]),
    dict(ckpt_cu=[0, 1], ckpt_pos=[512]),
    dict(ckpt_pos=[512], ckpt_page=[3]),
])
def test_prefill_host_array_lengths(kw):
    """A host array shorter than the count the C side reads through its pointer
    is refused by the binding before the call (no out-of-bounds host read)."""
    with pytest.raises(ValueError):
        _prefill_status(**kw)


@pytest.mark.parametrize("fn", ["kda_checkpoint_write", "kda_checkpoint_restore"])
def test_copy_host_array_lengths(fn):
    with pytest.raises(ValueError):
        getattr(K, fn)(pool(), [1, 2], [3], stream=0)


def test_c_consumer_builds(tmp_path):
    """include/kda.h is valid C99 (no C++ needed) and a C program using it
    links against the in-tree libkda.so (every symbol it calls resolves)."""
    import abi_consumer_build
    exe = abi_consumer_build.build(str(tmp_path / "abi_consumer"))
    assert os.path.exists(exe)
