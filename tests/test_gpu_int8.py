"""GPU parity of the int8 compressed checkpoints against oracle/quant.py:
compressed pages bit-exact (codes and scales), restored fp32 pages bit-exact,
poisoned pages outside the call untouched, and a prefix resume through an int8
checkpoint within the bf16 bar of the oracle resumed from the same codes."""
import numpy as np
import pytest
import torch

import hybrid_prefix_cache_amd as K
import kda_inputs as G
import oracle
from kda_gpu_util import POISON_WORD, PoolBuf, inputs_to_dev, prefill, rel_fro
from oracle import quant

pytestmark = pytest.mark.gpu
POISON = np.int32(np.uint32(POISON_WORD).view(np.int32))


class QPool:
    """A poisoned device region of compressed pages."""

    def __init__(self, num_pages, H, D, extra=0):
        self.H, self.D = H, D
        self.head_bytes = K.kda_ckpt_int8_head_bytes(D, D)
        need = H * self.head_bytes
        self.page_bytes = (need + extra + 255) // 256 * 256
        self.buf = torch.full((num_pages * self.page_bytes // 4,), int(POISON), dtype=torch.int32,
                              device="cuda")
        self.pool = K.make_pool(self.buf, self.page_bytes, num_pages, H, D)

    def page(self, p):
        b = self.buf.view(torch.uint8)[p * self.page_bytes:(p + 1) * self.page_bytes]
        return b.cpu().numpy()


def _states(seed, n, H, D):
    s = G.random_states(seed, n, H, D)
    s[0, 0, 3] = 0.0                      # a zero row
    s[0, 0, 5, 7] = 1e4                   # one dominant element
    s[min(1, n - 1), H - 1, 9] *= 1e-6    # tiny magnitudes
    return s


@pytest.mark.parametrize("H,D,extra", [(32, 128, 0), (3, 64, 4096)])
def test_write_and_restore_bitexact(H, D, extra):
    n = 12
    s = _states(21 + D, n, H, D)
    pb = PoolBuf(2 * n, H, D, page_bytes=0)
    for i in range(n):
        pb.set_states(i, s[i])
    qp = QPool(n + 2, H, D, extra)
    src, qdst = list(range(n)), [(i * 5) % (n + 2) for i in range(n)]
    K.kda_checkpoint_write_int8(pb.pool, src, qp.pool, qdst)
    torch.cuda.synchronize()
    need = H * qp.head_bytes
    for i in range(n):
        q, sc = quant.quantize(s[i])
        got = qp.page(qdst[i])
        assert np.array_equal(got[:need], quant.pack_page(q, sc)), f"page {i}"
        assert np.all(got[need:].view(np.int32) == POISON) if (qp.page_bytes - need) % 4 == 0 else True
    for p in set(range(n + 2)) - set(qdst):
        assert np.all(qp.page(p).view(np.int32) == POISON)
    # restore into pages n..2n-1 of the fp32 pool
    before = pb.snapshot()
    K.kda_checkpoint_restore_int8(qp.pool, qdst, pb.pool, list(range(n, 2 * n)))
    torch.cuda.synchronize()
    after = pb.snapshot()
    w = pb.page_bytes // 4
    assert np.array_equal(before[:n * w], after[:n * w])  # sources untouched
    for i in range(n):
        q, sc = quant.quantize(s[i])
        ref = quant.dequantize(q, sc)
        got = pb.states(n + i).astype(np.float32)
        assert np.array_equal(got, ref), f"restored page {i}"
        assert np.all(np.abs(got.astype(np.float64) - s[i]) <= sc[..., None] * (0.5 + 1e-5) + 1e-30)


def test_batch_over_one_launch():
    """500 pairs (more than one launch's worth of page pairs)."""
    H, D, n = 1, 64, 500
    s = G.random_states(5, n, H, D)
    pb = PoolBuf(n, H, D)
    for i in range(n):
        pb.set_states(i, s[i])
    qp = QPool(n, H, D)
    perm = list(np.random.default_rng(0).permutation(n))
    K.kda_checkpoint_write_int8(pb.pool, list(range(n)), qp.pool, perm)
    torch.cuda.synchronize()
    allq = qp.buf.view(torch.uint8).cpu().numpy().reshape(n, qp.page_bytes)
    need = H * qp.head_bytes
    for i in range(n):
        q, sc = quant.quantize(s[i])
        assert np.array_equal(allq[perm[i], :need], quant.pack_page(q, sc))


def test_resume_through_int8_checkpoint():
    """Prefill [0, B) with a checkpoint at B, compress it, restore it into a
    fresh active page, prefill the suffix: within the bf16 bar of the oracle
    that resumes from the dequantised oracle checkpoint."""
    H, D, T, B = 4, 128, 1536, 1024
    d = G.kda_tokens(99, H, D, 0, T, "bf16")
    di = inputs_to_dev(d, "bf16")
    pb = PoolBuf(4, H, D)
    pre = {k: v[:B] for k, v in di.items()}
    prefill(pb, pre, [0, B], "bf16", ckpt_cu=[0, 1], ckpt_pos=[B], ckpt_page=[0])
    qp = QPool(1, H, D)
    K.kda_checkpoint_write_int8(pb.pool, [0], qp.pool, [0])
    K.kda_checkpoint_restore_int8(qp.pool, [0], pb.pool, [1])
    suf = {k: v[B:] for k, v in di.items()}
    o = prefill(pb, suf, [0, T - B], "bf16", start_pos=[B], state_in_page=[1], state_out_page=[2])
    ref_b = oracle.run(d["q"][:B], d["k"][:B], d["v"][:B], d["g"][:B], d["beta"][:B], [0, B])
    q, sc = quant.quantize(ref_b["s_final"][0].astype(np.float32))
    s0 = quant.dequantize(q, sc).astype(np.float64)[None]
    ref = oracle.run(d["q"][B:], d["k"][B:], d["v"][B:], d["g"][B:], d["beta"][B:], [0, T - B], s0=s0)
    got = o.double().cpu().numpy()
    err_o = max(rel_fro(got[:, h], ref["o"][:, h]) for h in range(H))
    err_s = max(rel_fro(pb.states(2)[h], ref["s_final"][0, h]) for h in range(H))
    assert err_o <= 2e-2 and err_s <= 2e-2, (err_o, err_s)


def _tie_states(seed, H, D):
    """Rows built so that most quotients x / scale land on a half-integer or
    one ulp beside one (where a reciprocal multiply and the IEEE division could
    round differently), with denormal, power-of-two and constant rows."""
    rng = np.random.default_rng(seed)
    s = np.empty((H, D, D), np.float32)
    for h in range(H):
        for i in range(D):
            kind = (h * D + i) % 5
            m = np.float32(2.0 ** int(rng.integers(-20, 20)) * rng.uniform(1, 2))
            if kind == 3:
                m = np.float32(2.0 ** int(rng.integers(-10, 10)))
            if kind == 4:
                m = np.float32(1e-40 * (1 + i))           # denormal row maximum
            scale = np.float32(m / np.float32(127.0))
            ks = rng.integers(-126, 126, D).astype(np.float64) + 0.5
            x = (ks * np.float64(scale)).astype(np.float32)
            nud = rng.integers(-1, 2, D)
            x = np.where(nud > 0, np.nextafter(x, np.float32(np.inf)),
                         np.where(nud < 0, np.nextafter(x, np.float32(-np.inf)), x)).astype(np.float32)
            x = np.clip(x, -m, m).astype(np.float32)
            x[0] = -m if kind == 2 else m
            if kind == 2 and i % 2:
                x[:] = -m                                   # every element at the maximum
            s[h, i] = x
    return s


@pytest.mark.parametrize("D", [128, 64])
def test_write_bitexact_at_rounding_ties(D):
    """Codes and scales bit-exact where the quotient sits on or next to a
    rounding boundary, for denormal and power-of-two scales too."""
    H = 2
    s = _tie_states(7 + D, H, D)
    pb = PoolBuf(1, H, D)
    pb.set_states(0, s)
    qp = QPool(1, H, D)
    K.kda_checkpoint_write_int8(pb.pool, [0], qp.pool, [0])
    torch.cuda.synchronize()
    q, sc = quant.quantize(s)
    ties = np.abs(np.abs(np.float32(s) / np.where(sc > 0, sc, 1)[..., None]) % 1 - 0.5) < 1e-5
    assert ties.mean() > 0.2  # the rows do exercise the boundary
    assert np.array_equal(qp.page(0)[:H * qp.head_bytes], quant.pack_page(q, sc))
