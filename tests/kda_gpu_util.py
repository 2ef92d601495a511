"""Helpers for the GPU parity tests: move generator outputs to the device, run
the library through its C ABI, read pages back, and measure errors against the
oracle (max relative Frobenius error, per (sequence, head) block)."""
from __future__ import annotations

import numpy as np
import torch

import hybrid_prefix_cache_amd as K

POISON_WORD = 0x7FC0DEAD  # a NaN pattern: any unintended read or write shows up


def dev(x: np.ndarray, dtype: str) -> torch.Tensor:
    """numpy generator output -> contiguous device tensor (bf16 from uint16 bits)."""
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.cuda()


def tdtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


class PoolBuf:
    """A device state pool filled with a poison pattern."""

    def __init__(self, num_pages, H, D, page_bytes=0, poison=True):
        self.H, self.D = H, D
        self.state_bytes = H * D * D * 4
        self.page_bytes = page_bytes or self.state_bytes
        self.num_pages = num_pages
        words = num_pages * self.page_bytes // 4
        self.buf = torch.empty(words, dtype=torch.int32, device="cuda")
        if poison:
            self.buf.fill_(np.int32(np.uint32(POISON_WORD).view(np.int32)))
        else:
            self.buf.zero_()
        self.pool = K.make_pool(self.buf, self.page_bytes, num_pages, H, D)
        assert K.kda_pool_check(self.pool) == K.KDA_OK, K.kda_last_error()

    def page_words(self, p):
        w = self.page_bytes // 4
        return self.buf[p * w:(p + 1) * w]

    def states(self, p) -> np.ndarray:
        """fp32 states of page p as float64 [H, D, D]."""
        w = self.page_words(p)[: self.state_bytes // 4]
        return w.view(torch.float32).reshape(self.H, self.D, self.D).cpu().numpy().astype(np.float64)

    def set_states(self, p, s: np.ndarray):
        w = self.page_words(p)[: self.state_bytes // 4]
        w.view(torch.float32).copy_(torch.from_numpy(np.ascontiguousarray(s, np.float32)).reshape(-1))

    def snapshot(self) -> np.ndarray:
        return self.buf.cpu().numpy().copy()


def workspace(pool, total_tokens, num_seqs, num_ckpts, in_dtype):
    n = K.kda_prefill_workspace_bytes(pool, total_tokens, num_seqs, num_ckpts, in_dtype)
    assert n > 0
    return torch.empty(n, dtype=torch.uint8, device="cuda")


def rel_fro(got: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / den) if den > 0 else float(np.linalg.norm(got))


def max_rel_blocks(got, ref, cu, H):
    """Max over (sequence, head) of ||got - ref||_F / ||ref||_F over [len, d_v]."""
    worst = 0.0
    for s in range(len(cu) - 1):
        a, b = int(cu[s]), int(cu[s + 1])
        if b == a:
            continue
        for h in range(H):
            worst = max(worst, rel_fro(got[a:b, h], ref[a:b, h]))
    return worst


def inputs_to_dev(d, dtype):
    return {name: dev(d[name], dtype) for name in ("q", "k", "v", "g", "beta")}


def prefill(pb: PoolBuf, di, cu, dtype, out_dtype=None, **kw):
    """Run kda_prefill_chunked on device inputs di (dict of tensors); returns o."""
    T = int(cu[-1])
    H, D = pb.H, pb.D
    out_dtype = out_dtype or ("f32" if dtype == "f32" else "bf16")
    o = torch.full((T, H, D), float("nan"), dtype=tdtype(out_dtype), device="cuda")
    ncks = 0 if kw.get("ckpt_cu") is None else int(kw["ckpt_cu"][-1])
    ind = K.KDA_BF16 if dtype == "bf16" else K.KDA_F32
    ws = workspace(pb.pool, T, len(cu) - 1, ncks, ind)
    K.kda_prefill_chunked(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, cu,
                          workspace=ws, **kw)
    torch.cuda.synchronize()
    return o
