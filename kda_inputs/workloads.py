"""Workload recipes: shapes, seeds and checkpoint sets of the synthetic configs.

Each recipe names its sizes; none holds any of the method's arithmetic.

* ``SINGLE_1K``   one sequence, H=1, d=64, T=1024, fp32, S0 = 0, checkpoints at
                  512 and 1024.
* ``PREFILL_8K``  one sequence, H=32, d=128, T=8192, bf16 inputs, fp32 state,
                  checkpoints at {2560, 6144, 8192} (2560 = 5 x 512 is the worked
                  prefix hit of page "Cache de préfixe hybride KDA–MLA",
                  sections "La solution" and "La recherche en deux étages").
* ``VARLEN_RESUME`` 16 sequences, lengths uniform in [1024, 32768]; each resumes
                  at a random 512-multiple boundary 0 < B < length.
* ``DECODE_256``  256 requests x 32 heads x d=128, one token per step, 1000 steps,
                  fp32 states N(0, 1/d) in a 512-page pool behind a random page
                  table.
* ``LONG_1M``     one sequence, H=32, d=128, T=2^20, bf16, checkpoints every 6144
                  tokens plus the final position.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HASH_BLOCK = 512
CHUNK = 64


@dataclass(frozen=True)
class Prefill:
    name: str
    H: int
    D: int
    T: int
    dtype: str
    ckpts: tuple
    seed: int
    page_bytes: int = 0  # 0 => exactly H*D*D*4

    def state_bytes(self) -> int:
        return self.H * self.D * self.D * 4


SINGLE_1K = Prefill("single_1k_h1_d64_f32", 1, 64, 1024, "f32", (512, 1024), 0x4B44411)
PREFILL_8K = Prefill("prefill_8k_h32_d128_bf16", 32, 128, 8192, "bf16", (2560, 6144, 8192),
                     0x4B44412, page_bytes=2 << 20)
LONG_1M = Prefill("long_1m_h32_d128_bf16", 32, 128, 1 << 20, "bf16",
                  tuple(list(range(6144, 1 << 20, 6144)) + [1 << 20]), 0x4B44415,
                  page_bytes=2 << 20)


@dataclass(frozen=True)
class VarlenResume:
    name: str = "varlen_resume_16_h32_d128_bf16"
    n_seqs: int = 16
    len_lo: int = 1024
    len_hi: int = 32768
    H: int = 32
    D: int = 128
    dtype: str = "bf16"
    seed: int = 0x4B44413


VARLEN_RESUME = VarlenResume()


def varlen_plan(w: VarlenResume = VARLEN_RESUME):
    """(lengths, boundaries): len uniform integer in [len_lo, len_hi]; B uniform
    over {512 m : m >= 1, 512 m < len}."""
    from . import TID_PLAN, stream_id, uniforms
    u = uniforms(w.seed, stream_id(TID_PLAN), 0, 2 * w.n_seqs)
    lens = (w.len_lo + np.floor(u[0::2] * (w.len_hi - w.len_lo + 1))).astype(np.int64)
    nb = (lens - 1) // HASH_BLOCK  # number of admissible boundaries
    bnd = (HASH_BLOCK * (1 + np.floor(u[1::2] * nb))).astype(np.int64)
    return lens, bnd


@dataclass(frozen=True)
class Decode:
    name: str = "decode_256req_h32_d128_bf16"
    n_req: int = 256
    H: int = 32
    D: int = 128
    steps: int = 1000
    pool_pages: int = 512
    dtype: str = "bf16"
    seed: int = 0x4B44414
    page_bytes: int = 2 << 20


DECODE_256 = Decode()


def decode_page_table(w: Decode = DECODE_256):
    """Distinct pages: a seeded random choice of n_req pages out of pool_pages."""
    from . import TID_PLAN, stream_id, uniforms
    u = uniforms(w.seed, stream_id(TID_PLAN, 1), 0, w.pool_pages)
    return np.argsort(u, kind="stable")[: w.n_req].astype(np.int32)


__all__ = ["HASH_BLOCK", "CHUNK", "Prefill", "SINGLE_1K", "PREFILL_8K", "LONG_1M",
           "VarlenResume", "VARLEN_RESUME", "varlen_plan", "Decode", "DECODE_256",
           "decode_page_table"]
