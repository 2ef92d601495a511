"""Oracle of the int8 compressed checkpoints.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import it;
the product path never does, and the two share no code.

Page "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app),
section 5.3 (Compressed Checkpoint): a cached recurrent state may be stored as
int8 with per-channel quantisation parameters; on a hit it is dequantised once
into a fresh active state and decoding continues at full precision.  Section
6.6.2 (Int8CheckpointStore): the scale has one entry per d_k index, from the
max-abs taken along d_v; the quantisation is symmetric.

Readings where the pages are silent (the same ones the library documents):
the scale is max-abs / 127; codes are round-half-to-even of x / scale,
clamped to [-127, 127]; a row whose max-abs is 0 has scale 0 and all codes 0;
every operation is fp32 (IEEE division), so each code is a fixed function of
the fp32 state.  Dequantisation is q * scale in fp32.

The state layout is the library's: [..., d_k, d_v] with row i the d_k index.
"""
from __future__ import annotations

import numpy as np


def quantize(S):
    """fp32 states [..., d_k, d_v] -> (int8 codes of the same shape, fp32 scales [..., d_k])."""
    S = np.asarray(S, dtype=np.float32)
    m = np.max(np.abs(S), axis=-1)
    scale = (m / np.float32(127.0)).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.rint(S / scale[..., None]).astype(np.float32)
    q = np.where(scale[..., None] > 0, np.clip(r, -127, 127), 0).astype(np.int8)
    return q, scale


def dequantize(q, scale):
    """(int8 codes [..., d_k, d_v], fp32 scales [..., d_k]) -> fp32 states."""
    return (np.asarray(q).astype(np.float32) * np.asarray(scale, np.float32)[..., None]).astype(np.float32)


def pack_page(q, scale):
    """Bytes of one compressed page as the library lays it out: for each head,
    int8 q[d_k][d_v] then fp32 scale[d_k] (q: [H, d_k, d_v], scale: [H, d_k])."""
    parts = []
    for h in range(q.shape[0]):
        parts.append(np.ascontiguousarray(q[h]).view(np.uint8).reshape(-1))
        parts.append(np.ascontiguousarray(scale[h], dtype=np.float32).view(np.uint8).reshape(-1))
    return np.concatenate(parts)
