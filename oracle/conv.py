"""Oracle of the short causal convolution with a checkpointed window state.

TEST INFRASTRUCTURE ONLY (same rule as the rest of ``oracle/``): only ``tests/``,
``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline`` leg may import it;
the product path never does, and the two share no code.

Page "KIMI K3 경량 복제에서 본 KDA의 AI 인프라 과제" (acpost.vercel.app):
section 1.1 (besides the recurrent state, the short convolution needs the
inputs of the last few tokens stored as its own state), 6.5 and 6.6.3 (the
checkpoint pool stores and loads that window beside the recurrent state),
8.2.3 (prefill runs a causal convolution over each of q, k and v before the
recurrence) and 8.2.4 (the checkpoint pass writes the convolution history of
the boundary together with the recurrent checkpoint); section 0x09 adds that
the local window is usually kept at its original precision.

Readings where the pages are silent (the same ones the library documents):
width W in {2, 3, 4}, one fp32 tap vector per channel, no activation, no bias:
    y[t][c] = sum_{j < W} w[c][j] * x[t - (W-1) + j][c],
with inputs at positions before a sequence's first token taken from the
entering window (zeros when there is none).  The window after P tokens is the
W-1 inputs at positions P-(W-1) .. P-1, oldest first.  Everything here is fp64
over the values the caller passes (bf16 inputs are exact in fp64).
"""
from __future__ import annotations

import numpy as np


def conv_segment(x, w, window_in=None):
    """One sequence segment.  x: [T, C]; w: [C, W]; window_in: [W-1, C] or None
    (zeros).  Returns (y [T, C], the extended input [W-1+T, C]): row r of the
    extended input is the input at position r - (W-1) relative to the segment
    start, so the window after n tokens is ext[n : n + W-1]."""
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    T, C = x.shape
    W = w.shape[1]
    win = np.zeros((W - 1, C)) if window_in is None else np.asarray(window_in, dtype=np.float64)
    assert win.shape == (W - 1, C)
    ext = np.concatenate([win, x], axis=0)
    y = np.zeros((T, C))
    for j in range(W):  # tap j multiplies the input W-1-j positions back
        y += w[:, j][None, :] * ext[j:j + T]
    return y, ext


def window_after(ext, n, W):
    """The W-1 most recent inputs after n tokens of the segment."""
    return ext[n:n + W - 1].copy()


def short_conv_varlen(x, w, cu_seqlens, start_pos=None, windows_in=None, ckpt_positions=None):
    """Packed sequences as the library takes them.

    x: [T, C]; cu_seqlens: [num_seqs+1]; start_pos: absolute position of each
    sequence's first token (only checkpoint positions depend on it);
    windows_in: per sequence an entering window [W-1, C] or None;
    ckpt_positions: per sequence a list of absolute positions P.
    Returns (y [T, C], final windows [num_seqs][W-1, C], checkpoint windows as
    a list per sequence, in the order of ckpt_positions)."""
    x = np.asarray(x, dtype=np.float64)
    W = np.asarray(w).shape[1]
    cu = [int(c) for c in cu_seqlens]
    ns = len(cu) - 1
    start_pos = [0] * ns if start_pos is None else [int(s) for s in start_pos]
    windows_in = [None] * ns if windows_in is None else windows_in
    ckpt_positions = [[] for _ in range(ns)] if ckpt_positions is None else ckpt_positions
    y = np.zeros(x.shape)
    finals, ckpts = [], []
    for s in range(ns):
        a, b = cu[s], cu[s + 1]
        ys, ext = conv_segment(x[a:b], w, windows_in[s])
        y[a:b] = ys
        finals.append(window_after(ext, b - a, W))
        ckpts.append([window_after(ext, P - start_pos[s], W) for P in ckpt_positions[s]])
    return y, finals, ckpts
