"""Pins of the short-convolution oracle against what the definition fixes: a
hand-worked example (tap order), pure-delay and identity taps, per-channel
equivalence with numpy's 1-D convolution, continuity of the window across a
split, checkpoint windows as plain input rows, and independence of packed
sequences."""
import numpy as np
import pytest

from oracle import conv


def test_hand_worked_width3():
    # x = 1, 2, 3, 4 with taps (0.5, -1, 2) for (t-2, t-1, t) and a zero window:
    #   y0 = 2*1 = 2;  y1 = -1*1 + 2*2 = 3;  y2 = 0.5*1 - 1*2 + 2*3 = 4.5;
    #   y3 = 0.5*2 - 1*3 + 2*4 = 6;  window after 4 tokens = (3, 4)
    x = np.array([[1.0], [2.0], [3.0], [4.0]])
    w = np.array([[0.5, -1.0, 2.0]])
    y, ext = conv.conv_segment(x, w)
    assert y[:, 0].tolist() == [2.0, 3.0, 4.5, 6.0]
    assert conv.window_after(ext, 4, 3)[:, 0].tolist() == [3.0, 4.0]
    # the same with an entering window (-1, 5): y0 = 0.5*-1 - 1*5 + 2*1 = -3.5
    y, _ = conv.conv_segment(x, w, np.array([[-1.0], [5.0]]))
    assert y[:, 0].tolist() == [-3.5, 0.5 * 5 - 1 * 1 + 2 * 2, 4.5, 6.0]


@pytest.mark.parametrize("W", [2, 3, 4])
def test_identity_and_delay(W):
    rng = np.random.default_rng(W)
    x = rng.standard_normal((37, 5))
    win = rng.standard_normal((W - 1, 5))
    ident = np.zeros((5, W)); ident[:, W - 1] = 1.0
    y, _ = conv.conv_segment(x, ident, win)
    assert np.array_equal(y, x)
    delay = np.zeros((5, W)); delay[:, 0] = 1.0           # y[t] = x[t - (W-1)]
    y, _ = conv.conv_segment(x, delay, win)
    assert np.array_equal(y[W - 1:], x[:len(x) - (W - 1)])
    assert np.array_equal(y[:W - 1], win)
    y, _ = conv.conv_segment(x, delay)                   # zero window
    assert np.all(y[:W - 1] == 0)


@pytest.mark.parametrize("W", [2, 3, 4])
def test_matches_numpy_convolve(W):
    """A causal FIR filter is numpy's 'valid' convolution of the window-padded
    signal with the taps reversed (tap W-1 multiplies the current input)."""
    rng = np.random.default_rng(10 + W)
    x = rng.standard_normal((50, 6))
    w = rng.standard_normal((6, W))
    win = rng.standard_normal((W - 1, 6))
    y, _ = conv.conv_segment(x, w, win)
    for c in range(6):
        padded = np.concatenate([win[:, c], x[:, c]])
        ref = np.convolve(padded, w[c, ::-1], mode="valid")
        np.testing.assert_allclose(y[:, c], ref, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("W,split", [(2, 1), (3, 17), (4, 2), (4, 63)])
def test_split_continuity(W, split):
    """Running a prefix, then the suffix from the prefix's final window, gives
    the whole-sequence result (the window carries all the state there is)."""
    rng = np.random.default_rng(W * 100 + split)
    x = rng.standard_normal((80, 4))
    w = rng.standard_normal((4, W))
    y, ext = conv.conv_segment(x, w)
    y1, ext1 = conv.conv_segment(x[:split], w)
    y2, _ = conv.conv_segment(x[split:], w, conv.window_after(ext1, split, W))
    np.testing.assert_allclose(np.concatenate([y1, y2]), y, rtol=0, atol=1e-14)


def test_checkpoint_windows_are_input_rows():
    rng = np.random.default_rng(5)
    W, C = 4, 3
    x = rng.standard_normal((1200, C))
    w = rng.standard_normal((C, W))
    win = rng.standard_normal((W - 1, C))
    start = 510  # absolute position of row 0
    _, finals, ck = conv.short_conv_varlen(x, w, [0, 1200], [start], [win], [[512, 1024, 1536]])
    # window at P = absolute positions P-3 .. P-1 = rows P-3-start ..
    assert np.array_equal(ck[0][1], x[1024 - 3 - start:1024 - start])
    assert np.array_equal(ck[0][2], x[1536 - 3 - start:1536 - start])
    # P = 512 is 2 tokens in: the last entering-window row, then rows 0 and 1
    assert np.array_equal(ck[0][0], np.concatenate([win[2:], x[:2]]))
    assert np.array_equal(finals[0], x[-3:])


def test_varlen_independence_and_empty():
    rng = np.random.default_rng(9)
    W, C = 3, 4
    cu = [0, 10, 10, 35]
    x = rng.standard_normal((35, C))
    w = rng.standard_normal((C, W))
    wins = [None, rng.standard_normal((W - 1, C)), rng.standard_normal((W - 1, C))]
    y, finals, _ = conv.short_conv_varlen(x, w, cu, windows_in=wins)
    x2 = x.copy(); x2[10:] += 1.0
    y2, _, _ = conv.short_conv_varlen(x2, w, cu, windows_in=wins)
    assert np.array_equal(y[:10], y2[:10])
    assert np.array_equal(finals[1], wins[1])            # empty sequence keeps its window
    y3, _ = conv.conv_segment(x[10:], w, wins[2])
    assert np.array_equal(y[10:], y3)
