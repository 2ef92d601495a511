"""Pins of the int8 checkpoint oracle against what the definition fixes: a
hand-worked example, brute-force nearest-code search, the error bound, the
exact max element, zero rows, sign symmetry and the page byte layout."""
import numpy as np

from oracle import quant


def test_hand_worked_rows():
    # row max-abs 127 -> scale exactly 1.0; row max-abs 63.5 -> scale exactly 0.5;
    # quotients that are exact halves round to even
    S = np.array([[[1.0, -2.0, 0.5, 127.0],
                   [2.5, -127.0, 3.5, 0.0],
                   [63.5, 1.25, -0.75, 0.25]]], np.float32)
    q, scale = quant.quantize(S)
    assert scale[0].tolist() == [1.0, 1.0, 0.5]
    assert q[0, 0].tolist() == [1, -2, 0, 127]
    assert q[0, 1].tolist() == [2, -127, 4, 0]
    assert q[0, 2].tolist() == [127, 2, -2, 0]
    assert quant.dequantize(q, scale)[0, 2].tolist() == [63.5, 1.0, -1.0, 0.0]


def test_zero_row_and_sign_symmetry():
    rng = np.random.default_rng(3)
    S = rng.standard_normal((2, 8, 16)).astype(np.float32)
    S[1, 3] = 0.0
    q, scale = quant.quantize(S)
    assert scale[1, 3] == 0 and np.all(q[1, 3] == 0)
    assert np.all(quant.dequantize(q, scale)[1, 3] == 0)
    qn, sn = quant.quantize(-S)
    assert np.array_equal(qn, -q) and np.array_equal(sn, scale)


def test_brute_force_nearest_code():
    """Each code is the integer in [-127, 127] whose multiple of the scale is
    nearest to x (ties are skipped: there the fp32 quotient decides)."""
    rng = np.random.default_rng(11)
    S = (rng.standard_normal((4, 32, 32)) * rng.uniform(0.01, 10, (4, 32, 1))).astype(np.float32)
    q, scale = quant.quantize(S)
    cand = np.arange(-127, 128, dtype=np.float64)
    for idx in np.ndindex(S.shape):
        sc = float(scale[idx[:-1]])
        t = float(S[idx]) / sc
        if abs(abs(t - np.floor(t)) - 0.5) < 1e-4:
            continue
        best = cand[np.argmin(np.abs(float(S[idx]) - cand * sc))]
        assert q[idx] == best, (idx, S[idx], sc, q[idx], best)


def test_error_bound_and_max_element():
    rng = np.random.default_rng(5)
    S = (rng.standard_normal((3, 64, 64)) / 8).astype(np.float32)
    q, scale = quant.quantize(S)
    R = quant.dequantize(q, scale)
    err = np.abs(R.astype(np.float64) - S)
    assert np.all(err <= scale[..., None] * (0.5 + 1e-5) + 1e-30)
    # the element of largest magnitude in each row maps to +-127
    j = np.argmax(np.abs(S), axis=-1)
    top = np.take_along_axis(q, j[..., None], axis=-1)[..., 0]
    assert np.all(np.abs(top.astype(int)) == 127)


def test_page_layout():
    rng = np.random.default_rng(2)
    S = rng.standard_normal((2, 64, 64)).astype(np.float32)
    q, scale = quant.quantize(S)
    page = quant.pack_page(q, scale)
    hb = 64 * 64 + 4 * 64
    assert page.size == 2 * hb
    assert np.array_equal(page[hb:hb + 64 * 64].view(np.int8).reshape(64, 64), q[1])
    assert np.array_equal(page[hb + 64 * 64:2 * hb].view(np.float32), scale[1])
