"""The seeded input generators (shared by both sides; no method arithmetic)."""
import numpy as np
import pytest


def test_philox_known_answers(gen):
    # Known-answer vectors published with Random123 for philox4x32-10.
    kat = [
        ([0, 0, 0, 0], [0, 0], [0x6627E8D5, 0xE169C58D, 0xBC57AC4C, 0x9B00DBD8]),
        ([0xFFFFFFFF] * 4, [0xFFFFFFFF] * 2, [0x408F276D, 0x41C83B0E, 0xA20BC7C6, 0x6D5451FD]),
        ([0x243F6A88, 0x85A308D3, 0x13198A2E, 0x03707344], [0xA4093822, 0x299F31D0],
         [0xD16CFE09, 0x94FDCCEB, 0x5001E420, 0x24126EA1]),
    ]
    for ctr, key, want in kat:
        assert list(gen.philox4x32_10(ctr, key)) == want


@pytest.mark.parametrize("x,bits", [
    (1.0, 0x3F80), (1.0 + 2**-8, 0x3F80), (1.0 + 3 * 2**-8, 0x3F82),
    (1.0 + 2**-8 + 2**-40, 0x3F81), (-(1.0 + 2**-8), 0xBF80), (0.0, 0x0000),
    (-0.05, 0xBD4D), (3.140625, 0x4049)])
def test_bf16_round_to_nearest_even(gen, x, bits):
    assert gen.bf16_rne(x) == bits


def test_deterministic_and_slice_independent(gen):
    a = gen.fill(7, 3, gen.NORMAL, 0, 10, 3, 16, "f32", threads=1)
    b = gen.fill(7, 3, gen.NORMAL, 0, 10, 3, 16, "f32", threads=4)
    c = gen.fill(7, 3, gen.NORMAL, 4, 6, 3, 16, "f32", threads=2)
    assert np.array_equal(a, b) and np.array_equal(a[4:], c)
    d = gen.fill(8, 3, gen.NORMAL, 0, 10, 3, 16, "f32")
    assert not np.array_equal(a, d)


def test_distributions(gen):
    d = gen.kda_tokens(11, 4, 64, 0, 2048, "f32")
    for name in ("q", "k"):
        n = np.linalg.norm(d[name].astype(np.float64), axis=-1)
        assert np.allclose(n, 1.0, atol=1e-6)
    v = d["v"].astype(np.float64)
    assert abs(v.mean()) < 0.01 and abs(v.std() - 1) < 0.01
    g = d["g"]
    assert g.min() >= -0.05 and g.max() <= 0.0 and abs(g.mean() + 0.025) < 1e-3
    b = d["beta"]
    assert b.min() > 0 and b.max() < 1 and abs(b.mean() - 0.5) < 0.01


def test_bf16_tensors_are_rounded_fp64_values(gen):
    x = gen.fill(3, 5, gen.NORMAL, 0, 2, 2, 8, "f64")
    xb = gen.fill(3, 5, gen.NORMAL, 0, 2, 2, 8, "bf16")
    assert all(gen.bf16_rne(float(a)) == int(b) for a, b in zip(x.ravel(), xb.ravel()))


def test_workload_plans(gen):
    lens, bnd = gen.varlen_plan()
    assert len(lens) == 16 and lens.min() >= 1024 and lens.max() <= 32768
    assert np.all(bnd % 512 == 0) and np.all(bnd > 0) and np.all(bnd < lens)
    pt = gen.decode_page_table()
    assert len(pt) == 256 and len(set(pt.tolist())) == 256 and pt.max() < 512
    ck = gen.LONG_1M.ckpts
    assert len(ck) == 171 and ck[0] == 6144 and ck[-1] == 1 << 20
