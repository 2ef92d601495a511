"""GPU decode-step parity: one launch per token step, states gathered and
scattered through a device page table, against the oracle's token loop (each
(request, head) pair is one oracle head running the steps as a sequence)."""
import numpy as np
import pytest
import torch

import hybrid_prefix_cache_amd as K
import kda_inputs as G
import oracle
from kda_gpu_util import PoolBuf, dev, rel_fro, tdtype

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _run_decode(n, H, D, steps, dtype, seed, pool_pages, page_table, sample, check_steps,
                in_place=True):
    """Returns (max err o, max err state) over the sampled (request, head) pairs."""
    s0 = G.random_states(seed, n, H, D)  # float32 [n, H, D, D]
    pb = PoolBuf(pool_pages, H, D, page_bytes=0)
    for r in range(n):
        pb.set_states(int(page_table[r]), s0[r])
    pin = torch.from_numpy(page_table.astype(np.int32)).cuda()
    if not in_place:  # second, disjoint page set in the upper half of the pool
        assert page_table.max() < pool_pages // 2
    pout = pin if in_place else torch.from_numpy(
        (page_table + pool_pages // 2).astype(np.int32)).cuda()
    # all steps' inputs: one logical [steps * n, H, D] token stream
    print(f"decode: n={n} H={H} D={D} steps={steps}: generating inputs", flush=True)
    d = G.kda_tokens(seed, H, D, 0, steps * n, dtype)
    di = {k: dev(v, dtype) for k, v in d.items()}
    o_all = torch.empty((steps, n, H, D), dtype=tdtype(dtype), device="cuda")
    snaps = {}
    for t in range(steps):
        sl = slice(t * n, (t + 1) * n)
        K.kda_decode_step(pb.pool, di["q"][sl], di["k"][sl], di["v"][sl], di["g"][sl],
                          di["beta"][sl], o_all[t], pin, pout)
        if not in_place:
            pin, pout = pout, pin
        if t + 1 in check_steps:
            torch.cuda.synchronize()
            snaps[t + 1] = {(r, h): pb.states(int(pin[r] if not in_place else page_table[r]))[h]
                            for (r, h) in sample}
    torch.cuda.synchronize()
    rs = torch.tensor([r for r, _ in sample], device="cuda")
    hs = torch.tensor([h for _, h in sample], device="cuda")
    o_np = o_all[:, rs, hs].double().cpu().numpy()  # [steps, n_sample, D]
    # oracle: each sampled (r, h) is one head of a length-`steps` sequence
    sel = {k: np.stack([d[k].reshape(steps, n, H, *d[k].shape[2:])[:, r, h] for (r, h) in sample],
                       axis=1) for k in ("q", "k", "v", "g")}
    sel["beta"] = np.stack([d["beta"].reshape(steps, n, H)[:, r, h] for (r, h) in sample], axis=1)
    s0_sel = np.stack([s0[r, h] for (r, h) in sample])[None].astype(np.float64)
    cks = sorted(check_steps)
    ref = oracle.run(sel["q"], sel["k"], sel["v"], sel["g"], sel["beta"], [0, steps], s0=s0_sel,
                     ckpt_cu=[0, len(cks)], ckpt_pos=cks)
    err_o = max(rel_fro(o_np[:, j], ref["o"][:, j]) for j in range(len(sample)))
    err_s = max(rel_fro(snaps[c][(r, h)], ref["ckpts"][m, j])
                for m, c in enumerate(cks) for j, (r, h) in enumerate(sample))
    return err_o, err_s


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("f32", 128), ("bf16", 64)])
def test_decode_small(dtype, D):
    n, H, steps = 8, 4, 100
    pt = np.array([9, 2, 14, 5, 0, 11, 7, 3])
    sample = [(r, h) for r in range(n) for h in range(H)]
    e_o, e_s = _run_decode(n, H, D, steps, dtype, 4242 + D, 16, pt, sample, {1, 10, 100})
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype], (e_o, e_s)


def test_decode_ping_pong_pages():
    """page_out != page_in (alternating between two page sets) gives the same
    result as the in-place update."""
    n, H, D, steps = 4, 2, 128, 20
    pt = np.array([1, 3, 5, 7])
    sample = [(r, h) for r in range(n) for h in range(H)]
    e_o, e_s = _run_decode(n, H, D, steps, "bf16", 17, 16, pt, sample, {20}, in_place=False)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"], (e_o, e_s)


@pytest.mark.timeout(600)
def test_decode_256_full():
    """256 requests x 32 heads x d=128, 1000 consecutive steps in place through a
    random page table of a 512-page pool; 48 sampled (request, head) pairs are
    checked against the oracle on o at every step and on the state after steps
    1, 10, 100 and 1000."""
    w = G.DECODE_256
    pt = G.decode_page_table(w)
    rng = np.random.default_rng(1)
    sample = [(int(r), int(h)) for r, h in zip(rng.integers(0, w.n_req, 48), rng.integers(0, w.H, 48))]
    e_o, e_s = _run_decode(w.n_req, w.H, w.D, w.steps, w.dtype, w.seed, w.pool_pages, pt, sample,
                           {1, 10, 100, 1000})
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"], (e_o, e_s)


def test_decode_bad_page_is_loud_and_harmless():
    """A page index outside the pool touches no state and yields NaN outputs for
    that request only (the kernel checks every index before using it)."""
    n, H, D = 3, 2, 64
    pb = PoolBuf(4, H, D)
    s0 = G.random_states(3, n, H, D)
    pb.set_states(0, s0[0])
    pb.set_states(2, s0[2])
    before = pb.snapshot()
    d = G.kda_tokens(3, H, D, 0, n, "bf16")
    di = {k: dev(v, "bf16") for k, v in d.items()}
    pin = torch.tensor([0, 99, 2], dtype=torch.int32, device="cuda")
    o = torch.zeros((n, H, D), dtype=torch.bfloat16, device="cuda")
    K.kda_decode_step(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, pin, pin)
    torch.cuda.synchronize()
    of = o.float().cpu().numpy()
    assert np.all(np.isnan(of[1])) and not np.any(np.isnan(of[[0, 2]]))
    after = pb.snapshot()
    w = pb.page_bytes // 4
    assert np.array_equal(before[w:2 * w], after[w:2 * w])  # page 1 untouched
    assert np.array_equal(before[3 * w:], after[3 * w:])    # page 3 untouched


def test_decode_deterministic():
    n, H, D = 16, 8, 128
    d = G.kda_tokens(8, H, D, 0, n, "bf16")
    di = {k: dev(v, "bf16") for k, v in d.items()}
    outs = []
    for _ in range(2):
        pb = PoolBuf(n, H, D, poison=False)
        for r in range(n):
            pb.set_states(r, G.random_states(8, n, H, D)[r])
        pin = torch.arange(n, dtype=torch.int32, device="cuda")
        o = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
        K.kda_decode_step(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, pin, pin)
        torch.cuda.synchronize()
        outs.append((o.view(torch.int16).cpu().numpy(), pb.snapshot()))
    assert np.array_equal(outs[0][0], outs[1][0]) and np.array_equal(outs[0][1], outs[1][1])
