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
                in_place=True, all_pairs=False):
    """Returns (max err o, max err state) over the sampled (request, head) pairs.
    With all_pairs, every (request, head) pair is also checked on o at every
    step and on the state after the last step (the sample's states are checked
    at every step of check_steps)."""
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
    if all_pairs:
        # pair j = r * H + h: the steps of that (request, head) as one oracle head
        print(f"decode: oracle on all {n * H} pairs x {steps} steps", flush=True)
        flat = {k: d[k].reshape(steps, n * H, *d[k].shape[2:]) for k in ("q", "k", "v", "g")}
        flat["beta"] = d["beta"].reshape(steps, n * H)
        ref = oracle.run(flat["q"], flat["k"], flat["v"], flat["g"], flat["beta"], [0, steps],
                         s0=s0.reshape(1, n * H, D, D).astype(np.float64))
        o_full = o_all.reshape(steps, n * H, D).double().cpu().numpy()
        err_o = max(err_o, max(rel_fro(o_full[:, j], ref["o"][:, j]) for j in range(n * H)))
        del o_full
        for r in range(n):
            st = pb.states(int(pin[r] if not in_place else page_table[r]))
            err_s = max(err_s, max(rel_fro(st[h], ref["s_final"][0, r * H + h]) for h in range(H)))
    return err_o, err_s


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64), ("f32", 128), ("bf16", 64)])
def test_decode_small(dtype, D):
    n, H, steps = 8, 4, 100
    pt = np.array([9, 2, 14, 5, 0, 11, 7, 3])
    sample = [(r, h) for r in range(n) for h in range(H)]
    e_o, e_s = _run_decode(n, H, D, steps, dtype, 4242 + D, 16, pt, sample, {1, 10, 100})
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype], (e_o, e_s)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_decode_many_heads(dtype, D):
    """96 heads (one layer's KDA heads in the pages' model), 37 requests in
    place through a permuted page table: every (request, head) pair checked on
    o at every step and on its state after the last step."""
    n, H, steps = 37, 96, 20
    pt = np.random.default_rng(3).permutation(80)[:n]
    sample = [(0, 0), (n - 1, H - 1), (17, 50)]
    e_o, e_s = _run_decode(n, H, D, steps, dtype, 515 + D, 80, pt, sample, {1, steps}, all_pairs=True)
    assert e_o <= TOL[dtype] and e_s <= TOL[dtype], (e_o, e_s)


def test_decode_ping_pong_pages():
    """page_out != page_in (alternating between two page sets) gives the same
    result as the in-place update."""
    n, H, D, steps = 4, 2, 128, 20
    pt = np.array([1, 3, 5, 7])
    sample = [(r, h) for r in range(n) for h in range(H)]
    e_o, e_s = _run_decode(n, H, D, steps, "bf16", 17, 16, pt, sample, {20}, in_place=False)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"], (e_o, e_s)


@pytest.mark.timeout(900)
def test_decode_256_full():
    """256 requests x 32 heads x d=128, 1000 consecutive steps in place through a
    random page table of a 512-page pool.  All 8192 (request, head) pairs are
    checked against the oracle on o at every step and on the state after step
    1000; 48 sampled pairs also on the states after steps 1, 10 and 100."""
    w = G.DECODE_256
    pt = G.decode_page_table(w)
    rng = np.random.default_rng(1)
    sample = [(int(r), int(h)) for r, h in zip(rng.integers(0, w.n_req, 48), rng.integers(0, w.H, 48))]
    e_o, e_s = _run_decode(w.n_req, w.H, w.D, w.steps, w.dtype, w.seed, w.pool_pages, pt, sample,
                           {1, 10, 100, 1000}, all_pairs=True)
    assert e_o <= TOL["bf16"] and e_s <= TOL["bf16"], (e_o, e_s)


def test_decode_bad_page_is_loud_and_harmless(monkeypatch):
    """A page index outside the pool touches no state and yields NaN outputs for
    that request only (the kernel checks every index before using it)."""
    monkeypatch.delenv("KDA_VALIDATE", raising=False)  # the device-side handling is under test
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


# ---- speculative verification: tokens per request in one launch ------------

def _verify_setup(n, H, D, ntok, dtype, seed):
    s0 = G.random_states(seed, n, H, D)
    d = G.kda_tokens(seed, H, D, 0, n * ntok, dtype)  # row r*ntok + t = token t of request r
    return s0, d


def test_verify_equals_sequential_steps_bitwise():
    """tokens = 4 in one launch == 4 kda_decode_step calls, bit for bit, on o
    and on every intermediate state."""
    n, H, D, ntok = 8, 4, 128, 4
    s0, d = _verify_setup(n, H, D, ntok, "bf16", 31)
    di = {k: dev(v, "bf16") for k, v in d.items()}
    pb = PoolBuf(n * (ntok + 1) * 2, H, D)
    base = n * (ntok + 1)
    for r in range(n):
        pb.set_states(r, s0[r])
        pb.set_states(base + r, s0[r])
    pin = torch.arange(n, dtype=torch.int32, device="cuda")
    pout = torch.arange(n, n + n * ntok, dtype=torch.int32, device="cuda")  # r*ntok + t -> page n + r*ntok + t
    o_v = torch.empty((n * ntok, H, D), dtype=torch.bfloat16, device="cuda")
    K.kda_decode_verify(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o_v, ntok, pin, pout)
    # sequential: step t reads the page written by step t-1
    o_s = torch.empty((n * ntok, H, D), dtype=torch.bfloat16, device="cuda")
    rows = torch.arange(n, device="cuda") * ntok
    cur = torch.arange(base, base + n, dtype=torch.int32, device="cuda")
    for t in range(ntok):
        nxt = (base + n + rows + t).to(torch.int32)
        sel = rows + t
        o_t = torch.empty((n, H, D), dtype=torch.bfloat16, device="cuda")
        K.kda_decode_step(pb.pool, di["q"][sel], di["k"][sel], di["v"][sel], di["g"][sel],
                          di["beta"][sel], o_t, cur, nxt)
        o_s[sel] = o_t
        cur = nxt
    torch.cuda.synchronize()
    assert torch.equal(o_v.view(torch.int16), o_s.view(torch.int16))
    for r in range(n):
        for t in range(ntok):
            assert np.array_equal(pb.states(n + r * ntok + t), pb.states(base + n + r * ntok + t)), (r, t)


@pytest.mark.parametrize("dtype,D,ntok", [("bf16", 128, 6), ("f32", 64, 5),
                                          ("f32", 128, 64), ("bf16", 64, 64)])  # 64: the most per call
def test_verify_oracle(dtype, D, ntok):
    """Each request's ntok tokens against the oracle run over them with a
    checkpoint after every token."""
    n, H = 4, 3
    s0, d = _verify_setup(n, H, D, ntok, dtype, 41 + D)
    di = {k: dev(v, dtype) for k, v in d.items()}
    pb = PoolBuf(n + n * ntok, H, D)
    for r in range(n):
        pb.set_states(r, s0[r])
    pin = torch.arange(n, dtype=torch.int32, device="cuda")
    pout = torch.arange(n, n + n * ntok, dtype=torch.int32, device="cuda")
    o = torch.empty((n * ntok, H, D), dtype=tdtype(dtype), device="cuda")
    K.kda_decode_verify(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, ntok, pin, pout)
    torch.cuda.synchronize()
    cu = [ntok * r for r in range(n + 1)]
    ref = oracle.run(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, s0=s0.astype(np.float64),
                     ckpt_cu=[ntok * r for r in range(n + 1)], ckpt_pos=[t + 1 for _ in range(n) for t in range(ntok)])
    got = o.double().cpu().numpy()
    worst = 0.0
    for r in range(n):
        for h in range(H):
            worst = max(worst, rel_fro(got[r * ntok:(r + 1) * ntok, h], ref["o"][r * ntok:(r + 1) * ntok, h]))
            for t in range(ntok):
                worst = max(worst, rel_fro(pb.states(n + r * ntok + t)[h], ref["ckpts"][r * ntok + t, h]))
    assert worst <= TOL[dtype], worst


def test_verify_bad_page_is_loud_and_harmless(monkeypatch):
    monkeypatch.delenv("KDA_VALIDATE", raising=False)  # the device-side handling is under test
    n, H, D, ntok = 3, 2, 64, 3
    s0, d = _verify_setup(n, H, D, ntok, "bf16", 7)
    di = {k: dev(v, "bf16") for k, v in d.items()}
    pb = PoolBuf(n + n * ntok, H, D)
    for r in range(n):
        pb.set_states(r, s0[r])
    before = pb.snapshot()
    pin = torch.arange(n, dtype=torch.int32, device="cuda")
    po = list(range(n, n + n * ntok))
    po[1 * ntok + 2] = 10 ** 6  # request 1's last page index is out of range
    pout = torch.tensor(po, dtype=torch.int32, device="cuda")
    o = torch.zeros((n * ntok, H, D), dtype=torch.bfloat16, device="cuda")
    K.kda_decode_verify(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, ntok, pin, pout)
    torch.cuda.synchronize()
    of = o.float().cpu().numpy()
    assert np.all(np.isnan(of[ntok:2 * ntok])) and not np.any(np.isnan(of[:ntok])) and not np.any(np.isnan(of[2 * ntok:]))
    after = pb.snapshot()
    w = pb.page_bytes // 4
    for p in range(n + ntok, n + 2 * ntok - 1):  # request 1's valid output pages stay untouched
        assert np.array_equal(before[p * w:(p + 1) * w], after[p * w:(p + 1) * w])


def test_validate_mode_checks_page_tables(monkeypatch):
    """With KDA_VALIDATE=1 the decode page tables are read back and checked on
    the host before anything runs: a valid call gives the bits of the unchecked
    one (single token and verify form); an index outside the pool, a repeated
    output page and an input page that is another request's output are rejected
    with the documented status, and the pool and the outputs stay untouched."""
    n, H, D, ntok = 4, 2, 64, 2
    s0 = G.random_states(5, n, H, D)
    d = G.kda_tokens(5, H, D, 0, n * ntok, "bf16")
    di = {k: dev(v, "bf16") for k, v in d.items()}

    def fresh():
        pb = PoolBuf(n + n * ntok, H, D)
        for r in range(n):
            pb.set_states(r, s0[r])
        return pb

    def step(pb, o, pin, pout, tokens):
        if tokens == 1:
            K.kda_decode_step(pb.pool, di["q"][:n], di["k"][:n], di["v"][:n], di["g"][:n],
                              di["beta"][:n], o, pin, pout)
        else:
            K.kda_decode_verify(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, tokens,
                                pin, pout)

    pin = torch.arange(n, dtype=torch.int32, device="cuda")
    for tokens in (1, ntok):
        pout = torch.arange(n, n + n * tokens, dtype=torch.int32, device="cuda")
        runs = []
        for val in (None, "1"):
            if val is None:
                monkeypatch.delenv("KDA_VALIDATE", raising=False)
            else:
                monkeypatch.setenv("KDA_VALIDATE", val)
            pb = fresh()
            o = torch.empty((n * tokens, H, D), dtype=torch.bfloat16, device="cuda")
            step(pb, o, pin, pout, tokens)
            torch.cuda.synchronize()
            runs.append((o.view(torch.int16).cpu(), pb.buf.cpu()))
        assert torch.equal(runs[0][0], runs[1][0]) and torch.equal(runs[0][1], runs[1][1]), tokens

    def with_(t, i, val):
        t = t.clone()
        t[i] = val
        return t

    p1 = torch.arange(n, 2 * n, dtype=torch.int32, device="cuda")
    p2 = torch.arange(n, n + n * ntok, dtype=torch.int32, device="cuda")
    cases = [
        (1, with_(pin, 2, 100), p1, K.KDA_ERR_PAGE_RANGE),
        (1, pin, with_(p1, 1, -1), K.KDA_ERR_PAGE_RANGE),
        (1, pin, with_(p1, 3, n), K.KDA_ERR_PAGE_ALIAS),         # output page n twice
        (1, with_(pin, 1, n), p1, K.KDA_ERR_PAGE_ALIAS),         # request 0's output read by request 1
        (ntok, pin, with_(p2, 1, n), K.KDA_ERR_PAGE_ALIAS),      # request 0's two tokens share a page
        (ntok, pin, with_(p2, 7, n + n * ntok), K.KDA_ERR_PAGE_RANGE),
    ]
    for tokens, bad_in, bad_out, status in cases:
        pb = fresh()
        before = pb.buf.clone()
        o = torch.full((n * tokens, H, D), 3.0, dtype=torch.bfloat16, device="cuda")
        with pytest.raises(K.KdaError) as e:
            step(pb, o, bad_in, bad_out, tokens)
        assert e.value.status == status, (tokens, e.value, status)
        torch.cuda.synchronize()
        assert torch.equal(pb.buf, before) and bool(torch.all(o == 3.0))


def test_serving_loop_graph_replay_bitwise(monkeypatch):
    """A serving loop captured once in a HIP graph: 8 single-token decode steps
    in place through a device page table, a 3-token verify into fresh pages,
    then a checkpoint copy of each request's first verified state.  Replayed
    three times from the same starting pool, with eager work and
    synchronisation between replays: every replay leaves the outputs and the
    pool bit-identical to the eager run."""
    monkeypatch.delenv("KDA_VALIDATE", raising=False)  # its host read-back cannot be captured
    n, H, D, steps, ntok = 16, 4, 128, 8, 3
    s0 = G.random_states(21, n, H, D)
    d = G.kda_tokens(21, H, D, 0, (steps + ntok) * n, "bf16")
    di = {k: dev(v, "bf16") for k, v in d.items()}
    pb = PoolBuf(n + n * ntok + n, H, D)
    for r in range(n):
        pb.set_states(r, s0[r])
    start = pb.buf.clone()
    pt = torch.arange(n, dtype=torch.int32, device="cuda")
    pv = torch.arange(n, n + n * ntok, dtype=torch.int32, device="cuda")
    src = [n + r * ntok for r in range(n)]
    dst = [n + n * ntok + r for r in range(n)]
    o = torch.empty((steps, n, H, D), dtype=torch.bfloat16, device="cuda")
    ov = torch.empty((n * ntok, H, D), dtype=torch.bfloat16, device="cuda")

    def loop():
        for t in range(steps):
            sl = slice(t * n, (t + 1) * n)
            K.kda_decode_step(pb.pool, di["q"][sl], di["k"][sl], di["v"][sl], di["g"][sl],
                              di["beta"][sl], o[t], pt, pt)
        b = steps * n
        K.kda_decode_verify(pb.pool, di["q"][b:], di["k"][b:], di["v"][b:], di["g"][b:],
                            di["beta"][b:], ov, ntok, pt, pv)
        K.kda_checkpoint_write(pb.pool, src, dst)

    loop()
    torch.cuda.synchronize()
    ref = (o.view(torch.int16).cpu(), ov.view(torch.int16).cpu(), pb.buf.cpu())
    pb.buf.copy_(start)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        loop()  # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        loop()
    for _ in range(3):
        pb.buf.copy_(start)
        o.fill_(float("nan"))
        ov.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(o.view(torch.int16).cpu(), ref[0])
        assert torch.equal(ov.view(torch.int16).cpu(), ref[1])
        assert torch.equal(pb.buf.cpu(), ref[2])
