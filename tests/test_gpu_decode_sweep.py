"""GPU decode parity on a seeded sweep of small random calls: libkda vs the
fp64 oracle, through the C ABI.

Each case draws the request count, the head count, d, the input dtype and the
number of tokens per request (1: kda_decode_step, in place or into a fresh
page; more: kda_decode_verify keeping every intermediate state), with the
pages scattered through a larger poisoned pool.  Checked: o and every state
written against the oracle run over each request's tokens from its entering
state (max relative Frobenius error <= 1e-4 for fp32 inputs, <= 2e-2 for
bf16), and that every page the call does not write keeps its bytes.
"""
import numpy as np
import pytest
import torch

import hybrid_prefix_cache_amd as K
import kda_inputs as G
import oracle
from kda_gpu_util import PoolBuf, dev, rel_fro, tdtype

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.mark.parametrize("seed", range(24))
def test_random_decode_call(seed):
    rng = np.random.default_rng(0xDEC0DE + seed)
    n = int(rng.integers(1, 41))
    H = int(rng.integers(1, 7))
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    ntok = int(rng.choice([1, 1, 2, 3, 4, 7, 10]))
    in_place = ntok == 1 and bool(rng.random() < 0.5)
    need = n if in_place else n + n * ntok
    npages = need + int(rng.integers(0, 16))
    perm = rng.permutation(npages)
    pin_l = [int(x) for x in perm[:n]]
    pout_l = pin_l if in_place else [int(x) for x in perm[n:n + n * ntok]]
    s0 = G.random_states(900 + seed, n, H, D)
    d = G.kda_tokens(950 + seed, H, D, 0, n * ntok, dtype)  # row r*ntok + t = token t of request r
    di = {k_: dev(v_, dtype) for k_, v_ in d.items()}
    pb = PoolBuf(npages, H, D)
    for r in range(n):
        pb.set_states(pin_l[r], s0[r])
    before = pb.snapshot()
    pin = torch.tensor(pin_l, dtype=torch.int32, device="cuda")
    pout = torch.tensor(pout_l, dtype=torch.int32, device="cuda")
    o = torch.empty((n * ntok, H, D), dtype=tdtype(dtype), device="cuda")
    if ntok == 1:
        K.kda_decode_step(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, pin, pout)
    else:
        K.kda_decode_verify(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, ntok, pin, pout)
    torch.cuda.synchronize()
    desc = dict(n=n, H=H, D=D, dtype=dtype, ntok=ntok, in_place=in_place, npages=npages)
    cu = [ntok * r for r in range(n + 1)]
    ref = oracle.run(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, s0=s0.astype(np.float64),
                     ckpt_cu=cu, ckpt_pos=[t + 1 for _ in range(n) for t in range(ntok)])
    got = o.double().cpu().numpy()
    for r in range(n):
        for h in range(H):
            e = rel_fro(got[r * ntok:(r + 1) * ntok, h], ref["o"][r * ntok:(r + 1) * ntok, h])
            assert e <= TOL[dtype], ("o", r, h, e, desc)
            for t in range(ntok):
                e = rel_fro(pb.states(pout_l[r * ntok + t])[h], ref["ckpts"][r * ntok + t, h])
                assert e <= TOL[dtype], ("state", r, t, h, e, desc)
    after = pb.snapshot()
    w = pb.page_bytes // 4
    written = set(pout_l)
    for p in range(npages):
        if p not in written:
            assert np.array_equal(before[p * w:(p + 1) * w], after[p * w:(p + 1) * w]), ("page", p, desc)
