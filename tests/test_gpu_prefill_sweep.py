"""GPU prefill parity on a seeded sweep of small random calls: libkda vs the
fp64 oracle, through the C ABI.

Each case draws the head count, d, the input dtype, 1-6 sequences of ragged
lengths (empty, 1-token and chunk-boundary lengths included), resume
positions (multiples of 64) with random entering states on some sequences,
a hash block of 64, 128 or 512 tokens with a checkpoint at every block end
the sequence crosses, and a workspace anywhere between the smallest accepted
size and the preferred one (so windows cut sequences at arbitrary chunks).
Checked: o per (sequence, head), every checkpoint and final state against the
oracle (max relative Frobenius error <= 1e-4 for fp32 inputs, <= 2e-2 for
bf16), and placement bit-exact on a poisoned pool (exactly the designated
state bytes change).
"""
import numpy as np
import pytest
import torch

import hybrid_prefix_cache_amd as K
import kda_inputs as G
import oracle
from kda_gpu_util import POISON_WORD, PoolBuf, inputs_to_dev, max_rel_blocks, rel_fro

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
SPECIAL_LENS = (0, 1, 63, 64, 65, 127, 128, 129)


def _case(seed):
    rng = np.random.default_rng(0x5EED + seed)
    H = int(rng.integers(1, 7))
    D = int(rng.choice([64, 128]))
    dtype = str(rng.choice(["bf16", "f32"]))
    ns = int(rng.integers(1, 7))
    lens = [int(rng.choice(SPECIAL_LENS)) if rng.random() < 0.35 else int(rng.integers(1, 900))
            for _ in range(ns)]
    hb = int(rng.choice([64, 128, 512]))
    sp = [64 * int(rng.integers(0, 12)) if rng.random() < 0.6 else 0 for _ in range(ns)]
    with_state = [bool(sp[i] > 0 and rng.random() < 0.7) for i in range(ns)]
    return rng, H, D, dtype, ns, lens, hb, sp, with_state


@pytest.mark.parametrize("seed", range(40))
def test_random_call(seed):
    rng, H, D, dtype, ns, lens, hb, sp, with_state = _case(seed)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    T = int(cu[-1])
    # pages: entering states, final states, checkpoints
    s_in = [-1] * ns
    npg = 0
    for i in range(ns):
        if with_state[i]:
            s_in[i] = npg
            npg += 1
    s_out = list(range(npg, npg + ns))
    npg += ns
    ck_cu, ck_pos, ck_page = [0], [], []
    for i in range(ns):
        for pos in range((sp[i] // hb + 1) * hb, sp[i] + lens[i] + 1, hb):
            ck_pos.append(pos)
            ck_page.append(npg)
            npg += 1
        ck_cu.append(len(ck_pos))
    nck = len(ck_pos)
    d = G.kda_tokens(7100 + seed, H, D, 0, max(T, 1), dtype)
    if T == 0:
        d = {k_: v_[:0] for k_, v_ in d.items()}
    s0 = np.zeros((ns, H, D, D))
    pb = PoolBuf(max(npg, 1), H, D)
    for i in range(ns):
        if with_state[i]:
            s = (rng.standard_normal((H, D, D)) / np.sqrt(D)).astype(np.float32)
            pb.set_states(s_in[i], s)
            s0[i] = s
    before = pb.snapshot()
    ind = K.KDA_BF16 if dtype == "bf16" else K.KDA_F32
    full = K.kda_prefill_workspace_bytes(pb.pool, T, ns, nck, ind)
    least = K.kda_prefill_workspace_min_bytes(pb.pool, ns, nck, ind)
    assert 0 < least <= full
    nbytes = int(rng.integers(least, full + 1)) // 256 * 256
    nbytes = max(nbytes, (least + 255) // 256 * 256)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device="cuda")
    o = torch.full((T, H, D), float("nan"), device="cuda",
                   dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
    di = inputs_to_dev(d, dtype)
    K.kda_prefill_chunked(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, cu,
                          start_pos=sp, state_in_page=s_in, state_out_page=s_out,
                          ckpt_cu=ck_cu, ckpt_pos=ck_pos, ckpt_page=ck_page, hash_block=hb,
                          workspace=ws, workspace_bytes=nbytes)
    torch.cuda.synchronize()
    desc = dict(H=H, D=D, dtype=dtype, lens=lens, sp=sp, hb=hb, nck=nck, ws=nbytes, full=full)
    ref = oracle.run(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, start_pos=sp, s0=s0,
                     ckpt_cu=ck_cu, ckpt_pos=ck_pos)
    if T > 0:
        err_o = max_rel_blocks(o.double().cpu().numpy(), ref["o"], cu, H)
        assert err_o <= TOL[dtype], (err_o, desc)
    for i in range(ns):
        got = pb.states(s_out[i])
        for h in range(H):
            e = rel_fro(got[h], ref["s_final"][i, h])
            assert e <= TOL[dtype], ("final", i, h, e, desc)
    for m in range(nck):
        got = pb.states(ck_page[m])
        for h in range(H):
            e = rel_fro(got[h], ref["ckpts"][m, h])
            assert e <= TOL[dtype], ("ckpt", m, h, e, desc)
    # placement: exactly the final-state and checkpoint pages changed (fully)
    after = pb.snapshot()
    w = pb.page_bytes // 4
    changed = set(s_out) | set(ck_page)
    poison = np.int32(np.uint32(POISON_WORD).view(np.int32))
    for p in range(pb.num_pages):
        blk_b, blk_a = before[p * w:(p + 1) * w], after[p * w:(p + 1) * w]
        if p in changed:
            assert not np.any(blk_a == poison), ("unwritten word on page", p, desc)
        else:
            assert np.array_equal(blk_b, blk_a), ("page changed", p, desc)
