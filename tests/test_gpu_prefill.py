"""GPU prefill parity: libkda (HIP, gfx950) vs the fp64 oracle, through the C ABI.

Bar: max relative Frobenius error (per (sequence, head) block of o, per
checkpointed / final state) <= 1e-4 for fp32 inputs and <= 2e-2 for bf16 inputs;
checkpoint placement and page indexing bit-exact (poisoned pool: exactly the
designated state bytes change); repeated runs and resumed runs bitwise equal.
"""
import numpy as np
import pytest
import torch

import hybrid_prefix_cache_amd as K
import kda_inputs as G
import oracle
from kda_gpu_util import (POISON_WORD, PoolBuf, inputs_to_dev, max_rel_blocks, prefill,
                          rel_fro)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


def _poison_mask_ok(before, after, pb, changed_pages):
    """Only the state bytes of `changed_pages` may differ; everything else keeps
    its previous bytes (page padding included)."""
    w = pb.page_bytes // 4
    sw = pb.state_bytes // 4
    allowed = np.zeros(before.shape, bool)
    for p in changed_pages:
        allowed[p * w:p * w + sw] = True
    if np.any(before[~allowed] != after[~allowed]):
        return False
    # every designated word was written (no poison left behind)
    for p in changed_pages:
        if np.any(after[p * w:p * w + sw] == np.int32(np.uint32(POISON_WORD).view(np.int32))):
            return False
    return True


def _oracle_prefill(d, cu, **kw):
    return oracle.run(d["q"], d["k"], d["v"], d["g"], d["beta"], cu, **kw)


# ---------------------------------------------------------------------------
def test_single_1k_f32():
    """One sequence, H=1, d=64, T=1024, fp32, S0 = 0, checkpoints at 512 and 1024."""
    w = G.SINGLE_1K
    d = G.kda_tokens(w.seed, w.H, w.D, 0, w.T, w.dtype)
    pb = PoolBuf(4, w.H, w.D)
    before = pb.snapshot()
    o = prefill(pb, inputs_to_dev(d, w.dtype), [0, w.T], w.dtype, ckpt_cu=[0, 2],
                ckpt_pos=list(w.ckpts), ckpt_page=[1, 2], state_out_page=[3])
    ref = _oracle_prefill(d, [0, w.T], ckpt_cu=[0, 2], ckpt_pos=list(w.ckpts))
    err_o = max_rel_blocks(o.double().cpu().numpy(), ref["o"], [0, w.T], w.H)
    err_c = max(rel_fro(pb.states(1 + m)[0], ref["ckpts"][m, 0]) for m in range(2))
    assert err_o <= TOL["f32"] and err_c <= TOL["f32"], (err_o, err_c)
    assert np.array_equal(pb.states(2), pb.states(3))  # checkpoint at T == final state
    assert _poison_mask_ok(before, pb.snapshot(), pb, [1, 2, 3])


@pytest.mark.parametrize("dtype,D,H,cu", [
    ("bf16", 128, 4, [0, 1000]),                      # ragged tail (1000 = 15*64 + 40)
    ("bf16", 64, 3, [0, 700]),
    ("f32", 128, 2, [0, 300]),
    ("f32", 64, 2, [0, 130, 130, 200, 777]),          # varlen with an empty sequence
    ("bf16", 128, 2, [0, 1, 65, 129, 700, 1212]),     # 1-token and 64-token sequences
])
def test_small_cases(dtype, D, H, cu):
    T = cu[-1]
    d = G.kda_tokens(1234 + D + H, H, D, 0, T, dtype)
    ns = len(cu) - 1
    pb = PoolBuf(2 * ns + 2, H, D)
    out_pages = list(range(ns))
    o = prefill(pb, inputs_to_dev(d, dtype), cu, dtype, state_out_page=out_pages)
    ref = _oracle_prefill(d, cu)
    err_o = max_rel_blocks(o.double().cpu().numpy(), ref["o"], cu, H)
    err_s = max(rel_fro(pb.states(s)[h], ref["s_final"][s, h]) if cu[s + 1] > cu[s] else 0.0
                for s in range(ns) for h in range(H))
    assert err_o <= TOL[dtype] and err_s <= TOL[dtype], (err_o, err_s)
    for s in range(ns):  # empty sequence with no entering state: zero final state
        if cu[s + 1] == cu[s]:
            assert np.all(pb.states(s) == 0)


def _f64(x, dtype):
    """Stored input values (bf16 bit patterns or fp32) as float64."""
    if dtype == "bf16":
        return (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def _const(x, dtype, value):
    """An input array of the generator's shape and dtype holding `value`."""
    if dtype == "bf16":
        bits = np.float32(value).view(np.uint32) >> 16  # value is exact in bf16
        return np.full(x.shape, bits, np.uint16)
    return np.full(x.shape, value, x.dtype)


@pytest.mark.parametrize("dtype,g_lo,g_hi", [
    ("bf16", -1.2, 0.0), ("f32", -1.2, 0.0),   # strong, mixed decay
    ("bf16", -3.0, 0.0), ("f32", -3.0, 0.0),   # chunk sums near -96
    ("bf16", -2.7, -2.6), ("f32", -2.7, -2.6),  # edge: ~86 of log-decay per half chunk
])
def test_strong_decay(dtype, g_lo, g_hi):
    """Strong per-channel decay.  With g near -2.7 every channel's log decay over
    a chunk is about -173, far past the fp32 range of exp; the chunk form keeps
    each factor within one half chunk of the middle (|G - G_31| <= ~86) and
    matches the oracle, o and every checkpoint and final state, with a resumed
    second sequence and a ragged tail."""
    H, D = 2, 128
    cu = [0, 1000, 1700]
    d = G.kda_tokens(4242, H, D, 0, cu[-1], dtype, g_lo=g_lo, g_hi=g_hi)
    s0 = (np.random.default_rng(7).standard_normal((H, D, D)) / np.sqrt(D)).astype(np.float32)
    pb = PoolBuf(6, H, D)
    pb.set_states(5, s0)
    ck = dict(ckpt_cu=[0, 1, 2], ckpt_pos=[512, 1536], ckpt_page=[2, 3])
    o = prefill(pb, inputs_to_dev(d, dtype), cu, dtype, start_pos=[0, 1024],
                state_in_page=[-1, 5], state_out_page=[0, 1], **ck)
    s_in = np.zeros((2, H, D, D))
    s_in[1] = s0
    ref = _oracle_prefill(d, cu, start_pos=[0, 1024], s0=s_in, **{k: ck[k] for k in ("ckpt_cu", "ckpt_pos")})
    got = o.double().cpu().numpy()
    assert np.all(np.isfinite(got))
    err = max_rel_blocks(got, ref["o"], cu, H)
    for m, p in enumerate(ck["ckpt_page"]):
        err = max(err, max(rel_fro(pb.states(p)[h], ref["ckpts"][m, h]) for h in range(H)))
    for s_ in range(2):
        err = max(err, max(rel_fro(pb.states(s_)[h], ref["s_final"][s_, h]) for h in range(H)))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_identity_beta0_alpha1(dtype):
    """beta = 0 and alpha = 1 (g = 0): S_t = S_{t-1}.  The entering state comes
    back bit for bit in every checkpoint and in the final state, and
    o_t = S0^T q_t matches the oracle."""
    H, D = 2, 128
    T = 700
    d = G.kda_tokens(99, H, D, 0, T, dtype)
    d["beta"] = _const(d["beta"], dtype, 0.0)
    d["g"] = _const(d["g"], dtype, 0.0)
    s0 = (np.random.default_rng(11).standard_normal((H, D, D)) / np.sqrt(D)).astype(np.float32)
    pb = PoolBuf(4, H, D)
    pb.set_states(3, s0)
    o = prefill(pb, inputs_to_dev(d, dtype), [0, T], dtype, start_pos=[512], state_in_page=[3],
                state_out_page=[0], ckpt_cu=[0, 1], ckpt_pos=[1024], ckpt_page=[1])
    assert np.array_equal(pb.states(0), s0.astype(np.float64))
    assert np.array_equal(pb.states(1), s0.astype(np.float64))
    ref = _oracle_prefill(d, [0, T], start_pos=[512], s0=s0[None].astype(np.float64))
    err = max_rel_blocks(o.double().cpu().numpy(), ref["o"], [0, T], H)
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_out_of_domain_gates_are_not_silent(dtype):
    """Gates past the chunk form's domain (g = -4 everywhere: a half chunk of
    gates sums to -128, beyond the |G_i - G_31| < 87 that include/kda.h states)
    give non-finite outputs and a non-finite state, never finite values that
    could pass for a result.  (The recurrence itself is finite there; the
    oracle is not consulted.)"""
    H, D, T = 2, 128, 300
    d = G.kda_tokens(5, H, D, 0, T, dtype)
    d["g"] = _const(d["g"], dtype, -4.0)
    pb = PoolBuf(2, H, D)
    o = prefill(pb, inputs_to_dev(d, dtype), [0, T], dtype, state_out_page=[0])
    assert not bool(torch.isfinite(o).all())
    assert not np.isfinite(pb.states(0)).all()


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_exact_write_beta1_unit_key(dtype):
    """beta = 1 with unit keys: the delta rule overwrites the value stored under
    the key, S_t^T k_t = v_t (up to ||k_t||^2 - 1, the rounding of the stored
    keys).  Checked on the final state against the last token, and against
    the oracle."""
    H, D = 2, 128
    T = 333
    d = G.kda_tokens(2718, H, D, 0, T, dtype)
    d["beta"] = _const(d["beta"], dtype, 1.0)
    pb = PoolBuf(2, H, D)
    o = prefill(pb, inputs_to_dev(d, dtype), [0, T], dtype, state_out_page=[0])
    k_last, v_last = _f64(d["k"][T - 1], dtype), _f64(d["v"][T - 1], dtype)
    S = pb.states(0)
    for h in range(H):
        kn2 = float(k_last[h] @ k_last[h])
        got = S[h].T @ k_last[h]
        # S'^T k + ||k||^2 (v - S'^T k) = v + (||k||^2 - 1)(v - S'^T k)
        # plus the state's own error, at most TOL * ||S||_F (checked below)
        bound = (2 * abs(kn2 - 1.0) * (np.linalg.norm(v_last[h]) + np.linalg.norm(got))
                 + TOL[dtype] * np.linalg.norm(S[h]))
        assert np.linalg.norm(got - v_last[h]) <= bound, (h, np.linalg.norm(got - v_last[h]), bound)
    ref = _oracle_prefill(d, [0, T])
    err = max(rel_fro(S[h], ref["s_final"][0, h]) for h in range(H))
    err = max(err, max_rel_blocks(o.double().cpu().numpy(), ref["o"], [0, T], H))
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("page_bytes", [2 << 20, (2 << 20) + 4096])
def test_prefill_8k_full(page_bytes):
    """H=32, d=128, T=8192, bf16 inputs, fp32 state, checkpoints {2560, 6144, 8192}
    into 2 MiB pages (and a padded page size); all heads checked."""
    w = G.PREFILL_8K
    d = G.kda_tokens(w.seed, w.H, w.D, 0, w.T, w.dtype)
    pb = PoolBuf(8, w.H, w.D, page_bytes=page_bytes)
    ck_pages = [5, 2, 7]
    before = pb.snapshot()
    di = inputs_to_dev(d, w.dtype)
    kw = dict(ckpt_cu=[0, 3], ckpt_pos=list(w.ckpts), ckpt_page=ck_pages, state_out_page=[0])
    o = prefill(pb, di, [0, w.T], w.dtype, **kw)
    after = pb.snapshot()
    ref = _oracle_prefill(d, [0, w.T], ckpt_cu=[0, 3], ckpt_pos=list(w.ckpts))
    err_o = max_rel_blocks(o.double().cpu().numpy(), ref["o"], [0, w.T], w.H)
    err_c = max(rel_fro(pb.states(p)[h], ref["ckpts"][m, h])
                for m, p in enumerate(ck_pages) for h in range(w.H))
    assert err_o <= TOL["bf16"] and err_c <= TOL["bf16"], (err_o, err_c)
    assert _poison_mask_ok(before, after, pb, ck_pages + [0])
    assert np.array_equal(pb.states(7), pb.states(0))  # checkpoint at T == final state
    # determinism: a second run gives bitwise-identical outputs and pages
    o2 = prefill(pb, di, [0, w.T], w.dtype, **kw)
    assert torch.equal(o.view(torch.int16), o2.view(torch.int16))
    assert np.array_equal(after, pb.snapshot())


@pytest.mark.parametrize("g_lo", [-0.05, -0.001])
def test_resume_bitwise_and_oracle(g_lo):
    """Prefill [0, B) with a checkpoint at B, restore it into a fresh active page,
    prefill [B, T) from it: bitwise equal to the uninterrupted GPU run, and both
    match the oracle.  The slow-decay variant keeps a wrong restore visible long
    after B."""
    H, D, T, B = 8, 128, 3000, 1536
    d = G.kda_tokens(777, H, D, 0, T, "bf16", g_lo=g_lo)
    di = inputs_to_dev(d, "bf16")
    pb = PoolBuf(8, H, D)
    o_full = prefill(pb, di, [0, T], "bf16", ckpt_cu=[0, 1], ckpt_pos=[B], ckpt_page=[1],
                     state_out_page=[2])
    pre = {k: v[:B] for k, v in di.items()}
    suf = {k: v[B:].contiguous() for k, v in di.items()}
    o_pre = prefill(pb, pre, [0, B], "bf16", ckpt_cu=[0, 1], ckpt_pos=[B], ckpt_page=[3])
    ck_bytes = pb.page_words(3).clone()
    K.kda_checkpoint_restore(pb.pool, [3], [4])
    o_suf = prefill(pb, suf, [0, T - B], "bf16", start_pos=[B], state_in_page=[4],
                    state_out_page=[5])
    assert torch.equal(pb.page_words(3), ck_bytes)  # checkpoint stayed read-only
    assert torch.equal(o_full[:B].view(torch.int16), o_pre.view(torch.int16))
    assert torch.equal(o_full[B:].view(torch.int16), o_suf.view(torch.int16))
    assert np.array_equal(pb.states(1), pb.states(3))
    assert np.array_equal(pb.states(2), pb.states(5))
    ref = _oracle_prefill(d, [0, T], ckpt_cu=[0, 1], ckpt_pos=[B])
    err = max(max_rel_blocks(o_full.double().cpu().numpy(), ref["o"], [0, T], H),
              max(rel_fro(pb.states(1)[h], ref["ckpts"][0, h]) for h in range(H)),
              max(rel_fro(pb.states(2)[h], ref["s_final"][0, h]) for h in range(H)))
    assert err <= TOL["bf16"], err


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_many_heads(dtype, D):
    """96 heads (one layer's KDA heads in the pages' model): the library picks
    32-column slabs on its own at this head count and cuts the call into windows
    of 21 chunks, which sequences cross.  Three sequences, one entering from a
    state at position 1024, checkpoints inside and at the ends; every head
    compared with the oracle on o, the checkpoints and the final states."""
    H = 96
    cu = [0, 2900, 4100, 4800]
    T = cu[-1]
    d = G.kda_tokens(4242 + D, H, D, 0, T, dtype)
    pb = PoolBuf(9, H, D)
    rng = np.random.default_rng(11)
    s_in = (rng.standard_normal((H, D, D)) / np.sqrt(D)).astype(np.float32).astype(np.float64)
    pb.set_states(8, s_in)
    start = [0, 1024, 0]
    # absolute checkpoint positions: seq 0 at 512, 1536 and its end (2900 is no
    # block end: only 512 and 1536 qualify), seq 1 at 1536 and 2048, seq 2 none
    ckpt_cu, ckpt_pos, ckpt_page = [0, 2, 4, 4], [512, 1536, 1536, 2048], [3, 4, 5, 6]
    before = pb.snapshot()
    o = prefill(pb, inputs_to_dev(d, dtype), cu, dtype, start_pos=start, state_in_page=[-1, 8, -1],
                state_out_page=[0, 1, 2], ckpt_cu=ckpt_cu, ckpt_pos=ckpt_pos, ckpt_page=ckpt_page)
    s0 = np.zeros((3, H, D, D))
    s0[1] = s_in
    ref = _oracle_prefill(d, cu, start_pos=start, s0=s0, ckpt_cu=ckpt_cu, ckpt_pos=ckpt_pos)
    err_o = max_rel_blocks(o.double().cpu().numpy(), ref["o"], cu, H)
    err_c = max(rel_fro(pb.states(ckpt_page[m])[h], ref["ckpts"][m, h]) for m in range(4) for h in range(H))
    err_s = max(rel_fro(pb.states(s)[h], ref["s_final"][s, h]) for s in range(3) for h in range(H))
    assert max(err_o, err_c, err_s) <= TOL[dtype], (err_o, err_c, err_s)
    assert _poison_mask_ok(before, pb.snapshot(), pb, [0, 1, 2, 3, 4, 5, 6])


def test_in_place_and_empty_sequence_with_state():
    """state_in == state_out updates in place; a zero-length sequence with an
    entering state copies it to its output page unchanged."""
    H, D = 4, 64
    cu = [0, 640, 640]
    d = G.kda_tokens(99, H, D, 0, 640, "f32")
    pb = PoolBuf(6, H, D)
    rng = np.random.default_rng(5)
    s0 = rng.standard_normal((2, H, D, D)) / np.sqrt(D)
    pb.set_states(1, s0[0])
    pb.set_states(2, s0[1])
    o = prefill(pb, inputs_to_dev(d, "f32"), cu, "f32", start_pos=[1024, 4096],
                state_in_page=[1, 2], state_out_page=[1, 3],
                ckpt_cu=[0, 1, 1], ckpt_pos=[1536], ckpt_page=[4])
    s0_f32 = s0.astype(np.float32).astype(np.float64)
    ref = _oracle_prefill(d, cu, start_pos=[1024, 4096], s0=s0_f32, ckpt_cu=[0, 1, 1],
                          ckpt_pos=[1536])
    assert max_rel_blocks(o.double().cpu().numpy(), ref["o"], cu, H) <= 1e-4
    assert max(rel_fro(pb.states(1)[h], ref["s_final"][0, h]) for h in range(H)) <= 1e-4
    assert max(rel_fro(pb.states(4)[h], ref["ckpts"][0, h]) for h in range(H)) <= 1e-4
    assert np.array_equal(pb.states(3), s0_f32[1])


def test_varlen_resume_batch():
    """16 sequences, lengths uniform in [1024, 32768]; each resumes from a
    checkpoint at a random 512-multiple B < len.  Prefix pass writes the
    checkpoints, restore copies them to fresh active pages, the packed suffix
    pass resumes.  Checked against the uninterrupted oracle on all 32 heads:
    the suffix o, the checkpoint at B and the final state of every sequence."""
    w = G.VARLEN_RESUME
    lens, bnd = G.varlen_plan(w)
    print(f"varlen: lens {lens.tolist()} boundaries {bnd.tolist()}", flush=True)
    ns, H, D = w.n_seqs, w.H, w.D
    seqs = [G.kda_tokens(w.seed, H, D, 0, int(L), w.dtype, seq_id=s) for s, L in enumerate(lens)]
    cat = lambda parts: np.concatenate(parts, axis=0)  # noqa: E731
    pre = {k: cat([sq[k][:b] for sq, b in zip(seqs, bnd)]) for k in seqs[0]}
    suf = {k: cat([sq[k][b:] for sq, b in zip(seqs, bnd)]) for k in seqs[0]}
    cu_pre = np.concatenate([[0], np.cumsum(bnd)])
    cu_suf = np.concatenate([[0], np.cumsum(lens - bnd)])
    pb = PoolBuf(3 * ns, H, D, page_bytes=2 << 20)
    ck_pages = list(range(ns))
    act_pages = list(range(ns, 2 * ns))
    fin_pages = list(range(2 * ns, 3 * ns))
    prefill(pb, inputs_to_dev(pre, "bf16"), cu_pre, "bf16", ckpt_cu=np.arange(ns + 1),
            ckpt_pos=bnd, ckpt_page=ck_pages)
    K.kda_checkpoint_restore(pb.pool, ck_pages, act_pages)
    o_suf = prefill(pb, inputs_to_dev(suf, "bf16"), cu_suf, "bf16", start_pos=bnd,
                    state_in_page=act_pages, state_out_page=fin_pages)
    o_suf = o_suf.double().cpu().numpy()
    heads = list(range(H))
    full = {k: cat([sq[k] for sq in seqs]) for k in seqs[0]}
    cu_full = np.concatenate([[0], np.cumsum(lens)])
    print(f"varlen: oracle on {int(cu_full[-1])} tokens x {H} heads", flush=True)
    ref = _oracle_prefill(full, cu_full, ckpt_cu=np.arange(ns + 1), ckpt_pos=bnd)
    worst = 0.0
    for s in range(ns):
        a, b = int(cu_full[s]) + int(bnd[s]), int(cu_full[s + 1])
        sa, sb = int(cu_suf[s]), int(cu_suf[s + 1])
        ck_s, fin_s = pb.states(ck_pages[s]), pb.states(fin_pages[s])
        for j, h in enumerate(heads):
            worst = max(worst, rel_fro(o_suf[sa:sb, h], ref["o"][a:b, j]),
                        rel_fro(ck_s[h], ref["ckpts"][s, j]),
                        rel_fro(fin_s[h], ref["s_final"][s, j]))
    assert worst <= TOL["bf16"], worst


@pytest.mark.slow
@pytest.mark.timeout(900)
def test_long_1m():
    """T = 2^20 tokens, H=32, d=128, bf16, 171 checkpoints streamed to the pool
    through the library's windows.  The oracle runs four full heads (0, 5, 13,
    31: all tokens, all checkpoints), each checked on o and on every one of
    the 171 checkpoints; every head's checkpoints must be finite."""
    w = G.LONG_1M
    print("long_1m: generating inputs", flush=True)
    d = G.kda_tokens(w.seed, w.H, w.D, 0, w.T, w.dtype)
    print("long_1m: copying to device", flush=True)
    di = inputs_to_dev(d, w.dtype)
    nck = len(w.ckpts)
    pb = PoolBuf(nck + 1, w.H, w.D, page_bytes=w.page_bytes)
    o = prefill(pb, di, [0, w.T], w.dtype, ckpt_cu=[0, nck], ckpt_pos=list(w.ckpts),
                ckpt_page=list(range(nck)), state_out_page=[nck])
    del di
    heads = [0, 5, 13, 31]
    print(f"long_1m: GPU done, running the oracle on heads {heads}", flush=True)
    ref = _oracle_prefill(d, [0, w.T], ckpt_cu=[0, nck], ckpt_pos=list(w.ckpts), heads=heads)
    err_c = np.zeros(len(heads))
    for m in range(nck):
        st = pb.states(m)
        for j, h in enumerate(heads):
            err_c[j] = max(err_c[j], rel_fro(st[h], ref["ckpts"][m, j]))
    for j, h in enumerate(heads):
        err_o = rel_fro(o[:, h].double().cpu().numpy(), ref["o"][:, j])
        print(f"long_1m: head {h}: o {err_o:.2e}, worst of {nck} checkpoints {err_c[j]:.2e}", flush=True)
        assert err_o <= TOL["bf16"] and err_c[j] <= TOL["bf16"], (h, err_o, err_c[j])
    assert np.array_equal(pb.states(nck - 1), pb.states(nck))
    for m in range(0, nck, 17):
        assert np.all(np.isfinite(pb.states(m)))


def test_metadata_paths_bitwise():
    """Calls with at most 16 sequences and 64 checkpoints carry their tables in
    the kernel arguments, larger ones in the workspace: 20 sequences with a
    checkpoint each in one call (workspace tables) must equal, bit for bit, the
    same sequences in two calls of 10 (inline tables)."""
    H, D, dtype = 2, 128, "bf16"
    lens = [600 + 64 * (i % 7) + (i * 37) % 50 for i in range(20)]
    cu = np.concatenate([[0], np.cumsum(lens)])
    d = G.kda_tokens(4321, H, D, 0, int(cu[-1]), dtype)
    di = inputs_to_dev(d, dtype)
    ck = [512] * 20
    pb = PoolBuf(80, H, D)
    o_all = prefill(pb, di, cu, dtype, ckpt_cu=np.arange(21), ckpt_pos=ck, ckpt_page=list(range(20)),
                    state_out_page=list(range(20, 40)))
    outs = []
    for half in range(2):
        a, b = 10 * half, 10 * half + 10
        sub = {k: v[int(cu[a]):int(cu[b])] for k, v in di.items()}
        outs.append(prefill(pb, sub, cu[a:b + 1] - cu[a], dtype, ckpt_cu=np.arange(11), ckpt_pos=ck[a:b],
                            ckpt_page=list(range(40 + a, 40 + b)), state_out_page=list(range(60 + a, 60 + b))))
    assert torch.equal(o_all, torch.cat(outs, dim=0))
    for s in range(20):
        assert np.array_equal(pb.states(s), pb.states(40 + s))        # checkpoints
        assert np.array_equal(pb.states(20 + s), pb.states(60 + s))   # final states


def test_graph_replay_bitwise():
    """The prefill call captured once in a HIP graph (metadata travels in kernel
    arguments, so nothing is re-validated at replay) and replayed three times,
    with eager work and synchronisation between replays: every replay rewrites
    o, the checkpoint page and the final page bit-identically to the eager call."""
    H, D, T = 4, 128, 1000
    d = G.kda_tokens(77, H, D, 0, T, "bf16")
    di = inputs_to_dev(d, "bf16")
    pb = PoolBuf(3, H, D)
    kw = dict(ckpt_cu=[0, 1], ckpt_pos=[512], ckpt_page=[1], state_out_page=[2])
    ws = torch.empty(K.kda_prefill_workspace_bytes(pb.pool, T, 1, 1, K.KDA_BF16), dtype=torch.uint8,
                     device="cuda")
    o = torch.empty((T, H, D), dtype=torch.bfloat16, device="cuda")

    def call():
        K.kda_prefill_chunked(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, [0, T],
                              workspace=ws, **kw)

    call()
    torch.cuda.synchronize()
    ref_o, ref_pool = o.view(torch.int16).cpu().numpy().copy(), pb.snapshot()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        call()
    torch.cuda.current_stream().wait_stream(side)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        call()
    poison = np.int32(np.uint32(POISON_WORD).view(np.int32))
    for _ in range(3):
        o.fill_(float("nan"))
        pb.buf.fill_(poison)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_pool = pb.snapshot()
        assert np.array_equal(o.view(torch.int16).cpu().numpy(), ref_o)
        sw = pb.state_bytes // 4
        for p in (1, 2):
            assert np.array_equal(got_pool[p * sw:(p + 1) * sw], ref_pool[p * sw:(p + 1) * sw])
        assert np.all(got_pool[:sw] == poison)  # page 0 is not an output of the call


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_slab_width_bitwise(dtype, monkeypatch):
    """Every value column of the state is carried on its own (the d_v split), so
    16- and 32-column slabs (KDA_SCAN_SLAB=1 / 2 overrides the size-based choice)
    give bit-identical o, checkpoints and final states."""
    H, D = 4, 128
    cu = np.array([0, 700, 2000])
    d = G.kda_tokens(99, H, D, 0, int(cu[-1]), dtype)
    di = inputs_to_dev(d, dtype)
    res = []
    for nh in ("1", "2"):
        monkeypatch.setenv("KDA_SCAN_SLAB", nh)
        pb = PoolBuf(4, H, D)
        o = prefill(pb, di, cu, dtype, ckpt_cu=[0, 1, 2], ckpt_pos=[512, 1024], ckpt_page=[0, 1],
                    state_out_page=[2, 3])
        res.append((o.cpu(), pb.snapshot()))
    assert torch.equal(res[0][0].view(torch.int16) if dtype == "bf16" else res[0][0],
                       res[1][0].view(torch.int16) if dtype == "bf16" else res[1][0])
    assert np.array_equal(res[0][1], res[1][1])


@pytest.mark.parametrize("dtype,nseq", [("bf16", 4), ("f32", 4), ("bf16", 20)])
def test_window_size_bitwise(dtype, nseq):
    """A call runs in windows of consecutive chunks that fit the workspace it is
    given.  The preferred workspace, the smallest accepted one (one chunk per
    window) and one of three chunks per window give bit-identical o,
    checkpoints and final states: a sequence cut by a window edge carries its
    fp32 state across unchanged.  Covers resumed sequences, an empty sequence
    with a state, checkpoints on window edges and inside windows, and (20
    sequences) the tables shipped through the workspace rather than inline.
    The preferred run matches the oracle."""
    H, D = 4, 128
    rng = np.random.default_rng(nseq)
    if nseq == 4:
        lens = [2500, 0, 1600, 900]
    else:
        lens = [int(x) for x in rng.integers(1, 700, nseq)]
        lens[1] = 0
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    sp = [64 * int(x) for x in rng.integers(0, 20, nseq)]
    sp[0] = 0
    s_in = [-1] * nseq
    s_in[1], s_in[2] = 2 * nseq, 2 * nseq + 1
    s_out = list(range(nseq))
    ck_cu, ck_pos, ck_page = [0], [], []
    for i in range(nseq):
        for pos in range((sp[i] // 512 + 1) * 512, sp[i] + lens[i] + 1, 512):
            ck_pos.append(pos)
            ck_page.append(2 * nseq + 2 + len(ck_page))
        ck_cu.append(len(ck_pos))
    nck = len(ck_pos)
    npages = 2 * nseq + 2 + nck
    d = G.kda_tokens(2024 + nseq, H, D, 0, int(cu[-1]), dtype)
    di = inputs_to_dev(d, dtype)
    ind = K.KDA_BF16 if dtype == "bf16" else K.KDA_F32
    pool0 = PoolBuf(npages, H, D).pool
    full = K.kda_prefill_workspace_bytes(pool0, int(cu[-1]), nseq, nck, ind)
    small = K.kda_prefill_workspace_min_bytes(pool0, nseq, nck, ind)
    op = 2 if dtype == "bf16" else 4
    blk = ((3 * 64 * D + 2 * 64 * 64) * op + 4 * D + 255) // 256 * 256  # one (chunk, head) block
    assert 0 < small < full // 4, (small, full)
    s0 = (np.random.default_rng(3).standard_normal((2, H, D, D)) / np.sqrt(D)).astype(np.float32)
    res = []
    for nbytes in (full, small, small + 2 * H * blk):
        pb = PoolBuf(npages, H, D)
        pb.set_states(2 * nseq, s0[0])
        pb.set_states(2 * nseq + 1, s0[1])
        ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
        o = torch.full((int(cu[-1]), H, D), float("nan"), device="cuda",
                       dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
        K.kda_prefill_chunked(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, cu,
                              start_pos=sp, state_in_page=s_in, state_out_page=s_out, workspace=ws,
                              ckpt_cu=ck_cu, ckpt_pos=ck_pos, ckpt_page=ck_page)
        torch.cuda.synchronize()
        res.append(((o.view(torch.int16) if dtype == "bf16" else o.view(torch.int32)).cpu().numpy(),
                    pb.snapshot(), o.double().cpu().numpy(), pb))
    for r in res[1:]:
        assert np.array_equal(res[0][0], r[0])
        assert np.array_equal(res[0][1], r[1])
    s0_in = np.zeros((nseq, H, D, D))
    s0_in[1], s0_in[2] = s0[0], s0[1]
    ref = _oracle_prefill(d, cu, start_pos=sp, s0=s0_in, ckpt_cu=ck_cu, ckpt_pos=ck_pos)
    pb = res[0][3]
    err = max_rel_blocks(res[0][2], ref["o"], cu, H)
    for m, p in enumerate(ck_page):
        err = max(err, max(rel_fro(pb.states(p)[h], ref["ckpts"][m, h]) for h in range(H)))
    for s_, p in enumerate(s_out):
        if lens[s_] > 0 or s_in[s_] >= 0:
            err = max(err, max(rel_fro(pb.states(p)[h], ref["s_final"][s_, h]) for h in range(H)))
    assert np.array_equal(pb.states(s_out[1]), s0_in[1])  # the empty sequence keeps its state
    assert err <= TOL[dtype], err


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 128)])
def test_unwritten_workspace_never_read(dtype, D):
    """Workspace bytes that a call does not write (the zero fragments of the
    triangular intermediates, padding) are never read: a workspace filled with
    NaN bit patterns (every byte 0xFF) and one filled with zeros give finite,
    bit-identical o, checkpoints and final states."""
    H, cu = 4, [0, 700, 2000]
    d = G.kda_tokens(101, H, D, 0, cu[-1], dtype)
    di = inputs_to_dev(d, dtype)
    ind = K.KDA_BF16 if dtype == "bf16" else K.KDA_F32
    res = []
    for fill in (0, 255):
        pb = PoolBuf(4, H, D)
        ws = torch.full((K.kda_prefill_workspace_bytes(pb.pool, cu[-1], 2, 2, ind),), fill,
                        dtype=torch.uint8, device="cuda")
        o = torch.full((cu[-1], H, D), float("nan"), device="cuda",
                       dtype=torch.bfloat16 if dtype == "bf16" else torch.float32)
        K.kda_prefill_chunked(pb.pool, di["q"], di["k"], di["v"], di["g"], di["beta"], o, cu,
                              workspace=ws, ckpt_cu=[0, 1, 2], ckpt_pos=[512, 1024],
                              ckpt_page=[0, 1], state_out_page=[2, 3])
        torch.cuda.synchronize()
        assert torch.isfinite(o.float()).all()
        res.append(((o.view(torch.int16) if dtype == "bf16" else o.view(torch.int32)).cpu().numpy(),
                    pb.snapshot()))
    assert np.array_equal(res[0][0], res[1][0])
    assert np.array_equal(res[0][1], res[1][1])
