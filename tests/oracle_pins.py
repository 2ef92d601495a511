"""Pins for the fp64 oracle: checks against what the pages and the mathematics
fix, independent of the oracle's own code.

Every pin is a function ``pin_xxx(lib_path) -> (ok: bool, detail: str)`` so the
same checks run against the real oracle (must all pass) and against the planted
mistakes of ``kda_oracle.c`` (each must fail at least one).
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np

import oracle
from oracle import exact

RNG_SEED = 20261202


def _run(lib_path, q, k, v, g, beta, **kw):
    """Single-sequence helper: arrays [T, H, d] / [T, H]."""
    T = q.shape[0]
    return oracle.run(q, k, v, g, beta, np.array([0, T]), lib_path=lib_path, **kw)


def _rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    den = max(np.linalg.norm(b), 1e-300)
    return float(np.linalg.norm(a - b) / den)


# --------------------------------------------------------------------------
# exact rational brute force (recurrence and unrolled closed form)
# --------------------------------------------------------------------------
def _rand_frac(rng, lo, hi, den=16):
    return Fraction(int(rng.integers(lo * den, hi * den + 1)), den)


def _tiny_case(rng, dk, dv, T):
    alpha = [[_rand_frac(rng, 0.25, 1.0) for _ in range(dk)] for _ in range(T)]
    beta = [_rand_frac(rng, 0.0, 1.0) for _ in range(T)]
    q = [[_rand_frac(rng, -1, 1) for _ in range(dk)] for _ in range(T)]
    k = [[_rand_frac(rng, -1, 1, 8) for _ in range(dk)] for _ in range(T)]
    v = [[_rand_frac(rng, -2, 2) for _ in range(dv)] for _ in range(T)]
    s0 = [[_rand_frac(rng, -1, 1) for _ in range(dv)] for _ in range(dk)]
    return alpha, beta, q, k, v, s0


def _to_np(x):
    return np.array([[float(e) for e in row] for row in x], np.float64)


def pin_exact_bruteforce(lib_path=None, cases=12):
    """fp64 oracle vs the exact-rational recurrence; and the exact recurrence vs
    the exact unrolled closed form (bitwise-equal rationals)."""
    rng = np.random.default_rng(RNG_SEED)
    worst = 0.0
    for case in range(cases):
        dk = int(rng.integers(2, 5))
        dv = int(rng.integers(2, 5))
        T = int(rng.integers(1, 9))
        alpha, beta, q, k, v, s0 = _tiny_case(rng, dk, dv, T)
        o_ex, st_ex = exact.recurrence(alpha, beta, q, k, v, s0)
        if case < 6:
            o_cf, st_cf = exact.closed_form(alpha, beta, q, k, v, s0)
            if o_cf != o_ex or st_cf != st_ex:
                return False, f"closed form != recurrence (case {case})"
        Q = _to_np(q)[:, None, :]
        K = _to_np(k)[:, None, :]
        V = _to_np(v)[:, None, :]
        A = _to_np(alpha)[:, None, :]
        B = np.array([float(b) for b in beta])[:, None]
        S0 = _to_np(s0)[None, None]
        r = _run(lib_path, Q, K, V, A, B, s0=S0, gate_is_alpha=True,
                 ckpt_cu=np.array([0, T]), ckpt_pos=np.arange(1, T + 1))
        worst = max(worst, _rel(r["o"][:, 0, :], _to_np(o_ex)))
        for t in range(T):
            worst = max(worst, _rel(r["ckpts"][t, 0], _to_np(st_ex[t])))
    return worst < 1e-13, f"max rel err {worst:.2e}"


# --------------------------------------------------------------------------
# special cases with closed forms
# --------------------------------------------------------------------------
def _rand_inputs(rng, T, H, dk, dv):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    g = rng.uniform(-0.05, 0.0, (T, H, dk))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    return q, k, v, g, beta


def pin_identity(lib_path=None):
    """beta = 0 and alpha = 1: the state never changes and o_t = S_0^T q_t."""
    rng = np.random.default_rng(RNG_SEED + 1)
    T, H, dk, dv = 9, 2, 5, 3
    q, k, v, _, _ = _rand_inputs(rng, T, H, dk, dv)
    g = np.zeros((T, H, dk))
    beta = np.zeros((T, H))
    s0 = rng.standard_normal((1, H, dk, dv))
    r = _run(lib_path, q, k, v, g, beta, s0=s0)
    if not np.array_equal(r["s_final"], s0):
        return False, "state changed"
    o_ref = np.einsum("hcj,thc->thj", s0[0], q)
    err = _rel(r["o"], o_ref)
    return err < 1e-14, f"o err {err:.1e}"


def pin_pure_decay(lib_path=None):
    """beta = 0: S_T = Diag(prod_t alpha_t) S_0.  With power-of-two alphas the
    products are exact, so the comparison is bitwise."""
    rng = np.random.default_rng(RNG_SEED + 2)
    T, H, dk, dv = 7, 2, 4, 6
    q, k, v, _, _ = _rand_inputs(rng, T, H, dk, dv)
    alpha = 2.0 ** (-rng.integers(0, 3, (T, H, dk)).astype(np.float64))
    beta = np.zeros((T, H))
    s0 = rng.standard_normal((1, H, dk, dv))
    r = _run(lib_path, q, k, v, alpha, beta, s0=s0, gate_is_alpha=True)
    expect = np.prod(alpha, axis=0)[:, :, None] * s0[0]
    if not np.array_equal(r["s_final"][0], expect):
        return False, f"decay mismatch {_rel(r['s_final'][0], expect):.1e}"
    # log-gate path: exp(g) in fp64, within rounding of a product of T exps
    g = rng.uniform(-0.05, 0.0, (T, H, dk))
    r2 = _run(lib_path, q, k, v, g, beta, s0=s0)
    expect2 = np.exp(g.sum(axis=0))[:, :, None] * s0[0]
    err = _rel(r2["s_final"][0], expect2)
    return err < 1e-14, f"log-gate decay err {err:.1e}"


def pin_exact_write(lib_path=None):
    """beta_t = 1 and |k_t| = 1: after token t the state maps k_t exactly to
    v_t (S_t^T k_t = v_t) whatever alpha_t and S_{t-1} are.  This holds when the
    decay is applied before the delta-rule write and fails for the reading that
    decays only inside the erase term."""
    rng = np.random.default_rng(RNG_SEED + 3)
    T, H, dk, dv = 8, 2, 6, 5
    q, k, v, g, _ = _rand_inputs(rng, T, H, dk, dv)
    g = rng.uniform(-0.7, 0.0, (T, H, dk))
    beta = np.ones((T, H))
    s0 = rng.standard_normal((1, H, dk, dv))
    r = _run(lib_path, q, k, v, g, beta, s0=s0, ckpt_cu=np.array([0, T]),
             ckpt_pos=np.arange(1, T + 1))
    worst = 0.0
    for t in range(T):
        for h in range(H):
            got = r["ckpts"][t, h].T @ k[t, h]
            worst = max(worst, float(np.max(np.abs(got - v[t, h]))))
    return worst < 1e-13, f"max |S_t^T k_t - v_t| = {worst:.1e}"


def pin_associative_memory(lib_path=None):
    """alpha = 1, beta = 1, orthonormal keys, S_0 = 0: S_n = sum_i k_i v_i^T and
    querying with k_j returns v_j (the textbook outer-product memory)."""
    rng = np.random.default_rng(RNG_SEED + 4)
    dk, dv, n = 8, 5, 6
    Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
    k = Qm[:, :n].T.copy()[:, None, :]  # n orthonormal keys
    v = rng.standard_normal((n, 1, dv))
    q = k.copy()
    g = np.zeros((n, 1, dk))
    beta = np.ones((n, 1))
    r = _run(lib_path, q, k, v, g, beta)
    expect = sum(np.outer(k[i, 0], v[i, 0]) for i in range(n))
    err = _rel(r["s_final"][0, 0], expect)
    # o_t = S_t^T k_t = v_t (the just-written pair is retrievable)
    err_o = _rel(r["o"][:, 0], v[:, 0])
    # after all writes every stored pair is retrievable
    retr = np.stack([r["s_final"][0, 0].T @ k[j, 0] for j in range(n)])
    err_r = _rel(retr, v[:, 0])
    worst = max(err, err_o, err_r)
    return worst < 1e-13, f"err {worst:.1e}"


def pin_affine_composition(lib_path=None):
    """Segment maps F_C(S) = M_C S + b_C compose as
    F_C2(F_C1(S)) = M_C2 M_C1 S + M_C2 b_C1 + b_C2, and the order matters."""
    rng = np.random.default_rng(RNG_SEED + 5)
    dk, dv, T1, T2 = 5, 4, 6, 9
    q1, k1, v1, g1, b1 = _rand_inputs(rng, T1, 1, dk, dv)
    q2, k2, v2, g2, b2 = _rand_inputs(rng, T2, 1, dk, dv)

    def seg(q, k, v, g, b, s0):
        return _run(lib_path, q, k, v, g, b, s0=s0[None, None], want_o=False)["s_final"][0, 0]

    def seg_map(q, k, v, g, b):
        T = q.shape[0]
        zv = np.zeros((T, 1, dk))
        M = _run(lib_path, q, k, zv, g, b, s0=np.eye(dk)[None, None], want_o=False)["s_final"][0, 0]
        bC = seg(q, k, v, g, b, np.zeros((dk, dv)))
        return M, bC

    M1, bb1 = seg_map(q1, k1, v1, g1, b1)
    M2, bb2 = seg_map(q2, k2, v2, g2, b2)
    S = rng.standard_normal((dk, dv))
    composed = seg(q2, k2, v2, g2, b2, seg(q1, k1, v1, g1, b1, S))
    law = M2 @ M1 @ S + M2 @ bb1 + bb2
    err = _rel(composed, law)
    # each segment is itself affine: F_C(S) = M_C S + b_C
    err1 = _rel(seg(q1, k1, v1, g1, b1, S), M1 @ S + bb1)
    swapped = seg(q1, k1, v1, g1, b1, seg(q2, k2, v2, g2, b2, S))
    noncomm = _rel(swapped, composed)
    ok = err < 1e-13 and err1 < 1e-13 and noncomm > 1e-3
    return ok, f"law err {err:.1e}, affine err {err1:.1e}, swapped diff {noncomm:.1e}"


def pin_column_independence(lib_path=None):
    """Column j of S (and of o) depends only on column j of v: running on a
    subset J of value columns reproduces S[:, J] and o[:, J] bitwise."""
    rng = np.random.default_rng(RNG_SEED + 6)
    T, H, dk, dv = 11, 2, 6, 8
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    s0 = rng.standard_normal((1, H, dk, dv))
    full = _run(lib_path, q, k, v, g, beta, s0=s0)
    J = np.array([1, 4, 5, 7])
    sub = _run(lib_path, q, k, np.ascontiguousarray(v[:, :, J]), g, beta,
               s0=np.ascontiguousarray(s0[:, :, :, J]))
    ok = (np.array_equal(sub["s_final"], full["s_final"][:, :, :, J])
          and np.array_equal(sub["o"], full["o"][:, :, J]))
    return ok, "bitwise" if ok else "column subset differs"


def pin_resume(lib_path=None):
    """Resuming from the checkpoint at B equals the uninterrupted run, bitwise
    (same fp64 operation sequence), including varlen packing."""
    rng = np.random.default_rng(RNG_SEED + 7)
    T, H, dk, dv, B = 40, 2, 5, 4, 24
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    full = _run(lib_path, q, k, v, g, beta, ckpt_cu=np.array([0, 1]), ckpt_pos=np.array([B]))
    ck = full["ckpts"][0]
    # the checkpoint equals the final state of a run over [0, B)
    pre = _run(lib_path, q[:B], k[:B], v[:B], g[:B], beta[:B])
    if not np.array_equal(pre["s_final"][0], ck):
        return False, "checkpoint != state after B tokens"
    suf = oracle.run(q[B:], k[B:], v[B:], g[B:], beta[B:], np.array([0, T - B]),
                     start_pos=np.array([B]), s0=ck[None], lib_path=lib_path)
    if not (np.array_equal(suf["o"], full["o"][B:]) and np.array_equal(suf["s_final"], full["s_final"])):
        return False, "resume differs from the uninterrupted run"
    # varlen packing: [prefix | suffix] as two sequences in one call
    packed = oracle.run(q, k, v, g, beta, np.array([0, B, T]), start_pos=np.array([0, B]),
                        s0=np.stack([np.zeros((H, dk, dv)), ck]), lib_path=lib_path)
    ok = np.array_equal(packed["o"], full["o"]) and np.array_equal(packed["s_final"][1], full["s_final"][0])
    return ok, "bitwise" if ok else "packed run differs"


def pin_checkpoint_positions(lib_path=None):
    """A checkpoint at P is the state after exactly P tokens; one at the final
    position equals the final state."""
    rng = np.random.default_rng(RNG_SEED + 8)
    T, H, dk, dv = 20, 1, 4, 4
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    P = np.array([3, 8, 20])
    r = _run(lib_path, q, k, v, g, beta, ckpt_cu=np.array([0, 3]), ckpt_pos=P)
    for m, p in enumerate(P):
        ref = _run(lib_path, q[:p], k[:p], v[:p], g[:p], beta[:p], want_o=False)["s_final"][0]
        if not np.array_equal(r["ckpts"][m], ref):
            return False, f"checkpoint at {p} is not the state after {p} tokens"
    return np.array_equal(r["ckpts"][2], r["s_final"][0]), "ok"


# --------------------------------------------------------------------------
# input decoding and head selection
# --------------------------------------------------------------------------
def _bf16_bits(x):
    """Round-to-nearest-even fp64 -> bf16 bit patterns, done by numpy on the
    fp32 bit pattern (independent of the oracle's decoding)."""
    f = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    r = ((f + 0x7FFF + ((f >> 16) & 1)) >> 16).astype(np.uint16)
    return r


def _bits_to_f64(b):
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def pin_input_widening(lib_path=None):
    """The oracle reads bf16 and fp32 inputs exactly: a run on bf16 bit
    patterns (and on the same values stored as fp32) is bitwise equal to the
    run on those values already widened to fp64 by numpy.  The inputs use
    every bf16 mantissa bit (random normals, not short fractions), and the
    fp32 run also gets values with non-zero low 16 bits."""
    rng = np.random.default_rng(RNG_SEED + 9)
    T, H, dk, dv = 13, 3, 6, 5
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    bits = [_bf16_bits(x) for x in (q, k, v, g, beta)]
    wide = [_bits_to_f64(b) for b in bits]
    kw = dict(ckpt_cu=np.array([0, 2]), ckpt_pos=np.array([5, 13]))
    ref = _run(lib_path, *wide, **kw)
    got_bf = _run(lib_path, *bits, **kw)
    got_f32 = _run(lib_path, *[w.astype(np.float32) for w in wide], **kw)
    for name, got in (("bf16", got_bf), ("fp32 (bf16 values)", got_f32)):
        for key in ("o", "s_final", "ckpts"):
            if not np.array_equal(got[key], ref[key]):
                return False, f"{name} inputs decoded differently ({key})"
    # full fp32 mantissas: fp32 storage vs the same values as fp64
    f32 = [np.asarray(x, np.float32) for x in (q, k, v, g, beta)]
    if not any(np.any(x.view(np.uint32) & 0xFFFF) for x in f32):
        return False, "fixture lacks low fp32 mantissa bits"
    r32 = _run(lib_path, *f32, **kw)
    r64 = _run(lib_path, *[x.astype(np.float64) for x in f32], **kw)
    ok = all(np.array_equal(r32[key], r64[key]) for key in ("o", "s_final", "ckpts"))
    return ok, "bitwise" if ok else "fp32 inputs decoded differently"


def pin_head_subset(lib_path=None):
    """Running a subset of heads (in any order) gives, bit for bit, the same
    outputs, final states and checkpoints as the matching slices of the
    all-heads run, with per-head entering states selected by position."""
    rng = np.random.default_rng(RNG_SEED + 10)
    T, H, dk, dv = 17, 4, 5, 3
    q, k, v, g, beta = _rand_inputs(rng, T, H, dk, dv)
    cu = np.array([0, 7, 17])
    s0 = rng.standard_normal((2, H, dk, dv))
    kw = dict(ckpt_cu=np.array([0, 1, 2]), ckpt_pos=np.array([4, 12]),
              start_pos=np.array([0, 2]))
    full = oracle.run(q, k, v, g, beta, cu, s0=s0, lib_path=lib_path, **kw)
    sel = np.array([2, 0, 3])
    sub = oracle.run(q, k, v, g, beta, cu, s0=np.ascontiguousarray(s0[:, sel]), heads=sel,
                     lib_path=lib_path, **kw)
    ok = (np.array_equal(sub["o"], full["o"][:, sel]) and
          np.array_equal(sub["s_final"], full["s_final"][:, sel]) and
          np.array_equal(sub["ckpts"], full["ckpts"][:, sel]))
    return ok, "bitwise" if ok else "head subset differs from the all-heads slices"


ALL_PINS = [pin_exact_bruteforce, pin_identity, pin_pure_decay, pin_exact_write,
            pin_associative_memory, pin_affine_composition, pin_column_independence,
            pin_resume, pin_checkpoint_positions, pin_input_widening,
            pin_head_subset]
