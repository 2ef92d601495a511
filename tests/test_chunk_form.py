"""The chunk-parallel form used by the GPU prefill equals the token recurrence.

Derivation (from the per-token steps; the acpost page, section 1.3, only says a
token segment collapses to one affine map, which is what licenses chunking):
inside a chunk of C tokens with entering state S0, let G_r = sum_{i<=r} g_i
(per key channel), e_r = exp(G_r), and

    Kt = K * e,  Kh = K * e^-1,  Qt = Q * e,  Kend = K * (e_C / e),
    A  = strictLower(Kt Kh^T),   Aq = lowerIncl(Qt Kh^T),
    T  = (I + diag(beta) A)^-1 diag(beta).
Then  W = T (V - Kt S0),  O = Qt S0 + Aq W,  S_C = diag(e_C) S0 + Kend^T W.
The GPU keeps the S-independent parts precomputed (Keff = T Kt, Qt, Aq, T,
Kend), so that W = T V - Keff S0 and O = Qt S0 + Aq W.
A partial final chunk is padded with k = q = v = g = beta = 0 rows, which leave
the state unchanged.  This is a CPU model of the GPU algorithm; the oracle it
is compared with is the token loop.
"""
import numpy as np
import pytest

import oracle


def chunk_prefill(q, k, v, g, beta, s0, C=64):
    T, dk = q.shape
    dv = v.shape[1]
    S = s0.copy()
    o = np.zeros((T, dv))
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pad = lambda x: np.concatenate([x[c0:c0 + n], np.zeros((C - n,) + x.shape[1:])])  # noqa
        Q, K, V, Gt, b = pad(q), pad(k), pad(v), pad(g), pad(beta)
        G = np.cumsum(Gt, axis=0)
        e = np.exp(G)
        Kt, Kh, Qt = K * e, K / e, Q * e
        Kend = K * (e[-1] / e)
        A = np.tril(Kt @ Kh.T, -1)
        Aq = np.tril(Qt @ Kh.T)
        Tm = np.linalg.solve(np.eye(C) + b[:, None] * A, np.diag(b))
        Keff = Tm @ Kt
        W = Tm @ V - Keff @ S
        O = Qt @ S + Aq @ W
        S = e[-1][:, None] * S + Kend.T @ W
        o[c0:c0 + n] = O[:n]
    return o, S


@pytest.mark.parametrize("T,dk,dv,C", [(64, 8, 8, 64), (200, 16, 8, 64), (150, 8, 12, 32), (7, 4, 4, 64)])
def test_chunk_form_matches_token_recurrence(oracle_lib, T, dk, dv, C):
    rng = np.random.default_rng(T * 31 + dk)
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    g = rng.uniform(-0.05, 0, (T, dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    s0 = rng.standard_normal((dk, dv))
    o, S = chunk_prefill(q, k, v, g, beta, s0, C)
    r = oracle.run(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                   np.array([0, T]), s0=s0[None, None])
    assert np.linalg.norm(o - r["o"][:, 0]) / np.linalg.norm(r["o"]) < 1e-12
    assert np.linalg.norm(S - r["s_final"][0, 0]) / np.linalg.norm(S) < 1e-12


def chunk_prefill_f32_midref(q, k, v, g, beta, s0, C=64):
    """The same chunk form evaluated in fp32 with the factorisation of the GPU
    prefill: the Gram products take the prefix through the chunk's 32nd token
    as reference (Kt' = K e^(G - G_31), Kh' = K e^(G_31 - G), Qt' = Q e^(G - G_31);
    products over a channel equal K_i K_j e^(G_i - G_j) as before), the
    state-side operands the chunk start (Kt = K e^G, Qt = Q e^G,
    Kend = K e^(G_C - G)), so no factor exceeds half a chunk of gates."""
    f = np.float32
    T, dk = q.shape
    dv = v.shape[1]
    S = s0.astype(f)
    o = np.zeros((T, dv), f)
    finite = True
    for c0 in range(0, T, C):
        n = min(C, T - c0)
        pad = lambda x: np.concatenate([x[c0:c0 + n], np.zeros((C - n,) + x.shape[1:])]).astype(f)  # noqa
        Q, K, V, Gt, b = pad(q), pad(k), pad(v), pad(g), pad(beta)
        G = np.cumsum(Gt, axis=0, dtype=f)
        GM = G[min(31, C - 1)]
        em, im = np.exp(G - GM), np.exp(GM - G)
        Ktp, Khp, Qtp = K * em, K * im, Q * em
        Kt, Qt, Kend = K * np.exp(G), Q * np.exp(G), K * np.exp(G[-1] - G)
        finite &= bool(np.all(np.isfinite(em)) and np.all(np.isfinite(im)))
        with np.errstate(over="ignore", invalid="ignore"):  # right of the diagonal: discarded
            A = np.tril(Ktp @ Khp.T, -1)
            Aq = np.tril(Qtp @ Khp.T)
        Tm = np.linalg.solve(np.eye(C, dtype=f) + b[:, None] * A, np.diag(b)).astype(f)
        Keff = Tm @ Kt
        W = Tm @ V - Keff @ S
        O = Qt @ S + Aq @ W
        S = np.exp(G[-1])[:, None] * S + Kend.T @ W
        o[c0:c0 + n] = O[:n]
    return o, S, finite


@pytest.mark.parametrize("g_lo,g_hi", [(-3.0, 0.0), (-2.7, -2.6), (-0.05, 0.0)])
def test_midchunk_reference_in_fp32(oracle_lib, g_lo, g_hi):
    """With strong gates (log alpha ~ U(-3, 0), or about -2.7 per token: the gate
    sums over a chunk reach about -96 and -173) the fp32 evaluation with the
    mid-chunk reference keeps every factor finite and matches the token
    recurrence to fp32 accuracy, while the chunk-start factor exp(-G) of the
    same chunks overflows fp32."""
    T, dk, dv = 200, 16, 8
    rng = np.random.default_rng(int(-g_lo * 100))
    q = rng.standard_normal((T, dk)); q /= np.linalg.norm(q, axis=1, keepdims=True)
    k = rng.standard_normal((T, dk)); k /= np.linalg.norm(k, axis=1, keepdims=True)
    v = rng.standard_normal((T, dv))
    g = rng.uniform(g_lo, g_hi, (T, dk))
    beta = 1 / (1 + np.exp(-rng.standard_normal(T)))
    s0 = rng.standard_normal((dk, dv))
    o, S, finite = chunk_prefill_f32_midref(q, k, v, g, beta, s0)
    assert finite
    r = oracle.run(q[:, None], k[:, None], v[:, None], g[:, None], beta[:, None],
                   np.array([0, T]), s0=s0[None, None])
    assert np.linalg.norm(o - r["o"][:, 0]) / np.linalg.norm(r["o"]) < 1e-4
    assert np.linalg.norm(S - r["s_final"][0, 0]) / np.linalg.norm(r["s_final"]) < 1e-4
    G = np.cumsum(g[:64].astype(np.float32), axis=0)
    with np.errstate(over="ignore"):
        overflow = not np.all(np.isfinite(np.exp(-G)))
    assert overflow == (g_lo <= -2.0)

