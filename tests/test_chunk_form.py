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
