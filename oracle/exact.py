"""Exact-rational brute force of the KDA recurrence (test infrastructure only).

Two independent statements of the same definition over ``fractions.Fraction``,
for tiny inputs (d <= 4, T <= 8):

* ``recurrence``: the per-token steps in the order fixed by page
  "Kimi K3 -- Lesson 01 - Architecture map" (gentlecold.top), section
  "两种 Attention，两种状态": decay the rows of S by alpha_t, delta-rule write
  with beta_t, k_t, v_t, then read o_t = S_t^T q_t.
* ``closed_form``: the unrolled product form of page "KIMI K3 경량 복제에서 본
  KDA의 AI 인프라 과제" (acpost.vercel.app), section 9.1:
  S_n = M_n...M_1 S_0 + sum_i M_n...M_{i+1} b_i, with the per-token affine pieces
  of its section 1.1/1.3, M_t = (I - beta_t k_t k_t^T) Diag(alpha_t) and
  b_t = beta_t k_t v_t^T.

Matrices are lists of lists of Fractions; vectors are lists.  alpha is given
directly (exact rationals), not as a log.
"""
from __future__ import annotations

from fractions import Fraction


def zeros(r, c):
    return [[Fraction(0)] * c for _ in range(r)]


def eye(n):
    m = zeros(n, n)
    for i in range(n):
        m[i][i] = Fraction(1)
    return m


def matmul(a, b):
    n, kk, m = len(a), len(b), len(b[0])
    out = zeros(n, m)
    for i in range(n):
        for p in range(kk):
            aip = a[i][p]
            if aip == 0:
                continue
            row = b[p]
            for j in range(m):
                out[i][j] += aip * row[j]
    return out


def matadd(a, b):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(a, b)]


def transpose_times_vec(s, x):
    """S^T x for S [dk][dv], x [dk]."""
    dk, dv = len(s), len(s[0])
    return [sum((s[c][j] * x[c] for c in range(dk)), Fraction(0)) for j in range(dv)]


def recurrence(alpha, beta, q, k, v, s0):
    """Token loop.  alpha/q/k: [T][dk], v: [T][dv], beta: [T], s0: [dk][dv].
    Returns (o [T][dv], states [T][dk][dv]) where states[t] is S after t+1 tokens."""
    s = [row[:] for row in s0]
    dk = len(s)
    outs, states = [], []
    for t in range(len(beta)):
        for c in range(dk):
            s[c] = [alpha[t][c] * x for x in s[c]]
        sk = transpose_times_vec(s, k[t])
        u = [v[t][j] - sk[j] for j in range(len(v[t]))]
        for c in range(dk):
            bk = beta[t] * k[t][c]
            s[c] = [s[c][j] + bk * u[j] for j in range(len(u))]
        outs.append(transpose_times_vec(s, q[t]))
        states.append([row[:] for row in s])
    return outs, states


def token_map(alpha_t, beta_t, k_t, v_t):
    """(M_t, b_t) with M_t = (I - beta k k^T) Diag(alpha), b_t = beta k v^T."""
    dk = len(k_t)
    m = eye(dk)
    for i in range(dk):
        for j in range(dk):
            m[i][j] -= beta_t * k_t[i] * k_t[j]
    for i in range(dk):
        for j in range(dk):
            m[i][j] *= alpha_t[j]
    b = [[beta_t * k_t[i] * v_t[j] for j in range(len(v_t))] for i in range(dk)]
    return m, b


def closed_form(alpha, beta, q, k, v, s0):
    """Unrolled form S_n = M_n...M_1 S_0 + sum_i M_n...M_{i+1} b_i for every n,
    and o_n = S_n^T q_n.  Same return convention as ``recurrence``."""
    maps = [token_map(alpha[t], beta[t], k[t], v[t]) for t in range(len(beta))]
    dk = len(s0)
    outs, states = [], []
    for n in range(1, len(maps) + 1):
        prod = eye(dk)  # M_n ... M_1 accumulated from the right
        for t in range(n):
            prod = matmul(maps[t][0], prod)
        s = matmul(prod, s0)
        for i in range(n):
            tail = eye(dk)  # M_n ... M_{i+2}  (0-based: maps[i+1..n-1])
            for t in range(i + 1, n):
                tail = matmul(maps[t][0], tail)
            s = matadd(s, matmul(tail, maps[i][1]))
        states.append(s)
        outs.append(transpose_times_vec(s, q[n - 1]))
    return outs, states


def segment_map(alpha, beta, k, v, dv):
    """(M_C, b_C) of a token segment: M_C = M_n...M_1, b_C = F_C(0)."""
    dk = len(k[0])
    m = eye(dk)
    b = zeros(dk, dv)
    for t in range(len(beta)):
        mt, bt = token_map(alpha[t], beta[t], k[t], v[t])
        m = matmul(mt, m)
        b = matadd(matmul(mt, b), bt)
    return m, b
