"""Closed parallel forms on tiny inputs (single sequence, single head).

TEST INFRASTRUCTURE ONLY (see the package docstring).

These are different statements of the same outputs, used to pin the
recurrence from outside itself:
  * ``linear_parallel_fp64``  - masked (and optionally decayed) linear attention
    as one score matrix times V ("From Attention to Learned Memory" section 2,
    the fully parallel masked form; decayed scores from the RetNet, Mamba-2 and
    GLA parallel forms of "Linear attention visualized"). Decay factors are
    explicit products of alpha, not differences of cumulative sums.
  * ``delta_parallel_fp64``   - ungated DeltaNet from zero state through the
    full-sequence triangular correction system of "Linear attention
    visualized" (DeltaNet: "The triangular correction system" and "Parallel
    output"), solved row by row.
  * ``four_token_chunk_fractions`` - the four-token chunk of section 6 of "You
    Could Have Come Up With Kimi Delta Attention", every printed term
    (provisional errors, the e_0..e_3 substitutions, the chunk-end state and
    o_0..o_3) written out one by one in exact rational arithmetic.
"""
from __future__ import annotations

from fractions import Fraction
from typing import List, Sequence

import numpy as np

__all__ = ["linear_parallel_fp64", "delta_parallel_fp64",
           "four_token_chunk_fractions"]


def linear_parallel_fp64(q, k, v, scale, alpha=None, S0=None):
    """o_t = s [ sum_{j<=t} (q_t^T Diag(a_{j+1..t}) k_j) v_j + S0 Diag(a_{1..t}) q_t ].

    q, k [T, d_k]; v [T, d_v]; alpha None (no decay), [T] (scalar per token) or
    [T, d_k] (per key channel); S0 [d_v, d_k] or None. a_{j+1..t} is the
    product of the per-token retention factors strictly after j up to t.
    Returns (o [T, d_v], S_T [d_v, d_k]).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, dk = q.shape
    dv = v.shape[1]
    if alpha is None:
        a = np.ones((T, dk))
    else:
        a = np.asarray(alpha, np.float64)
        a = np.repeat(a[:, None], dk, 1) if a.ndim == 1 else a
    S0 = np.zeros((dv, dk)) if S0 is None else np.asarray(S0, np.float64)

    def decay(lo, hi):             # product of a_u for u in [lo, hi], per channel
        d = np.ones(dk)
        for u in range(lo, hi + 1):
            d = d * a[u]
        return d

    o = np.zeros((T, dv))
    for t in range(T):
        acc = S0 @ (decay(0, t) * q[t])
        for j in range(t + 1):
            acc = acc + np.dot(q[t], decay(j + 1, t) * k[j]) * v[j]
        o[t] = scale * acc
    ST = S0 * decay(0, T - 1)[None, :]
    for j in range(T):
        ST = ST + np.outer(v[j], decay(j + 1, T - 1) * k[j])
    return o, ST


def delta_parallel_fp64(q, k, v, beta, scale):
    """Ungated DeltaNet from S0 = 0 as one triangular solve over the sequence.

    u_t = beta_t (v_t - sum_{i<t} (k_i . k_t) u_i)  i.e. (I + B L) U = B V with
    L_ti = k_t . k_i strictly below the diagonal; the state is sum_i u_i k_i^T
    and o_t = s sum_{i<=t} (k_i . q_t) u_i (the linear-attention read with U in
    place of V).
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    beta = np.asarray(beta, np.float64)
    T = q.shape[0]
    U = np.zeros_like(v)
    for t in range(T):
        acc = v[t].copy()
        for i in range(t):
            acc = acc - np.dot(k[i], k[t]) * U[i]
        U[t] = beta[t] * acc
    o = np.zeros_like(v)
    for t in range(T):
        for i in range(t + 1):
            o[t] = o[t] + np.dot(k[i], q[t]) * U[i]
    ST = U.T @ k
    return scale * o, ST


# ----------------------------------------------------------------------------
# exact rational four-token chunk
# ----------------------------------------------------------------------------

Vec = List[Fraction]


def _mv(M, x):                      # matrix [rows][cols] times column vector
    return [sum((M[r][c] * x[c] for c in range(len(x))), Fraction(0))
            for r in range(len(M))]


def _dot(a, b):
    return sum((x * y for x, y in zip(a, b)), Fraction(0))


def _had(a, b):                     # elementwise product (diagonal matrices)
    return [x * y for x, y in zip(a, b)]


def _axpy(alpha, x, y):             # y + alpha x
    return [yi + alpha * xi for xi, yi in zip(x, y)]


def _outer(a, b):
    return [[x * y for y in b] for x in a]


def _madd(A, B):
    return [[x + y for x, y in zip(ra, rb)] for ra, rb in zip(A, B)]


def _mcolscale(M, d):               # M Diag(d)
    return [[x * di for x, di in zip(row, d)] for row in M]


def four_token_chunk_fractions(S: Sequence[Sequence[Fraction]],
                               alpha: Sequence[Vec], beta: Sequence[Fraction],
                               k: Sequence[Vec], v: Sequence[Vec],
                               q: Sequence[Vec], s: Fraction):
    """Section 6.1-6.5 of the KDA page for tokens 0..3, term by term.

    S [d_v][d_k] incoming state, alpha[i] the per-channel retention of token i
    (a scalar gate is a constant vector), beta[i], k[i], v[i], q[i] vectors, s
    the query scale. Returns (outputs o_0..o_3, S_{c+1}) as Fractions.
    """
    one = [Fraction(1)] * len(k[0])
    D = [list(a) for a in alpha]                      # D_i = Diag(alpha_i)
    D01 = _had(D[0], D[1])
    D012 = _had(D01, D[2])
    D0123 = _had(D012, D[3])
    D12 = _had(D[1], D[2])
    D123 = _had(D12, D[3])
    D23 = _had(D[2], D[3])

    # 6.2 provisional errors: ebar_i = beta_i (v_i - S_c D_{0:i} k_i)
    Dpre = [D[0], D01, D012, D0123]
    ebar = [[beta[i] * (v[i][r] - x) for r, x in
             enumerate(_mv(S, _had(Dpre[i], k[i])))] for i in range(4)]

    # 6.3 causal substitutions, exactly as printed
    e0 = ebar[0]
    e1 = _axpy(-beta[1] * _dot(k[0], _had(D[1], k[1])), e0, ebar[1])
    e2 = ebar[2]
    e2 = _axpy(-beta[2] * _dot(k[0], _had(D12, k[2])), e0, e2)
    e2 = _axpy(-beta[2] * _dot(k[1], _had(D[2], k[2])), e1, e2)
    e3 = ebar[3]
    e3 = _axpy(-beta[3] * _dot(k[0], _had(D123, k[3])), e0, e3)
    e3 = _axpy(-beta[3] * _dot(k[1], _had(D23, k[3])), e1, e3)
    e3 = _axpy(-beta[3] * _dot(k[2], _had(D[3], k[3])), e2, e3)

    # 6.4 chunk-end state
    S_next = _mcolscale(S, D0123)
    S_next = _madd(S_next, _outer(e0, _had(k[0], D123)))
    S_next = _madd(S_next, _outer(e1, _had(k[1], D23)))
    S_next = _madd(S_next, _outer(e2, _had(k[2], D[3])))
    S_next = _madd(S_next, _outer(e3, _had(k[3], one)))

    # 6.5 outputs, as printed
    def sread(Dx, qi):
        return [s * x for x in _mv(S, _had(Dx, qi))]

    o0 = _axpy(s * _dot(k[0], q[0]), e0, sread(D[0], q[0]))
    o1 = sread(D01, q[1])
    o1 = _axpy(s * _dot(k[0], _had(D[1], q[1])), e0, o1)
    o1 = _axpy(s * _dot(k[1], q[1]), e1, o1)
    o2 = sread(D012, q[2])
    o2 = _axpy(s * _dot(k[0], _had(D12, q[2])), e0, o2)
    o2 = _axpy(s * _dot(k[1], _had(D[2], q[2])), e1, o2)
    o2 = _axpy(s * _dot(k[2], q[2]), e2, o2)
    o3 = sread(D0123, q[3])
    o3 = _axpy(s * _dot(k[0], _had(D123, q[3])), e0, o3)
    o3 = _axpy(s * _dot(k[1], _had(D23, q[3])), e1, o3)
    o3 = _axpy(s * _dot(k[2], _had(D[3], q[3])), e2, o3)
    o3 = _axpy(s * _dot(k[3], q[3]), e3, o3)
    return [o0, o1, o2, o3], S_next
