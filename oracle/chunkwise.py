"""Independent fp64 chunkwise form of the gated delta rule.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Written from section 6 of "You Could Have Come Up With Kimi Delta Attention"
(chunked KDA: provisional errors, the causal key-key coefficients rho, the
unit lower triangular system, the chunk-end state and the causal outputs) and
section 4 of "From Attention to Learned Memory" (the triangular system of the
WY/UT representation, solved by forward substitution). The linear rule uses
section 2's chunk equation (Eq. 4) of the same page.

Per chunk of C tokens with incoming state S_c (d_v x d_k) and the inclusive
in-chunk cumulative log-decay G_i (one value per key channel; a scalar gate is
broadcast over channels), D_{j+1:i} = exp(G_i - G_j) and D_{0:i} = exp(G_i):

    ebar_i  = beta_i (v_i - S_c D_{0:i} k_i)                 provisional errors
    rho_ij  = beta_i <k_j| D_{j+1:i} |k_i>          (j < i)  key-key coefficients
    e_i     = ebar_i - sum_{j<i} rho_ij e_j                   forward substitution
    S_{c+1} = S_c D_{0:C-1} + sum_j e_j (D_{j+1:C-1} k_j)^T   chunk-end state
    chi_ij  = s <k_j| D_{j+1:i} |q_i>               (j <= i)  query-key coefficients
    o_i     = s S_c D_{0:i} q_i + sum_{j<=i} chi_ij e_j       causal outputs

A chunk never spans two sequences; the last chunk of a sequence may be short.
Nothing here is blocked, fused or reordered beyond these equations.
"""
from __future__ import annotations

import numpy as np

from .recurrent import round_to_storage

__all__ = ["chunkwise_fp64", "forward_substitution_unit_lower"]


def forward_substitution_unit_lower(L: np.ndarray, B: np.ndarray) -> np.ndarray:
    """Solve (I + L) X = B for strictly lower triangular L, row by row.

    Row i only needs the rows before it ("From Attention to Learned Memory",
    section 4: the unit lower triangular system is solved from its first row
    to its last).
    """
    C = L.shape[0]
    X = np.zeros_like(B, dtype=np.float64)
    for i in range(C):
        X[i] = B[i] - L[i, :i] @ X[:i]
    return X


def _chunk_delta(S, q, k, v, G, beta, scale):
    """One chunk of the delta rule; returns (outputs [C, d_v], S_next)."""
    C = q.shape[0]
    Dq = np.exp(G)                                   # D_{0:i} per channel [C, d_k]
    ebar = beta[:, None] * (v - (S @ (Dq * k).T).T)  # [C, d_v]
    rho = np.zeros((C, C))
    chi = np.zeros((C, C))
    for i in range(C):
        for j in range(i + 1):
            dij = np.exp(G[i] - G[j])                # D_{j+1:i}
            if j < i:
                rho[i, j] = beta[i] * np.sum(k[j] * dij * k[i])
            chi[i, j] = scale * np.sum(k[j] * dij * q[i])
    e = forward_substitution_unit_lower(rho, ebar)
    kend = np.exp(G[-1][None, :] - G) * k            # D_{j+1:C-1} k_j
    S_next = S * np.exp(G[-1])[None, :] + e.T @ kend
    o = scale * (S @ (Dq * q).T).T + chi @ e
    return o, S_next


def _chunk_linear(S, q, k, v, G, scale):
    """One chunk of (optionally decayed) linear attention; Eq. (4) of section 2
    of "From Attention to Learned Memory" with the decayed scores of the
    Mamba-2 / GLA chunkwise forms of "Linear attention visualized"."""
    C = q.shape[0]
    Dq = np.exp(G)
    score = np.zeros((C, C))
    for i in range(C):
        for j in range(i + 1):
            score[i, j] = np.sum(q[i] * np.exp(G[i] - G[j]) * k[j])
    o = scale * ((S @ (Dq * q).T).T + score @ v)
    kend = np.exp(G[-1][None, :] - G) * k
    S_next = S * np.exp(G[-1])[None, :] + v.T @ kend
    return o, S_next


def chunkwise_fp64(q, k, v, g, beta, pool, slot_idx, cu_seqlens, *, scale,
                   chunk_size, rule="delta", gate="scalar", zero_init=False,
                   state_dtype="f32"):
    """Same contract as ``recurrent_fp64`` but evaluated chunk by chunk."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, HK, DK = q.shape
    HV = v.shape[1]
    cu = np.asarray(cu_seqlens, np.int64)
    N = len(cu) - 1
    pool = np.asarray(pool, np.float64)
    pool_out = pool.copy()
    o = np.zeros((T, HV, v.shape[2]))
    ratio = HV // HK
    for n in range(N):
        for h in range(HV):
            hk = h // ratio
            S = (np.zeros((v.shape[2], DK)) if zero_init
                 else pool[slot_idx[n], h].T.copy())
            for a in range(cu[n], cu[n + 1], chunk_size):
                b = min(a + chunk_size, cu[n + 1])
                if gate == "none":
                    G = np.zeros((b - a, DK))
                elif gate == "scalar":
                    G = np.repeat(np.cumsum(np.asarray(g[a:b, h], np.float64))[:, None], DK, 1)
                else:
                    G = np.cumsum(np.asarray(g[a:b, h], np.float64), axis=0)
                if rule == "delta":
                    oc, S = _chunk_delta(S, q[a:b, hk], k[a:b, hk], v[a:b, h], G,
                                         np.asarray(beta[a:b, h], np.float64), scale)
                else:
                    oc, S = _chunk_linear(S, q[a:b, hk], k[a:b, hk], v[a:b, h], G, scale)
                o[a:b, h] = oc
            pool_out[slot_idx[n], h] = round_to_storage(S.T, state_dtype)
    return o, pool_out
