"""Gradients of causal linear attention, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"From Attention to Learned Memory", section "Backward: reverse the boundary
scan, then differentiate each chunk", differentiates the plain linear rule
(no gate, no delta): per token o_t = scale * S_t q_t with
S_t = S_0 + sum_{tau <= t} v_tau k_tau^T (value-by-key). For a loss with
upstream gradient dO (dL/do_t = do_t), written out from that definition:

    dq_t   = scale * ( S_0^T do_t + sum_{tau <= t} (do_t . v_tau) k_tau )
    dk_tau = scale * sum_{t >= tau} (do_t . v_tau) q_t
    dv_tau = scale * sum_{t >= tau} (q_t . k_tau) do_t

The page's chunked form (the boundary-state gradient G scanned from the last
chunk back, then per-chunk products with the masked score matrices) regroups
these sums; this module evaluates the sums directly, per sequence, as masked
T x T products. Readings where the page is silent: the gradient reaching the
final state is zero (the loss reads the outputs only) and the initial state's
own gradient is not formed.
"""
from __future__ import annotations

import numpy as np

__all__ = ["linear_attention_grads_fp64"]


def linear_attention_grads_fp64(q, k, v, do, pool, slot_idx, cu_seqlens, *, scale,
                                zero_init=False):
    """(dq, dk, dv) for a ragged batch; q, k [T, H, DK], v, do [T, H, DV]
    (one value head per key head), pool [slots, H, DK, DV] holding S_0^T."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    T, H, DK = q.shape
    DV = v.shape[2]
    assert k.shape == q.shape and v.shape == (T, H, DV) and do.shape == v.shape
    cu = np.asarray(cu_seqlens, np.int64)
    pool = np.asarray(pool, np.float64)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    s = float(scale)
    for n in range(len(cu) - 1):
        a, b = int(cu[n]), int(cu[n + 1])
        if a == b:
            continue
        L = b - a
        mask = np.tril(np.ones((L, L)))          # [t, tau]: tau <= t
        for h in range(H):
            Q, K, V, dO = q[a:b, h], k[a:b, h], v[a:b, h], do[a:b, h]
            E = (dO @ V.T) * mask                # do_t . v_tau
            A = (Q @ K.T) * mask                 # q_t . k_tau
            dq[a:b, h] = s * (E @ K)
            if not zero_init:
                S0T = pool[slot_idx[n], h]       # S_0^T [DK, DV]
                dq[a:b, h] += s * (dO @ S0T.T)   # rows (S_0^T do_t)
            dk[a:b, h] = s * (E.T @ Q)
            dv[a:b, h] = s * (A.T @ dO)
    return dq, dk, dv
