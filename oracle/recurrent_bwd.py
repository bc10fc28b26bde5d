"""Gradients of the gated delta rule (and of the gated linear rule), in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages give the forward recurrence ("You Could Have Come Up With Kimi Delta
Attention", the recurrent form; the "gated_delta" Mojo module page, the state
update; "Linear attention visualized", the gated variants) but no backward
pass for the delta rule. This module is that recurrence differentiated in
reverse mode, one operation at a time. With S value-by-key [DV, DK], per
token t:

    St~ = S_{t-1} * a_t         (a_t = exp(g_t): a scalar, a column scale
                                  exp(g_t)[k] for the channel gate, 1 without)
    u_t = St~ k_t
    e_t = beta_t (v_t - u_t)    (delta rule; e_t = v_t for the linear rule)
    S_t = St~ + e_t k_t^T
    o_t = scale S_t q_t

and for a loss L with upstream gradient do_t = dL/do_t, walking t backwards
with D = dL/dS_t (zero after the last token: the loss reads outputs only):

    D     += scale do_t q_t^T
    dq_t   = scale S_t^T do_t
    de     = D k_t
    dk_t   = D^T e_t
    delta rule:  dv_t = beta_t de,  dbeta_t = de . (v_t - u_t),
                 D~ = D - beta_t de k_t^T,  dk_t -= beta_t St~^T de
    linear rule: dv_t = de,  D~ = D
    dg_t   = sum_j,k D~[j, k] St~[j, k]   (scalar gate; per column k for the
                                           channel gate, summed over j)
    D      = D~ * a_t                       (D is now dL/dS_{t-1})

The gradient of the initial state is what D holds after the first token,
returned transposed like the pool (S^T, [DK, DV]) per sequence. Grouped heads:
a key head's dq and dk sum over the value heads that read it. Readings where
the pages are silent: the final state's gradient is zero, and the in-kernel L2
normalisation is not part of the differentiated function (inputs arrive
normalised, as in recurrent.py).
"""
from __future__ import annotations

import numpy as np

__all__ = ["recurrent_grads_fp64"]


def recurrent_grads_fp64(q, k, v, g, beta, do, pool, slot_idx, cu_seqlens, *, scale,
                         rule="delta", gate="scalar", zero_init=False):
    """Return dict(dq, dk [T, HK, DK], dv [T, HV, DV], dbeta [T, HV] | None,
    dg like g | None, dstate0 [N, HV, DK, DV])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    do = np.asarray(do, np.float64)
    T, HK, DK = q.shape
    HV, DV = v.shape[1], v.shape[2]
    assert k.shape == q.shape and do.shape == v.shape and HV % HK == 0
    assert rule in ("delta", "linear") and gate in ("none", "scalar", "channel")
    G = HV // HK
    cu = np.asarray(cu_seqlens, np.int64)
    N = len(cu) - 1
    pool = np.asarray(pool, np.float64)
    s = float(scale)
    if gate != "none":
        g = np.asarray(g, np.float64)
    if rule == "delta":
        beta = np.asarray(beta, np.float64)

    dq = np.zeros((T, HK, DK))
    dk = np.zeros((T, HK, DK))
    dv = np.zeros((T, HV, DV))
    dbeta = np.zeros((T, HV)) if rule == "delta" else None
    dg = np.zeros_like(g) if gate != "none" else None
    dstate0 = np.zeros((N, HV, DK, DV))

    for n in range(N):
        a, b = int(cu[n]), int(cu[n + 1])
        for h in range(HV):
            hk = h // G
            # forward, keeping what the backward reads
            S = np.zeros((DV, DK)) if zero_init else pool[slot_idx[n], h].T.copy()
            St_, Ss, es, us = [], [], [], []
            for t in range(a, b):
                kt = k[t, hk]
                if gate == "scalar":
                    S = S * np.exp(g[t, h])
                elif gate == "channel":
                    S = S * np.exp(g[t, h])[None, :]
                u = S @ kt
                e = v[t, h] if rule == "linear" else beta[t, h] * (v[t, h] - u)
                St_.append(S)
                us.append(u)
                es.append(e)
                S = S + np.outer(e, kt)
                Ss.append(S)
            # reverse
            D = np.zeros((DV, DK))
            for i in range(b - a - 1, -1, -1):
                t = a + i
                qt, kt = q[t, hk], k[t, hk]
                D = D + s * np.outer(do[t, h], qt)
                dq[t, hk] += s * (Ss[i].T @ do[t, h])
                de = D @ kt
                dk[t, hk] += D.T @ es[i]
                if rule == "delta":
                    dv[t, h] = beta[t, h] * de
                    dbeta[t, h] = de @ (v[t, h] - us[i])
                    du = -beta[t, h] * de
                    dk[t, hk] += St_[i].T @ du
                    D = D + np.outer(du, kt)
                else:
                    dv[t, h] = de
                if gate == "scalar":
                    dg[t, h] = np.sum(D * St_[i])
                    D = D * np.exp(g[t, h])
                elif gate == "channel":
                    dg[t, h] = np.sum(D * St_[i], axis=0)
                    D = D * np.exp(g[t, h])[None, :]
            dstate0[n, h] = D.T
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, dg=dg, dstate0=dstate0)
