"""Gated DeltaProduct: n_h transitions per token, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

"Linear attention visualized", section "Gated Delta Product (GDP)": each real
token t carries n_h substeps, each with its own key k_{t,j}, value v_{t,j}
and correction gate beta_{t,j}. The token's decay a_t is applied once, before
the first substep; the substeps then apply the delta-rule write in order,
each predicting from the state the previous substep left; the query reads the
state only after the last substep:

    S~ = S * a_t   (scalar gate)  |  S Diag(a_t)  (channel gate)
    for j = 1 .. n_h:   S~ = S~ + beta_{t,j} (v_{t,j} - S~ k_{t,j}) k_{t,j}^T
    S = S~;   o_t = S (scale * q_t)

With the linear rule each substep adds v_{t,j} k_{t,j}^T instead.

Layouts: the substeps of token t are consecutive rows t * n_h + j of k, v and
beta (the page's flattening of (t, j) into virtual steps); q, g and o keep one
row per real token. cu_seqlens counts real tokens.

Reading where the page is silent: the page states GDP with a scalar decay; the
channel gate (KDA's diagonal decay) and the linear rule are accepted with the
same placement (decay before the first substep), which is what running the
virtual sequence through those variants gives.
"""
from __future__ import annotations

import numpy as np

from .recurrent import round_to_storage

__all__ = ["delta_product_fp64"]


def delta_product_fp64(q, k, v, g, beta, pool, slot_idx, cu_seqlens, *, products, scale,
                       rule="delta", gate="scalar", zero_init=False, state_dtype="f32"):
    """Run Gated DeltaProduct over a ragged batch; return (o, pool_out).

    Arguments (real-valued ones already widened to float64):
      q          [T, HK, DK]            one row per real token
      k          [T * n_h, HK, DK]      substep j of token t at row t * n_h + j
      v          [T * n_h, HV, DV]
      g          [T, HV] | [T, HV, DK] | None
      beta       [T * n_h, HV] | None (linear rule)
      pool       [num_slots, HV, DK, DV]: S^T per slot and value head
      slot_idx   [N], cu_seqlens [N+1] in real tokens
    Returns o [T, HV, DV] and the pool with the touched slots rounded to
    ``state_dtype``. Loops over sequences and real tokens; heads are
    vectorised.
    """
    P = int(products)
    assert P >= 1
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, HK, DK = q.shape
    HV, DV = v.shape[1], v.shape[2]
    assert k.shape == (T * P, HK, DK) and v.shape[0] == T * P
    assert HV % HK == 0
    assert rule in ("delta", "linear") and gate in ("none", "scalar", "channel")
    if rule == "delta":
        assert beta is not None and np.shape(beta) == (T * P, HV)
    if gate == "scalar":
        assert g is not None and np.shape(g) == (T, HV)
    elif gate == "channel":
        assert g is not None and np.shape(g) == (T, HV, DK)
    cu = np.asarray(cu_seqlens, np.int64)
    slot_idx = np.asarray(slot_idx, np.int64)
    N = len(cu) - 1
    assert len(slot_idx) == N and cu[0] == 0 and cu[-1] == T
    assert len(np.unique(slot_idx)) == N
    pool = np.asarray(pool, np.float64)
    kh = np.arange(HV) // (HV // HK)          # key head of each value head

    o = np.zeros((T, HV, DV))
    pool_out = pool.copy()
    for n in range(N):
        # S[h] in value-by-key orientation
        S = np.zeros((HV, DV, DK)) if zero_init else np.swapaxes(pool[slot_idx[n]], -1, -2).copy()
        for t in range(cu[n], cu[n + 1]):
            if gate == "scalar":
                S = S * np.exp(np.asarray(g[t], np.float64))[:, None, None]
            elif gate == "channel":
                S = S * np.exp(np.asarray(g[t], np.float64))[:, None, :]
            for j in range(P):
                m = t * P + j
                kj = k[m][kh]                  # [HV, DK]
                vj = v[m]                      # [HV, DV]
                if rule == "linear":
                    w = vj
                else:
                    pred = np.einsum("hvk,hk->hv", S, kj)
                    w = np.asarray(beta[m], np.float64)[:, None] * (vj - pred)
                S = S + w[:, :, None] * kj[:, None, :]
            o[t] = float(scale) * np.einsum("hvk,hk->hv", S, q[t][kh])
        pool_out[slot_idx[n]] = round_to_storage(np.swapaxes(S, -1, -2), state_dtype)
    return o, pool_out
