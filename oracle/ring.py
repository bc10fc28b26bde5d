"""Speculative-decode verify ring and state fold, in fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The "gated_delta" Mojo module page lists a verify kernel that "runs the
gated delta recurrence over a verify window and records a ring instead of
writing the state back", a function giving the elements of one ring record,
and a fold kernel that applies a verify's accepted records to the state pool.
It gives names only; the reading taken here:

  * verify walks each sequence's window of tokens with the recurrence of
    recurrent.py, writes every token's output, leaves the pool untouched, and
    records per (token, value head) what that token's state update consists
    of: S <- S~ + e k^T after the decay S~ = S alpha (or S Diag(alpha)), with
    e = beta (v - S~ k) (delta rule) or e = v (linear rule);
  * a record is [e (DV values), k (DK values), log-gate (1 value for a scalar
    gate, DK for a channel gate, none without a gate)], fp32;
  * fold applies, for each sequence, the records of its first accepted[n]
    window tokens, in order, to its pool slot: S <- S~ + e k^T.

Because each recorded e was computed from the state the earlier window tokens
left, folding the first j records reproduces the recurrence's state after j
tokens exactly; the tests pin that.
"""
from __future__ import annotations

import numpy as np

from .recurrent import round_to_storage

__all__ = ["ring_record_elements", "verify_ring_fp64", "state_fold_fp64"]


def ring_record_elements(DK, DV, gate):
    return DV + DK + {"none": 0, "scalar": 1, "channel": DK}[gate]


def verify_ring_fp64(q, k, v, g, beta, pool, slot_idx, cu_seqlens, *, scale, rule="delta",
                     gate="scalar", zero_init=False):
    """(o [T, HV, DV], ring [T, HV, E]); the pool is read, not written."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, HK, DK = q.shape
    HV, DV = v.shape[1], v.shape[2]
    kh = np.arange(HV) // (HV // HK)
    E = ring_record_elements(DK, DV, gate)
    cu = np.asarray(cu_seqlens, np.int64)
    pool = np.asarray(pool, np.float64)
    o = np.zeros((T, HV, DV))
    ring = np.zeros((T, HV, E))
    for n in range(len(cu) - 1):
        S = np.zeros((HV, DV, DK)) if zero_init else np.swapaxes(pool[slot_idx[n]], -1, -2).copy()
        for t in range(cu[n], cu[n + 1]):
            kt, qt = k[t][kh], q[t][kh]
            if gate == "scalar":
                S = S * np.exp(np.asarray(g[t], np.float64))[:, None, None]
            elif gate == "channel":
                S = S * np.exp(np.asarray(g[t], np.float64))[:, None, :]
            if rule == "linear":
                e = v[t]
            else:
                e = np.asarray(beta[t], np.float64)[:, None] * (v[t] - np.einsum("hvk,hk->hv", S, kt))
            S = S + e[:, :, None] * kt[:, None, :]
            o[t] = float(scale) * np.einsum("hvk,hk->hv", S, qt)
            ring[t, :, :DV] = e
            ring[t, :, DV:DV + DK] = kt
            if gate == "scalar":
                ring[t, :, DV + DK] = g[t]
            elif gate == "channel":
                ring[t, :, DV + DK:] = g[t]
    return o, ring


def state_fold_fp64(pool, ring, slot_idx, cu_seqlens, accepted, *, DK, DV, gate, state_dtype="f32"):
    """The pool after folding each sequence's first accepted[n] records."""
    pool = np.asarray(pool, np.float64)
    ring = np.asarray(ring, np.float64)
    cu = np.asarray(cu_seqlens, np.int64)
    out = pool.copy()
    for n in range(len(cu) - 1):
        S = np.swapaxes(pool[slot_idx[n]], -1, -2).copy()      # [HV, DV, DK]
        for t in range(cu[n], cu[n] + int(accepted[n])):
            e, kt = ring[t, :, :DV], ring[t, :, DV:DV + DK]
            if gate == "scalar":
                S = S * np.exp(ring[t, :, DV + DK])[:, None, None]
            elif gate == "channel":
                S = S * np.exp(ring[t, :, DV + DK:])[:, None, :]
            S = S + e[:, :, None] * kt[:, None, :]
        out[slot_idx[n]] = round_to_storage(np.swapaxes(S, -1, -2), state_dtype)
    return out
