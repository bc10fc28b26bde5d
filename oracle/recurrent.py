"""Tokenwise fp64 recurrence: the definition of the method.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The update for one value head, state S in R^{d_v x d_k} (value-by-key), follows
the boxed KDA equations of "You Could Have Come Up With Kimi Delta Attention"
(opening display and section 4) and the five steps of the "gated_delta" Mojo
module page (section "The five steps of the gated delta rule"):

    S~ = S * alpha            (scalar gate)  |  S Diag(alpha)  (channel gate)
    vhat = S~ k
    e    = beta (v - vhat)
    S    = S~ + e k^T
    o    = S (scale * q)      -- read after the write

with alpha = exp(g), g = log alpha <= 0 stored per token (section 4 of the KDA
page: implementations keep g and exponentiate it). The linear rule is the
additive write of "From Attention to Learned Memory" section 1 (S += v k^T),
optionally decayed first by the same gate (the RetNet / Mamba-2 / GLA rows of
"Linear attention visualized").

Readings of points the pages leave open:
  * decay happens before the prediction, the read happens after the write
    (KDA page section 3: the order matters);
  * the pool stores S^T as [slot, head, d_k, d_v] (KDA page section 4 speaks of
    the transposed d_k x d_v layout; the Mojo page indexes
    state[slot, head, k, vd]); slots not named by slot_idx are left untouched;
  * key head of value head h is h // (HV // HK) (Mojo page, GQA paragraph);
  * scale is an argument; callers default it to d_k^-1/2 (KDA page section 1);
  * no L2 normalisation is applied: inputs arrive normalised.
"""
from __future__ import annotations

import numpy as np

__all__ = ["recurrent_fp64", "round_to_storage", "round_f64_to_bf16", "l2_normalise_fp64",
           "L2_EPS"]

# Guard of the L2 normalisation (see l2_normalise_fp64).
L2_EPS = 1e-6


def round_f64_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float64 values to the nearest bfloat16, ties to even.

    bfloat16 keeps fp32's 8-bit exponent and 7 explicit mantissa bits, so a
    finite x with |x| in [2^e, 2^(e+1)) is a multiple of 2^(e-7); below the
    smallest normal (2^-126) the spacing stays 2^-133. ``np.rint`` rounds half
    to even. Values beyond the largest finite bf16 become +-inf.
    Direct fp64 -> bf16 rounding (no intermediate fp32 step).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = (x != 0) & np.isfinite(x)
    _, e = np.frexp(x[nz])                 # |x| = m 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, -126)            # floor(log2|x|), clamped at min normal
    quantum = np.ldexp(1.0, e - 7)
    out[nz] = np.rint(x[nz] / quantum) * quantum
    big = np.abs(out) > 3.3895313892515355e38   # largest finite bf16
    out[big] = np.copysign(np.inf, out[big])
    out[~nz] = x[~nz]
    return out


def round_to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    """Value of fp64 ``x`` once stored in ``dtype`` ("f32" | "bf16" | "f64")."""
    if dtype == "f64":
        return np.asarray(x, dtype=np.float64).copy()
    if dtype == "f32":
        return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    if dtype == "bf16":
        return round_f64_to_bf16(x)
    raise ValueError(dtype)


def recurrent_fp64(q, k, v, g, beta, pool, slot_idx, cu_seqlens, *, scale,
                   rule="delta", gate="scalar", zero_init=False,
                   state_dtype="f32"):
    """Run the recurrence over a ragged batch; return (o, pool_out).

    Arguments (all already widened to float64 where they are real-valued):
      q, k       [T, HK, DK]
      v          [T, HV, DV]
      g          [T, HV] (scalar gate) | [T, HV, DK] (channel gate) | None
      beta       [T, HV] | None (linear rule)
      pool       [num_slots, HV, DK, DV]: S^T per slot and value head
      slot_idx   [N] distinct slot per sequence
      cu_seqlens [N+1] token offsets; sequence n is tokens cu[n]..cu[n+1]-1
    Returns o [T, HV, DV] float64 and a new pool array whose touched slots hold
    the final state rounded (nearest even) to ``state_dtype``.

    Vectorised across (sequence, head) pairs only: all sequences advance one
    local token per iteration, finished sequences are masked out.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    T, HK, DK = q.shape
    HV, DV = v.shape[1], v.shape[2]
    assert k.shape == (T, HK, DK) and v.shape[0] == T
    assert HV % HK == 0
    assert rule in ("delta", "linear") and gate in ("none", "scalar", "channel")
    if rule == "delta":
        assert beta is not None and beta.shape == (T, HV)
    if gate == "scalar":
        assert g is not None and g.shape == (T, HV)
    elif gate == "channel":
        assert g is not None and g.shape == (T, HV, DK)
    cu = np.asarray(cu_seqlens, np.int64)
    slot_idx = np.asarray(slot_idx, np.int64)
    N = len(cu) - 1
    assert len(slot_idx) == N and cu[0] == 0 and cu[-1] == T
    assert np.all(np.diff(cu) >= 0)
    assert len(np.unique(slot_idx)) == N
    pool = np.asarray(pool, np.float64)
    kh = np.arange(HV) // (HV // HK)          # key head of each value head

    # S[n, h] in value-by-key orientation
    if zero_init:
        S = np.zeros((N, HV, DV, DK))
    else:
        S = np.swapaxes(pool[slot_idx], -1, -2).copy()
    o = np.zeros((T, HV, DV))
    lens = np.diff(cu)
    for t in range(int(lens.max()) if N else 0):
        act = np.nonzero(lens > t)[0]
        idx = cu[act] + t
        qt = q[idx][:, kh]                    # [Na, HV, DK]
        kt = k[idx][:, kh]
        vt = v[idx]                           # [Na, HV, DV]
        St = S[act]
        if gate == "scalar":
            St = St * np.exp(np.asarray(g[idx], np.float64))[:, :, None, None]
        elif gate == "channel":
            St = St * np.exp(np.asarray(g[idx], np.float64))[:, :, None, :]
        if rule == "linear":
            St = St + vt[..., :, None] * kt[..., None, :]
        else:
            vhat = np.matmul(St, kt[..., None])[..., 0]
            e = np.asarray(beta[idx], np.float64)[..., None] * (vt - vhat)
            St = St + e[..., :, None] * kt[..., None, :]
        o[idx] = float(scale) * np.matmul(St, qt[..., None])[..., 0]
        S[act] = St

    pool_out = pool.copy()
    for n in range(N):
        pool_out[slot_idx[n]] = round_to_storage(np.swapaxes(S[n], -1, -2), state_dtype)
    return o, pool_out


def l2_normalise_fp64(x: np.ndarray, eps: float = L2_EPS) -> np.ndarray:
    """x / sqrt(sum_k x_k^2 + eps) over the last axis, in fp64.

    The "gated_delta" Mojo page (its kernel steps 2, 4 and 5) reads the state
    with L2-normalised keys and queries, and "From Attention to Learned
    Memory" (the paragraph after the causal read) notes that models apply SiLU
    and then L2 normalisation to q and k ahead of the recurrence, leaving the
    state algebra unchanged. The pages give no guard for a zero vector; the
    reading taken here adds eps = 1e-6 to the squared norm, so a zero vector
    stays zero and any other vector comes out with norm
    sqrt(|x|^2 / (|x|^2 + eps)).
    """
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.sum(x * x, axis=-1, keepdims=True) + eps)
