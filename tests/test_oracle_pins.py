"""Pins of the fp64 oracle against facts the pages and the mathematics fix.

Every test here runs on the CPU. Each is chosen so that a plausible slip in
the oracle (a dropped term, a wrong sign, a decay applied after the
prediction, a transposed state, a read before the write) fails at least one.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle import (recurrent_fp64, chunkwise_fp64, linear_parallel_fp64,
                    delta_parallel_fp64, four_token_chunk_fractions,
                    forward_substitution_unit_lower, round_f64_to_bf16)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def unit(x, axis=-1):
    return x / np.linalg.norm(x, axis=axis, keepdims=True)


def tiny(rng, T=7, HK=1, HV=1, DK=5, DV=4, gate="scalar", S0=True):
    q = unit(rng.standard_normal((T, HK, DK)))
    k = unit(rng.standard_normal((T, HK, DK)))
    v = rng.standard_normal((T, HV, DV))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, HV))))
    if gate == "channel":
        g = -np.log1p(np.exp(-(rng.standard_normal((T, HV, DK)) - 1.0)))
    else:
        g = -np.log1p(np.exp(-(rng.standard_normal((T, HV)) - 1.0)))
    pool = rng.standard_normal((2, HV, DK, DV)) * (0.5 if S0 else 0.0)
    return q, k, v, g, beta, pool


def run(q, k, v, g, beta, pool, *, slot=0, scale=1.0, rule="delta",
        gate="scalar", zero_init=False, cu=None):
    T = q.shape[0]
    cu = np.array([0, T]) if cu is None else np.asarray(cu)
    slots = np.arange(len(cu) - 1) if cu is not None and len(cu) > 2 else np.array([slot])
    return recurrent_fp64(q, k, v, g, beta, pool, slots, cu, scale=scale,
                          rule=rule, gate=gate, zero_init=zero_init,
                          state_dtype="f64")


def state(pool, slot=0, h=0):
    """Value-by-key state of one slot and head."""
    return pool[slot, h].T


# ---------------------------------------------------------------------------
# delta write (KDA page 2.1; From Attention to Learned Memory section 3)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gate", ["none", "scalar"])
def test_beta_one_writes_exactly(gate):
    """beta = 1, alpha = 1, unit k: the post-write read at k_t returns v_t."""
    rng = np.random.default_rng(1)
    q, k, v, g, beta, pool = tiny(rng, T=9)
    g = np.zeros_like(g)
    beta = np.ones_like(beta)
    o, _ = run(k.copy(), k, v, g, beta, pool, gate=gate, scale=1.0)
    np.testing.assert_allclose(o, v, atol=1e-12)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_read_back_interpolates(gate):
    """S_t k_t = (1 - beta) S~_t k_t + beta v_t with S~_t the decayed state."""
    rng = np.random.default_rng(2)
    q, k, v, g, beta, pool = tiny(rng, T=6, gate=gate)
    for t in range(6):
        _, p_prev = run(q[:t], k[:t], v[:t], g[:t], beta[:t], pool, gate=gate)
        S_prev = state(p_prev)
        a = np.exp(g[t, 0])
        S_dec = S_prev * a if gate == "scalar" else S_prev * a[None, :]
        o, _ = run(k[:t + 1], k[:t + 1], v[:t + 1], g[:t + 1], beta[:t + 1], pool,
                   gate=gate, scale=1.0)
        expect = (1 - beta[t, 0]) * S_dec @ k[t, 0] + beta[t, 0] * v[t, 0]
        np.testing.assert_allclose(o[t, 0], expect, atol=1e-12)


def test_write_leaves_orthogonal_directions():
    """(S_t - S~_t) x = 0 for every x orthogonal to k_t (KDA page 2.1)."""
    rng = np.random.default_rng(3)
    q, k, v, g, beta, pool = tiny(rng, T=1, DK=6)
    _, p1 = run(q, k, v, g, beta, pool)
    S0 = state(pool)
    S_dec = S0 * np.exp(g[0, 0])
    kk = k[0, 0]
    for _ in range(4):
        x = rng.standard_normal(6)
        x -= kk * (kk @ x)
        np.testing.assert_allclose((state(p1) - S_dec) @ x, 0, atol=1e-12)
    # and the change along k is not zero (the write happened)
    assert np.linalg.norm((state(p1) - S_dec) @ kk) > 1e-3


def test_transition_spectrum():
    """With v = 0, alpha = 1 the transition I - beta k k^T has eigenvalue
    1 - beta along k and 1 on the orthogonal complement (KDA page 2.3)."""
    rng = np.random.default_rng(4)
    q, k, v, g, beta, pool = tiny(rng, T=1, DK=6)
    v = np.zeros_like(v)
    g = np.zeros_like(g)
    _, p1 = run(q, k, v, g, beta, pool)
    S0, S1 = state(pool), state(p1)
    kk = k[0, 0]
    np.testing.assert_allclose(S1 @ kk, (1 - beta[0, 0]) * (S0 @ kk), atol=1e-12)
    x = rng.standard_normal(6)
    x -= kk * (kk @ x)
    np.testing.assert_allclose(S1 @ x, S0 @ x, atol=1e-12)


def test_gradient_step_identity():
    """S_t = S~_t - beta grad(1/2 ||S k - v||^2)(S~_t) (KDA page 2.2); the
    gradient is taken by central differences, independent of the update."""
    rng = np.random.default_rng(5)
    q, k, v, g, beta, pool = tiny(rng, T=1, DK=4, DV=3)
    _, p1 = run(q, k, v, g, beta, pool)
    S_dec = state(pool) * np.exp(g[0, 0])
    kk, vv = k[0, 0], v[0, 0]

    def loss(S):
        r = S @ kk - vv
        return 0.5 * float(r @ r)

    grad = np.zeros_like(S_dec)
    h = 1e-3
    for i in range(S_dec.shape[0]):
        for j in range(S_dec.shape[1]):
            E = np.zeros_like(S_dec)
            E[i, j] = h
            grad[i, j] = (loss(S_dec + E) - loss(S_dec - E)) / (2 * h)
    np.testing.assert_allclose(state(p1), S_dec - beta[0, 0] * grad, atol=1e-9)


def test_single_token_from_zero_state():
    """From S0 = 0 one token gives S = beta v k^T and o = s beta (k.q) v."""
    rng = np.random.default_rng(6)
    q, k, v, g, beta, pool = tiny(rng, T=1, S0=False)
    s = 0.37
    o, p1 = run(q, k, v, g, beta, pool, scale=s)
    b = beta[0, 0]
    np.testing.assert_allclose(state(p1), b * np.outer(v[0, 0], k[0, 0]), atol=1e-14)
    np.testing.assert_allclose(o[0, 0], s * b * (k[0, 0] @ q[0, 0]) * v[0, 0], atol=1e-14)


# ---------------------------------------------------------------------------
# gate: placement, orientation, scalar vs channel (KDA page 3-4; Mojo page)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_decay_only_closed_form(gate):
    """With k = 0 nothing is written: S_t = S0 Diag(prod alpha) and the read is
    s S_t q_t. The channel gate scales key channels, i.e. columns of S."""
    rng = np.random.default_rng(7)
    q, k, v, g, beta, pool = tiny(rng, T=5, DK=5, DV=3, gate=gate)
    k = np.zeros_like(k)
    s = 0.8
    o, p = run(q, k, v, g, beta, pool, gate=gate, scale=s)
    S0 = state(pool)
    G = np.cumsum(g[:, 0], axis=0)
    for t in range(5):
        d = np.exp(G[t]) * np.ones(5)
        np.testing.assert_allclose(o[t, 0], s * (S0 * d[None, :]) @ q[t, 0], atol=1e-13)
    d = np.exp(G[-1]) * np.ones(5)
    np.testing.assert_allclose(state(p), S0 * d[None, :], atol=1e-14)


def test_pool_orientation_rectangular():
    """The pool stores S^T as [slot, head, d_k, d_v]: with no writes and no
    decay the read is s * pool[slot].T @ q (DK != DV catches a transpose)."""
    rng = np.random.default_rng(8)
    DK, DV = 3, 2
    q = rng.standard_normal((2, 1, DK))
    k = np.zeros((2, 1, DK))
    v = rng.standard_normal((2, 1, DV))
    pool = rng.standard_normal((3, 1, DK, DV))
    o, p = recurrent_fp64(q, k, v, None, np.full((2, 1), 0.5), pool, [2], [0, 2],
                          scale=1.5, gate="none", state_dtype="f64")
    for t in range(2):
        np.testing.assert_allclose(o[t, 0], 1.5 * pool[2, 0].T @ q[t, 0], atol=1e-14)
    np.testing.assert_array_equal(p, pool)


def test_channel_gate_constant_vector_equals_scalar_gate():
    """KDA with alpha_t = a_t 1 reduces exactly to GDN (Linear attention
    visualized, KDA section)."""
    rng = np.random.default_rng(9)
    q, k, v, g, beta, pool = tiny(rng, T=11, HK=1, HV=2)
    gc = np.repeat(g[:, :, None], q.shape[-1], axis=2)
    o1, p1 = run(q, k, v, g, beta, pool, gate="scalar")
    o2, p2 = run(q, k, v, gc, beta, pool, gate="channel")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1, p2)


def test_decay_precedes_prediction():
    """Gated DeltaNet forgets before it predicts (KDA page section 3): the
    one-step state from S0 equals a S0 (I - beta k k^T) + beta v k^T, not the
    other order (which would give a (S0 + beta (v - S0 k) k^T))."""
    rng = np.random.default_rng(10)
    q, k, v, g, beta, pool = tiny(rng, T=1)
    _, p1 = run(q, k, v, g, beta, pool)
    a, b, kk, vv = np.exp(g[0, 0]), beta[0, 0], k[0, 0], v[0, 0]
    S0 = state(pool)
    right = a * S0 @ (np.eye(len(kk)) - b * np.outer(kk, kk)) + b * np.outer(vv, kk)
    wrong = a * (S0 + b * np.outer(vv - S0 @ kk, kk))
    np.testing.assert_allclose(state(p1), right, atol=1e-14)
    assert np.abs(state(p1) - wrong).max() > 1e-3


# ---------------------------------------------------------------------------
# independent statements of the same outputs
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
def test_linear_rule_equals_masked_parallel_form(gate):
    """LINEAR mode = s (Q K^T (.) Gamma) V + decayed read of S0, brute force."""
    rng = np.random.default_rng(11)
    q, k, v, g, beta, pool = tiny(rng, T=9, DK=4, DV=3, gate=gate)
    s = 0.6
    o, p = run(q, k, v, g if gate != "none" else None, None, pool, rule="linear",
               gate=gate, scale=s)
    alpha = None if gate == "none" else np.exp(g[:, 0])
    ob, ST = linear_parallel_fp64(q[:, 0], k[:, 0], v[:, 0], s, alpha, state(pool))
    np.testing.assert_allclose(o[:, 0], ob, atol=1e-13)
    np.testing.assert_allclose(state(p), ST, atol=1e-13)


def test_delta_rule_equals_full_sequence_solve():
    """Ungated DeltaNet from zero = the full-sequence triangular correction
    system of Linear attention visualized, solved row by row."""
    rng = np.random.default_rng(12)
    q, k, v, g, beta, pool = tiny(rng, T=10, DK=4, DV=3, S0=False)
    o, p = run(q, k, v, None, beta, pool, gate="none", scale=0.7, zero_init=True)
    ob, ST = delta_parallel_fp64(q[:, 0], k[:, 0], v[:, 0], beta[:, 0], 0.7)
    np.testing.assert_allclose(o[:, 0], ob, atol=1e-13)
    np.testing.assert_allclose(state(p), ST, atol=1e-13)


def _rand_frac(rng, lo, hi, den=8):
    return Fraction(int(rng.integers(lo * den, hi * den + 1)), den)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_four_token_chunk_term_by_term(gate):
    """The recurrence reproduces section 6 of the KDA page (provisional errors,
    rho substitutions, chunk-end state, outputs) in exact arithmetic."""
    rng = np.random.default_rng(13)
    DK, DV = 3, 2
    S = [[_rand_frac(rng, -2, 2) for _ in range(DK)] for _ in range(DV)]
    if gate == "scalar":
        alpha = [[a] * DK for a in (_rand_frac(rng, 0.25, 1, 8) for _ in range(4))]
    else:
        alpha = [[_rand_frac(rng, 0.25, 1, 8) for _ in range(DK)] for _ in range(4)]
    beta = [_rand_frac(rng, 0.125, 1, 8) for _ in range(4)]
    k = [[_rand_frac(rng, -1, 1, 4) for _ in range(DK)] for _ in range(4)]
    v = [[_rand_frac(rng, -2, 2, 4) for _ in range(DV)] for _ in range(4)]
    q = [[_rand_frac(rng, -1, 1, 4) for _ in range(DK)] for _ in range(4)]
    s = Fraction(1, 2)
    o_ex, S_ex = four_token_chunk_fractions(S, alpha, beta, k, v, q, s)

    f = lambda x: np.array(x, dtype=np.float64)
    qa, ka = f(q)[:, None], f(k)[:, None]
    va = f(v)[:, None]
    ga = np.log(f(alpha))
    ga = ga[:, None, 0] if gate == "scalar" else ga[:, None, :]
    pool = f(S).T[None, None]
    o, p = recurrent_fp64(qa, ka, va, ga, f(beta)[:, None], pool, [0], [0, 4],
                          scale=0.5, gate=gate, state_dtype="f64")
    np.testing.assert_allclose(o[:, 0], f(o_ex), atol=1e-12)
    np.testing.assert_allclose(p[0, 0].T, f(S_ex), atol=1e-12)


# ---------------------------------------------------------------------------
# chunkwise regrouping (KDA page section 6; From Attention to Learned Memory 4)
# ---------------------------------------------------------------------------

def ragged_problem(rng, lens, HK, HV, DK, DV, gate, slots=6):
    T = int(sum(lens))
    q = unit(rng.standard_normal((T, HK, DK)))
    k = unit(rng.standard_normal((T, HK, DK)))
    v = rng.standard_normal((T, HV, DV))
    beta = 1 / (1 + np.exp(-rng.standard_normal((T, HV))))
    if gate == "channel":
        g = -np.log1p(np.exp(-(rng.standard_normal((T, HV, DK)) - 2.0)))
    elif gate == "scalar":
        g = -np.log1p(np.exp(-(rng.standard_normal((T, HV)) - 2.0)))
    else:
        g = None
    pool = 0.3 * rng.standard_normal((slots, HV, DK, DV))
    cu = np.concatenate([[0], np.cumsum(lens)])
    slot_idx = rng.choice(slots, size=len(lens), replace=False)
    return q, k, v, g, beta, pool, slot_idx, cu


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("rule", ["delta", "linear"])
@pytest.mark.parametrize("C", [1, 3, 16, 32, 64])
def test_chunkwise_equals_recurrence(gate, rule, C):
    rng = np.random.default_rng(14)
    lens = [70, 0, 33, 129]
    q, k, v, g, beta, pool, slot_idx, cu = ragged_problem(rng, lens, 2, 4, 6, 5, gate)
    b = beta if rule == "delta" else None
    o1, p1 = recurrent_fp64(q, k, v, g, b, pool, slot_idx, cu, scale=0.4,
                            rule=rule, gate=gate, state_dtype="f64")
    o2, p2 = chunkwise_fp64(q, k, v, g, b, pool, slot_idx, cu, scale=0.4,
                            chunk_size=C, rule=rule, gate=gate, state_dtype="f64")
    np.testing.assert_allclose(o2, o1, atol=1e-12, rtol=0)
    np.testing.assert_allclose(p2, p1, atol=1e-12, rtol=0)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_single_chunk_is_the_parallel_form(gate):
    """C = T: one chunk holds the whole sequence (the fully parallel form)."""
    rng = np.random.default_rng(15)
    q, k, v, g, beta, pool, slot_idx, cu = ragged_problem(rng, [90], 1, 1, 5, 4, gate)
    o1, p1 = recurrent_fp64(q, k, v, g, beta, pool, slot_idx, cu, scale=0.3,
                            gate=gate, state_dtype="f64")
    o2, p2 = chunkwise_fp64(q, k, v, g, beta, pool, slot_idx, cu, scale=0.3,
                            chunk_size=90, gate=gate, state_dtype="f64")
    np.testing.assert_allclose(o2, o1, atol=1e-12)
    np.testing.assert_allclose(p2, p1, atol=1e-12)


def test_forward_substitution_is_the_inverse():
    """(I + L) X = B solved row by row equals a library solve; T (I + L) = I."""
    rng = np.random.default_rng(16)
    L = np.tril(rng.standard_normal((64, 64)) * 0.2, -1)
    B = rng.standard_normal((64, 7))
    X = forward_substitution_unit_lower(L, B)
    np.testing.assert_allclose(X, np.linalg.solve(np.eye(64) + L, B), atol=1e-10)
    Tm = forward_substitution_unit_lower(L, np.eye(64))
    np.testing.assert_allclose(Tm @ (np.eye(64) + L), np.eye(64), atol=1e-10)


# ---------------------------------------------------------------------------
# batch structure: GQA, ragged sequences, pool slots, resume, scale
# ---------------------------------------------------------------------------

def test_gqa_equals_expanded_heads():
    """HV = 2 HK: value head h reads key head h // 2 (Mojo page, GQA)."""
    rng = np.random.default_rng(17)
    q, k, v, g, beta, pool, slot_idx, cu = ragged_problem(rng, [20, 13], 2, 4, 5, 3, "scalar")
    o1, p1 = recurrent_fp64(q, k, v, g, beta, pool, slot_idx, cu, scale=0.5,
                            state_dtype="f64")
    qe, ke = np.repeat(q, 2, axis=1), np.repeat(k, 2, axis=1)
    o2, p2 = recurrent_fp64(qe, ke, v, g, beta, pool, slot_idx, cu, scale=0.5,
                            state_dtype="f64")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1, p2)


def test_ragged_batch_equals_separate_runs_and_leaves_other_slots():
    rng = np.random.default_rng(18)
    lens = [9, 0, 17, 4]
    q, k, v, g, beta, pool, slot_idx, cu = ragged_problem(rng, lens, 1, 2, 4, 3,
                                                          "channel", slots=7)
    o, p = recurrent_fp64(q, k, v, g, beta, pool, slot_idx, cu, scale=0.5,
                          gate="channel", state_dtype="f64")
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        on, pn = recurrent_fp64(q[a:b], k[a:b], v[a:b], g[a:b], beta[a:b], pool,
                                [slot_idx[n]], [0, b - a], scale=0.5,
                                gate="channel", state_dtype="f64")
        np.testing.assert_array_equal(o[a:b], on)
        np.testing.assert_array_equal(p[slot_idx[n]], pn[slot_idx[n]])
    untouched = np.setdiff1d(np.arange(7), slot_idx)
    np.testing.assert_array_equal(p[untouched], pool[untouched])
    # the empty sequence passes its state through unchanged
    np.testing.assert_array_equal(p[slot_idx[1]], pool[slot_idx[1]])


def test_zero_init_ignores_pool_contents():
    rng = np.random.default_rng(19)
    q, k, v, g, beta, pool, slot_idx, cu = ragged_problem(rng, [12], 1, 1, 4, 3, "scalar")
    o1, p1 = recurrent_fp64(q, k, v, g, beta, pool, slot_idx, cu, scale=0.5,
                            zero_init=True, state_dtype="f64")
    z = pool.copy()
    z[slot_idx[0]] = 0
    o2, p2 = recurrent_fp64(q, k, v, g, beta, z, slot_idx, cu, scale=0.5,
                            state_dtype="f64")
    np.testing.assert_array_equal(o1, o2)
    np.testing.assert_array_equal(p1[slot_idx[0]], p2[slot_idx[0]])


def test_split_prefill_resumes_from_the_pool():
    """Tokens [0, m) then [m, T) through the pool = one pass over [0, T)
    (From Attention to Learned Memory section 1: S0 is the cached prefix)."""
    rng = np.random.default_rng(20)
    q, k, v, g, beta, pool, slot_idx, cu = ragged_problem(rng, [40], 1, 2, 4, 3, "scalar")
    o, p = recurrent_fp64(q, k, v, g, beta, pool, slot_idx, cu, scale=0.5,
                          state_dtype="f64")
    m = 17
    oa, pa = recurrent_fp64(q[:m], k[:m], v[:m], g[:m], beta[:m], pool, slot_idx,
                            [0, m], scale=0.5, state_dtype="f64")
    ob, pb = recurrent_fp64(q[m:], k[m:], v[m:], g[m:], beta[m:], pa, slot_idx,
                            [0, 40 - m], scale=0.5, state_dtype="f64")
    np.testing.assert_allclose(np.concatenate([oa, ob]), o, atol=1e-14)
    np.testing.assert_allclose(pb, p, atol=1e-14)


def test_scale_is_linear():
    rng = np.random.default_rng(21)
    q, k, v, g, beta, pool = tiny(rng, T=8)
    o1, p1 = run(q, k, v, g, beta, pool, scale=0.25)
    o2, p2 = run(q, k, v, g, beta, pool, scale=0.75)
    np.testing.assert_allclose(o2, 3 * o1, atol=1e-13)
    np.testing.assert_array_equal(p1, p2)


def test_alice_bob_golden():
    with open(os.path.join(GOLDEN, "alice_bob.json")) as f:
        gold = json.load(f)
    keys = {n: np.array(x) for n, x in gold["keys"].items()}
    vals = {n: np.array(x) for n, x in gold["values"].items()}
    for case in gold["cases"]:
        ks = np.stack([keys[a] for a, _ in gold["writes"]])[:, None]
        vs = np.stack([vals[b] for _, b in gold["writes"]])[:, None]
        beta = np.ones((len(ks), 1))
        beta[-1, 0] = case["last_beta"]
        pool = np.zeros((1, 1, 2, 3))
        _, p = recurrent_fp64(ks, ks, vs, None, beta, pool, [0], [0, len(ks)],
                              scale=1.0, gate="none", state_dtype="f64")
        S = p[0, 0].T
        np.testing.assert_array_equal(S @ keys["alice"], case["read_alice"])
        np.testing.assert_array_equal(S @ keys["bob"], case["read_bob"])


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------

def test_bf16_rounding_matches_library_on_fp32_values():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(22)
    x = np.concatenate([rng.standard_normal(20000) * 10.0 ** rng.integers(-30, 30, 20000),
                        [1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 2 ** -130, 0.0]])
    x = x.astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float64).numpy()
    np.testing.assert_array_equal(round_f64_to_bf16(x.astype(np.float64)), ref)


def test_bf16_rounding_is_direct_from_fp64():
    # 1 + 2^-8 + 2^-30 lies above the tie between 1 and 1 + 2^-7, so it rounds
    # up; an intermediate fp32 rounding would land on the tie and go to 1.0
    x = np.array([1 + 2 ** -8 + 2 ** -30, 1 + 2 ** -8, 1 + 3 * 2 ** -8])
    np.testing.assert_array_equal(round_f64_to_bf16(x), [1 + 2 ** -7, 1.0, 1 + 2 ** -6])


def test_pool_write_rounds_to_bf16():
    rng = np.random.default_rng(23)
    q, k, v, g, beta, pool = tiny(rng, T=5)
    _, p64 = run(q, k, v, g, beta, pool)
    _, pbf = recurrent_fp64(q, k, v, g, beta, pool, [0], [0, 5], scale=1.0,
                            state_dtype="bf16")
    np.testing.assert_array_equal(pbf[0], round_f64_to_bf16(p64[0]))
    np.testing.assert_array_equal(pbf[1], pool[1])


# ---------------------------------------------------------------------------
# L2 normalisation of q and k ("gated_delta" Mojo page, kernel steps 2, 4, 5)
# ---------------------------------------------------------------------------

def test_l2_normalise_closed_forms():
    """A 3-4-5 vector, a one-hot vector, the zero vector and the guard's
    effect, each against its value worked out by hand."""
    from oracle import l2_normalise_fp64, L2_EPS
    assert L2_EPS == 1e-6
    np.testing.assert_array_equal(l2_normalise_fp64(np.array([3.0, 4.0]), eps=0.0), [0.6, 0.8])
    np.testing.assert_array_equal(l2_normalise_fp64(np.array([0.0, -2.0, 0.0]), eps=0.0),
                                  [0.0, -1.0, 0.0])
    np.testing.assert_array_equal(l2_normalise_fp64(np.zeros(4)), np.zeros(4))
    # with the guard: 3 / sqrt(25 + 1e-6) = 0.6 / sqrt(1 + 4e-8)
    y = l2_normalise_fp64(np.array([3.0, 4.0]))
    np.testing.assert_allclose(y, np.array([0.6, 0.8]) / np.sqrt(1.0 + 4e-8), rtol=2e-16, atol=0)


def test_l2_normalise_norm_and_scale_invariance():
    """|x^|^2 = |x|^2 / (|x|^2 + eps) row by row (rows over the last axis of
    a [T, H, D] array), and with eps = 0 the result ignores positive scales."""
    from oracle import l2_normalise_fp64
    rng = np.random.default_rng(5)
    x = rng.standard_normal((6, 3, 16)) * rng.uniform(0.01, 5.0, size=(6, 3, 1))
    y = l2_normalise_fp64(x, eps=1e-6)
    n2 = np.sum(x * x, axis=-1)
    np.testing.assert_allclose(np.sum(y * y, axis=-1), n2 / (n2 + 1e-6), rtol=1e-14)
    np.testing.assert_allclose(l2_normalise_fp64(7.5 * x, eps=0.0), l2_normalise_fp64(x, eps=0.0),
                               rtol=1e-15, atol=1e-16)


def test_normalised_key_writes_exactly():
    """With beta = 1 and no decay, a raw key k writes v along k / |k| exactly:
    S (k / |k|) = v after the step (the delta write of the KDA page section 2
    with the Mojo page's normalised key)."""
    from oracle import l2_normalise_fp64
    rng = np.random.default_rng(6)
    DK, DV = 5, 3
    k = 3.0 * rng.standard_normal((1, 1, DK))
    q = rng.standard_normal((1, 1, DK))
    v = rng.standard_normal((1, 1, DV))
    pool = rng.standard_normal((1, 1, DK, DV))
    kn = l2_normalise_fp64(k, eps=0.0)
    _, p = oracle.recurrent_fp64(l2_normalise_fp64(q, eps=0.0), kn, v, np.zeros((1, 1)),
                                 np.ones((1, 1)), pool, [0], [0, 1], scale=1.0, state_dtype="f64")
    S = p[0, 0].T
    np.testing.assert_allclose(S @ kn[0, 0], v[0, 0], rtol=1e-13, atol=1e-13)
