"""Pins of the Gated DeltaProduct oracle ("Linear attention visualized",
section "Gated Delta Product (GDP)"), each against something other than the
oracle itself: the page's virtual-sequence construction run through the
tokenwise GDN recurrence, the product of generalised Householder transitions
written out as matrices, exact writes along orthonormal keys, the single
decay per token, and the reduction to GDN at one transition per token."""
import numpy as np
import pytest

from oracle import delta_product_fp64, recurrent_fp64


def unit(x, axis=-1):
    return x / np.linalg.norm(x, axis=axis, keepdims=True)


def problem(rng, lens, P, HK=1, HV=2, DK=6, DV=5, gate="scalar", slots=5):
    T = int(sum(lens))
    q = unit(rng.standard_normal((T, HK, DK)))
    k = unit(rng.standard_normal((T * P, HK, DK)))
    v = rng.standard_normal((T * P, HV, DV))
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T * P, HV))))
    if gate == "scalar":
        g = -np.log1p(np.exp(rng.standard_normal((T, HV)) - 1.0))
    elif gate == "channel":
        g = -np.log1p(np.exp(rng.standard_normal((T, HV, DK)) - 1.0))
    else:
        g = None
    pool = 0.3 * rng.standard_normal((slots, HV, DK, DV))
    slot_idx = rng.choice(slots, size=len(lens), replace=False)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int64)
    return dict(q=q, k=k, v=v, g=g, beta=beta, pool=pool, slot_idx=slot_idx, cu_seqlens=cu)


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("rule", ["delta", "linear"])
def test_one_transition_is_gdn(gate, rule):
    rng = np.random.default_rng(1)
    x = problem(rng, (4, 0, 3), 1, gate=gate)
    if rule == "linear":
        x["beta"] = None
    a = delta_product_fp64(**x, products=1, scale=0.7, rule=rule, gate=gate, state_dtype="f64")
    b = recurrent_fp64(**x, scale=0.7, rule=rule, gate=gate, state_dtype="f64")
    np.testing.assert_allclose(a[0], b[0], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(a[1], b[1], rtol=1e-13, atol=1e-14)


def virtual_sequence(x, P, gate):
    """The page's table: substep j of token t is virtual step t*P + j; the
    decay sits on the first virtual step of a token (1 elsewhere, g = 0), the
    query on the last (zero elsewhere)."""
    T = x["q"].shape[0]
    qv = np.zeros((T * P,) + x["q"].shape[1:])
    qv[P - 1::P] = x["q"]
    gv = None
    if gate != "none":
        gv = np.zeros((T * P,) + x["g"].shape[1:])
        gv[0::P] = x["g"]
    return dict(q=qv, k=x["k"], v=x["v"], g=gv, beta=x["beta"], pool=x["pool"],
                slot_idx=x["slot_idx"], cu_seqlens=np.asarray(x["cu_seqlens"]) * P)


@pytest.mark.parametrize("P", [2, 3])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("rule", ["delta", "linear"])
def test_equals_gdn_over_the_virtual_sequence(P, gate, rule):
    rng = np.random.default_rng(10 * P + len(gate))
    x = problem(rng, (5, 0, 2, 3), P, HK=1, HV=2, gate=gate)
    if rule == "linear":
        x["beta"] = None
    o, pool = delta_product_fp64(**x, products=P, scale=0.5, rule=rule, gate=gate,
                                 state_dtype="f64")
    ov, poolv = recurrent_fp64(**virtual_sequence(x, P, gate), scale=0.5, rule=rule, gate=gate,
                               state_dtype="f64")
    np.testing.assert_allclose(o, ov[P - 1::P], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(pool, poolv, rtol=1e-12, atol=1e-13)


def test_householder_product_closed_form():
    """One head, scalar gate: S_t = a_t S_{t-1} H_1 ... H_P + sum_j beta_j v_j
    k_j^T H_{j+1} ... H_P with H_j = I - beta_j k_j k_j^T (value-by-key S)."""
    rng = np.random.default_rng(5)
    P, T, DK, DV = 3, 4, 5, 4
    x = problem(rng, (T,), P, HK=1, HV=1, DK=DK, DV=DV, gate="scalar", slots=1)
    x["slot_idx"] = np.array([0])
    o, pool = delta_product_fp64(**x, products=P, scale=1.3, gate="scalar", state_dtype="f64")
    S = x["pool"][0, 0].T.copy()
    for t in range(T):
        H = [np.eye(DK) - x["beta"][t * P + j, 0] * np.outer(x["k"][t * P + j, 0], x["k"][t * P + j, 0])
             for j in range(P)]
        prod = np.eye(DK)
        for j in range(P):
            prod = prod @ H[j]
        Snew = np.exp(x["g"][t, 0]) * S @ prod
        for j in range(P):
            tail = np.eye(DK)
            for i in range(j + 1, P):
                tail = tail @ H[i]
            Snew += x["beta"][t * P + j, 0] * np.outer(x["v"][t * P + j, 0], x["k"][t * P + j, 0]) @ tail
        S = Snew
        np.testing.assert_allclose(o[t, 0], 1.3 * S @ x["q"][t, 0], rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(pool[0, 0], S.T, rtol=1e-12, atol=1e-13)


def test_orthonormal_substeps_write_exactly():
    """beta = 1 along orthonormal keys of one token: every substep's value is
    stored exactly along its key, and the later substeps leave it in place."""
    rng = np.random.default_rng(7)
    P, DK, DV = 3, 6, 4
    Qm, _ = np.linalg.qr(rng.standard_normal((DK, DK)))
    x = problem(rng, (1,), P, HK=1, HV=1, DK=DK, DV=DV, gate="none", slots=1)
    x["slot_idx"] = np.array([0])
    x["k"] = Qm[:, :P].T[:, None, :]
    x["beta"] = np.ones((P, 1))
    x["q"] = Qm[:, 1][None, None, :]
    o, pool = delta_product_fp64(**x, products=P, scale=1.0, gate="none", state_dtype="f64")
    S = pool[0, 0].T
    for j in range(P):
        np.testing.assert_allclose(S @ Qm[:, j], x["v"][j, 0], atol=1e-13)
    np.testing.assert_allclose(o[0, 0], x["v"][1, 0], atol=1e-13)
    # directions orthogonal to every key keep the initial state's read-out
    S0 = x["pool"][0, 0].T
    for j in range(P, DK):
        np.testing.assert_allclose(S @ Qm[:, j], S0 @ Qm[:, j], atol=1e-13)


def test_repeated_key_last_substep_wins():
    rng = np.random.default_rng(8)
    x = problem(rng, (1,), 2, HK=1, HV=1, gate="none", slots=1)
    x["slot_idx"] = np.array([0])
    x["k"][1] = x["k"][0]
    x["beta"][:] = 1.0
    x["q"] = x["k"][:1].copy()
    o, _ = delta_product_fp64(**x, products=2, scale=1.0, gate="none", state_dtype="f64")
    np.testing.assert_allclose(o[0, 0], x["v"][1, 0], atol=1e-13)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
@pytest.mark.parametrize("P", [1, 2, 4])
def test_decay_applied_once_per_token(gate, P):
    """With beta = 0 nothing is written: the state after T tokens is the
    initial state times the product of the T decays, whatever n_h is."""
    rng = np.random.default_rng(9)
    T = 5
    x = problem(rng, (T,), P, HK=1, HV=2, gate=gate, slots=1)
    x["slot_idx"] = np.array([0])
    x["beta"][:] = 0.0
    _, pool = delta_product_fp64(**x, products=P, scale=1.0, gate=gate, state_dtype="f64")
    G = x["g"].sum(axis=0)                     # [HV] or [HV, DK]
    S0 = x["pool"][0]                          # [HV, DK, DV]
    want = S0 * np.exp(G)[:, None, None] if gate == "scalar" else S0 * np.exp(G)[:, :, None]
    np.testing.assert_allclose(pool[0], want, rtol=1e-13)
