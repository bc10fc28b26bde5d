"""Pins of the gradient oracle of the gated delta and gated linear rules
(oracle/recurrent_bwd.py), each against something other than that oracle:
central finite differences of the forward oracle (the recurrence of "You
Could Have Come Up With Kimi Delta Attention" and the gated variants of
"Linear attention visualized") for every input, including the initial
state; the closed-form linear-attention gradients of "From Attention to
Learned Memory" (section "Backward: reverse the boundary scan, then
differentiate each chunk"); and the initial state's gradient of the plain
linear rule written out."""
import numpy as np
import pytest

from oracle import linear_attention_grads_fp64, recurrent_fp64, recurrent_grads_fp64


def unit(x):
    return x / np.linalg.norm(x, axis=-1, keepdims=True)


def problem(rng, lens, HK, HV, DK, DV, gate, rule, slots=4):
    T = int(sum(lens))
    x = dict(q=unit(rng.standard_normal((T, HK, DK))), k=unit(rng.standard_normal((T, HK, DK))),
             v=rng.standard_normal((T, HV, DV)),
             beta=1.0 / (1.0 + np.exp(-rng.standard_normal((T, HV)))) if rule == "delta" else None,
             g=None, pool=0.5 * rng.standard_normal((slots, HV, DK, DV)),
             slot_idx=rng.choice(slots, size=len(lens), replace=False),
             cu_seqlens=np.concatenate([[0], np.cumsum(lens)]).astype(np.int64))
    if gate == "scalar":
        x["g"] = -np.log1p(np.exp(rng.standard_normal((T, HV))))
    elif gate == "channel":
        x["g"] = -np.log1p(np.exp(rng.standard_normal((T, HV, DK))))
    return x


def loss(x, do, scale, rule, gate, zero_init):
    o, _ = recurrent_fp64(**x, scale=scale, rule=rule, gate=gate, zero_init=zero_init,
                          state_dtype="f64")
    return float(np.sum(o * do))


def fd_grad(x, name, do, scale, rule, gate, zero_init, eps=1e-6):
    base = x[name]
    grad = np.zeros_like(base)
    for idx in np.ndindex(base.shape):
        old = base[idx]
        base[idx] = old + eps
        lp = loss(x, do, scale, rule, gate, zero_init)
        base[idx] = old - eps
        lm = loss(x, do, scale, rule, gate, zero_init)
        base[idx] = old
        grad[idx] = (lp - lm) / (2 * eps)
    return grad


@pytest.mark.parametrize("zero_init", [False, True])
@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("rule", ["delta", "linear"])
def test_matches_finite_differences(rule, gate, zero_init):
    rng = np.random.default_rng(100 + 10 * len(gate) + len(rule) + zero_init)
    HK, HV, DK, DV = 1, 2, 4, 3
    x = problem(rng, (3, 0, 4), HK, HV, DK, DV, gate, rule)
    do = rng.standard_normal(x["v"].shape)
    scale = 0.8
    got = recurrent_grads_fp64(**x, do=do, scale=scale, rule=rule, gate=gate, zero_init=zero_init)
    tol = dict(rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(got["dq"], fd_grad(x, "q", do, scale, rule, gate, zero_init), **tol)
    np.testing.assert_allclose(got["dk"], fd_grad(x, "k", do, scale, rule, gate, zero_init), **tol)
    np.testing.assert_allclose(got["dv"], fd_grad(x, "v", do, scale, rule, gate, zero_init), **tol)
    if rule == "delta":
        np.testing.assert_allclose(got["dbeta"], fd_grad(x, "beta", do, scale, rule, gate, zero_init),
                                   **tol)
    else:
        assert got["dbeta"] is None
    if gate != "none":
        np.testing.assert_allclose(got["dg"], fd_grad(x, "g", do, scale, rule, gate, zero_init), **tol)
    else:
        assert got["dg"] is None
    # the initial state: perturb each sequence's pool slot (a zero-init run
    # ignores the pool, so its gradient is the one for a zero state and the
    # pool's own gradient is zero)
    dpool = fd_grad(x, "pool", do, scale, rule, gate, zero_init)
    if zero_init:
        np.testing.assert_allclose(dpool, 0.0, atol=1e-9)
        x0 = dict(x, pool=np.zeros_like(x["pool"]))
        dpool = fd_grad(x0, "pool", do, scale, rule, gate, False)
    for n, slot in enumerate(x["slot_idx"]):
        np.testing.assert_allclose(got["dstate0"][n], dpool[slot], **tol)


@pytest.mark.parametrize("zero_init", [False, True])
def test_plain_linear_matches_closed_form(zero_init):
    rng = np.random.default_rng(7)
    x = problem(rng, (5, 0, 7, 2), 3, 3, 6, 5, "none", "linear")
    do = rng.standard_normal(x["v"].shape)
    got = recurrent_grads_fp64(**x, do=do, scale=0.6, rule="linear", gate="none",
                               zero_init=zero_init)
    dq, dk, dv = linear_attention_grads_fp64(x["q"], x["k"], x["v"], do, x["pool"], x["slot_idx"],
                                             x["cu_seqlens"], scale=0.6, zero_init=zero_init)
    np.testing.assert_allclose(got["dq"], dq, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["dk"], dk, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(got["dv"], dv, rtol=1e-12, atol=1e-13)
    # dL/dS_0 of S_t = S_0 + ...: scale * sum_t do_t q_t^T, stored transposed
    cu = x["cu_seqlens"]
    for n in range(len(cu) - 1):
        want = 0.6 * np.einsum("thk,thv->hkv", x["q"][cu[n]:cu[n + 1]], do[cu[n]:cu[n + 1]])
        np.testing.assert_allclose(got["dstate0"][n], want, rtol=1e-12, atol=1e-13)


def test_zero_beta_freezes_the_state():
    """beta = 0: the delta rule writes nothing, so the outputs read the decayed
    initial state only and no gradient reaches k or v."""
    rng = np.random.default_rng(9)
    x = problem(rng, (6,), 1, 1, 5, 4, "scalar", "delta", slots=1)
    x["slot_idx"] = np.array([0])
    x["beta"][:] = 0.0
    do = rng.standard_normal(x["v"].shape)
    got = recurrent_grads_fp64(**x, do=do, scale=1.0, rule="delta", gate="scalar")
    np.testing.assert_allclose(got["dk"], 0.0, atol=1e-15)
    np.testing.assert_allclose(got["dv"], 0.0, atol=1e-15)
    # o_t = exp(G_t) S_0 q_t with G_t the running gate sum: dq_t = exp(G_t) S_0^T do_t
    G = np.cumsum(x["g"][:, 0])
    S0 = x["pool"][0, 0].T
    want = np.exp(G)[:, None] * (do[:, 0] @ S0)
    np.testing.assert_allclose(got["dq"][:, 0], want, rtol=1e-12, atol=1e-13)
