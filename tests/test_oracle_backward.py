"""Pins of the linear-attention gradient oracle ("From Attention to Learned
Memory", section "Backward: reverse the boundary scan, then differentiate
each chunk"), against the forward oracle: the loss L = sum(dO * O) is linear
in each of q, k and v separately, so a central difference of the tokenwise
forward recurrence along any direction equals the directional derivative up
to rounding; plus the page's chunked regrouping (the boundary-state gradient
scanned from the last chunk back) evaluated independently."""
import numpy as np
import pytest

from oracle import linear_attention_grads_fp64, recurrent_fp64


def problem(rng, lens, H=2, DK=5, DV=4, slots=4):
    T = int(sum(lens))
    x = dict(q=rng.standard_normal((T, H, DK)), k=rng.standard_normal((T, H, DK)),
             v=rng.standard_normal((T, H, DV)), do=rng.standard_normal((T, H, DV)),
             pool=rng.standard_normal((slots, H, DK, DV)),
             slot_idx=rng.choice(slots, size=len(lens), replace=False),
             cu_seqlens=np.concatenate([[0], np.cumsum(lens)]).astype(np.int64))
    return x


def loss(x, scale, zero_init):
    o, _ = recurrent_fp64(x["q"], x["k"], x["v"], None, None, x["pool"], x["slot_idx"],
                          x["cu_seqlens"], scale=scale, rule="linear", gate="none",
                          zero_init=zero_init, state_dtype="f64")
    return float(np.sum(o * x["do"]))


@pytest.mark.parametrize("zero_init", [True, False])
@pytest.mark.parametrize("name", ["q", "k", "v"])
def test_directional_derivative_matches_central_difference(name, zero_init):
    rng = np.random.default_rng(3 + len(name) + zero_init)
    x = problem(rng, (5, 0, 7, 1))
    dq, dk, dv = linear_attention_grads_fp64(x["q"], x["k"], x["v"], x["do"], x["pool"],
                                             x["slot_idx"], x["cu_seqlens"], scale=0.7,
                                             zero_init=zero_init)
    grad = {"q": dq, "k": dk, "v": dv}[name]
    D = rng.standard_normal(x[name].shape)
    h = 0.5   # L is linear in each argument: the central difference is exact
    xp, xm = dict(x), dict(x)
    xp[name] = x[name] + h * D
    xm[name] = x[name] - h * D
    fd = (loss(xp, 0.7, zero_init) - loss(xm, 0.7, zero_init)) / (2 * h)
    assert abs(fd - np.sum(grad * D)) <= 1e-10 * (1 + abs(fd))


def test_elementwise_gradients_by_finite_differences():
    """Every entry of dq, dk, dv on a 4-token sequence, one coordinate at a time."""
    rng = np.random.default_rng(11)
    x = problem(rng, (4,), H=1, DK=3, DV=2, slots=1)
    x["slot_idx"] = np.array([0])
    g = dict(zip("qkv", linear_attention_grads_fp64(x["q"], x["k"], x["v"], x["do"], x["pool"],
                                                   x["slot_idx"], x["cu_seqlens"], scale=1.3)))
    for name in "qkv":
        for idx in np.ndindex(x[name].shape):
            xp, xm = dict(x), dict(x)
            xp[name] = x[name].copy(); xp[name][idx] += 1.0
            xm[name] = x[name].copy(); xm[name][idx] -= 1.0
            fd = (loss(xp, 1.3, False) - loss(xm, 1.3, False)) / 2
            assert abs(fd - g[name][idx]) <= 1e-11 * (1 + abs(fd)), (name, idx)


def test_chunked_regrouping_of_the_page():
    """The page's schedule: G scanned from the last chunk back (G_c = G_{c+1} +
    scale dO_c^T Q_c, G after the last chunk = 0), then per chunk dV = scale
    (Q K^T (.) M)^T dO + K G_{c+1}^T, dK = scale E^T Q + V G_{c+1}, dQ = scale
    (dO S_c + E K) with E = (dO V^T) (.) M and S_c the incoming state."""
    rng = np.random.default_rng(17)
    T, C, DK, DV = 37, 8, 5, 4
    q, k = rng.standard_normal((T, DK)), rng.standard_normal((T, DK))
    v, do = rng.standard_normal((T, DV)), rng.standard_normal((T, DV))
    S0T = rng.standard_normal((DK, DV))
    s = 0.6
    want = linear_attention_grads_fp64(q[:, None], k[:, None], v[:, None], do[:, None], S0T[None, None],
                                       [0], [0, T], scale=s)
    bounds = list(range(0, T, C)) + [T]
    S = [S0T.T.copy()]                    # incoming states, value-by-key
    for a, b in zip(bounds[:-1], bounds[1:]):
        S.append(S[-1] + v[a:b].T @ k[a:b])
    G = np.zeros((DV, DK))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for c in range(len(bounds) - 2, -1, -1):
        a, b = bounds[c], bounds[c + 1]
        M = np.tril(np.ones((b - a, b - a)))
        Q, K, V, dO = q[a:b], k[a:b], v[a:b], do[a:b]
        E = (dO @ V.T) * M
        dv[a:b] = s * ((Q @ K.T) * M).T @ dO + K @ G.T
        dk[a:b] = s * E.T @ Q + V @ G
        dq[a:b] = s * (dO @ S[c] + E @ K)
        G = G + s * dO.T @ Q
    for got, ref in zip((dq, dk, dv), want):
        np.testing.assert_allclose(got, ref[:, 0], rtol=1e-12, atol=1e-12)
