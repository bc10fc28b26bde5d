"""Pins of the verify-ring oracle (the "gated_delta" Mojo page names a verify
kernel that records a ring instead of writing the state, and a fold that
applies accepted records): against the tokenwise recurrence, verify's outputs
are the recurrence's outputs, the pool is not written, and folding the first
j records of every sequence gives the recurrence's state after j tokens."""
import numpy as np
import pytest

from oracle import recurrent_fp64, state_fold_fp64, verify_ring_fp64


def problem(rng, lens, gate, HK=1, HV=2, DK=5, DV=4, slots=5):
    T = int(sum(lens))
    unit = lambda x: x / np.linalg.norm(x, axis=-1, keepdims=True)
    g = None
    if gate == "scalar":
        g = -np.log1p(np.exp(rng.standard_normal((T, HV))))
    elif gate == "channel":
        g = -np.log1p(np.exp(rng.standard_normal((T, HV, DK))))
    return dict(q=unit(rng.standard_normal((T, HK, DK))), k=unit(rng.standard_normal((T, HK, DK))),
                v=rng.standard_normal((T, HV, DV)), g=g,
                beta=1 / (1 + np.exp(-rng.standard_normal((T, HV)))),
                pool=rng.standard_normal((slots, HV, DK, DV)),
                slot_idx=rng.choice(slots, size=len(lens), replace=False),
                cu_seqlens=np.concatenate([[0], np.cumsum(lens)]).astype(np.int64))


@pytest.mark.parametrize("gate", ["none", "scalar", "channel"])
@pytest.mark.parametrize("rule", ["delta", "linear"])
def test_verify_outputs_and_every_fold_prefix(gate, rule):
    rng = np.random.default_rng(len(gate) + len(rule))
    lens = (4, 0, 1, 6)
    x = problem(rng, lens, gate)
    if rule == "linear":
        x["beta"] = None
    pool0 = x["pool"].copy()
    o, ring = verify_ring_fp64(**x, scale=0.8, rule=rule, gate=gate)
    assert np.array_equal(x["pool"], pool0)
    o_ref, _ = recurrent_fp64(**x, scale=0.8, rule=rule, gate=gate, state_dtype="f64")
    np.testing.assert_allclose(o, o_ref, rtol=1e-13, atol=1e-13)
    for j in range(max(lens) + 1):
        acc = np.minimum(j, lens)
        got = state_fold_fp64(x["pool"], ring, x["slot_idx"], x["cu_seqlens"], acc, DK=5, DV=4,
                              gate=gate, state_dtype="f64")
        # the recurrence over each sequence's first acc[n] tokens
        keep = np.concatenate([np.arange(c, c + a) for c, a in zip(x["cu_seqlens"][:-1], acc)]).astype(int)
        sub = {n: (None if x[n] is None else x[n][keep]) for n in ("q", "k", "v", "g", "beta")}
        cu = np.concatenate([[0], np.cumsum(acc)])
        _, want = recurrent_fp64(**sub, pool=x["pool"], slot_idx=x["slot_idx"], cu_seqlens=cu,
                                 scale=0.8, rule=rule, gate=gate, state_dtype="f64")
        np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-12)


def test_zero_accepted_leaves_the_state():
    rng = np.random.default_rng(2)
    x = problem(rng, (3, 2), "scalar")
    _, ring = verify_ring_fp64(**x, scale=1.0)
    got = state_fold_fp64(x["pool"], ring, x["slot_idx"], x["cu_seqlens"], [0, 0], DK=5, DV=4,
                          gate="scalar", state_dtype="f64")
    np.testing.assert_array_equal(got, x["pool"])
