"""GPU parity of the speculative-decode verify ring and state fold (the
"gated_delta" Mojo page names a verify that records a ring instead of writing
the state back, and a fold that applies accepted records) against the fp64
oracle: verify's outputs are the recurrence's, the pool is not written, and
the fold of every sequence's accepted prefix gives the recurrence's state
after those tokens."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from helpers import check_out, check_state, dev, host, widened

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

WINDOWS = (1, 4, 0, 7, 33, 64)


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


def small(D, in_dtype, gate, rule, state_dtype="f32", seed=91):
    return synth.Workload(name="win", seqlens=WINDOWS, HK=2, HV=4, DK=D, DV=D, in_dtype=in_dtype,
                          gate=gate, rule=rule, gate_shift=2.0 if gate != "channel" else 3.0,
                          state_dtype=state_dtype, num_slots=8, zero_init=False, seed=seed)


COMBOS = list(itertools.product([64, 128], ["bf16", "f32"], ["none", "scalar", "channel"],
                                ["delta", "linear"]))


@pytest.mark.parametrize("D,in_dtype,gate,rule", COMBOS,
                         ids=[f"d{D}-{i}-{g}-{r}" for D, i, g, r in COMBOS])
def test_verify_and_fold_match_oracle(D, in_dtype, gate, rule):
    gdr = _gdr()
    state_dtype = "bf16" if (D == 128 and gate == "scalar") else "f32"
    w = small(D, in_dtype, gate, rule, state_dtype)
    x = synth.generate(w)
    xw = widened(w, x)
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v")}
    g, beta = dev(x["g"], "f32"), dev(x["beta"], "f32")
    pool = dev(x["pool"], state_dtype)
    slot, cu = dev(x["slot_idx"], "i32"), dev(x["cu_seqlens"], "i32")
    pool0 = pool.clone()
    print(f"verify D={D} in={in_dtype} gate={gate} rule={rule} windows={WINDOWS}", flush=True)
    o, ring = gdr.verify_ring(d["q"], d["k"], d["v"], g, beta if rule == "delta" else None, pool, slot,
                              cu, scale=D ** -0.5, rule=rule, gate=gate)
    torch.cuda.synchronize()
    assert torch.equal(pool, pool0), "the verify must not write the pool"
    o_ref, ring_ref = oracle.verify_ring_fp64(xw["q"], xw["k"], xw["v"], xw["g"], xw["beta"], xw["pool"],
                                              x["slot_idx"], x["cu_seqlens"], scale=D ** -0.5, rule=rule,
                                              gate=gate)
    check_out(host(o, in_dtype), o_ref, in_dtype)
    E = ring_ref.shape[2]
    rg = host(ring, "f32")[:, :, :E]
    check_out(rg[:, :, :D], ring_ref[:, :, :D], in_dtype, what="e")
    np.testing.assert_allclose(rg[:, :, D:2 * D], ring_ref[:, :, D:2 * D], rtol=0, atol=1e-6)
    np.testing.assert_allclose(rg[:, :, 2 * D:], ring_ref[:, :, 2 * D:], rtol=0, atol=0)

    rng = np.random.default_rng(D + len(gate) + len(rule))
    lens = np.diff(x["cu_seqlens"])
    acc = np.array([rng.integers(0, n + 1) for n in lens], dtype=np.int32)
    acc[1] = lens[1] + 5           # more than the window: clamped
    gdr.state_fold(ring, dev(acc, "i32"), pool, slot, cu, HK=w.HK, gate=gate)
    torch.cuda.synchronize()
    want = oracle.state_fold_fp64(xw["pool"], ring_ref, x["slot_idx"], x["cu_seqlens"], np.minimum(acc, lens),
                                  DK=D, DV=D, gate=gate, state_dtype="f64")
    got = host(pool, state_dtype)
    for n, s in enumerate(x["slot_idx"]):
        if np.minimum(acc, lens)[n] == 0:
            assert torch.equal(pool[s], pool0[s])
        else:
            check_state(got[s], want[s], in_dtype, state_dtype)
    untouched = np.setdiff1d(np.arange(w.num_slots), x["slot_idx"])
    assert torch.equal(pool[untouched], pool0[untouched])


def test_full_fold_equals_recurrent_fwd():
    """Folding every record equals running the window with gdr_recurrent_fwd
    (the same schedule writing the state): bit-identical outputs."""
    gdr = _gdr()
    w = small(128, "bf16", "scalar", "delta")
    x = synth.generate(w)
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v")}
    g, beta = dev(x["g"], "f32"), dev(x["beta"], "f32")
    slot, cu = dev(x["slot_idx"], "i32"), dev(x["cu_seqlens"], "i32")
    p1, p2 = dev(x["pool"], "f32"), dev(x["pool"], "f32")
    o1, ring = gdr.verify_ring(d["q"], d["k"], d["v"], g, beta, p1, slot, cu)
    gdr.state_fold(ring, dev(np.diff(x["cu_seqlens"]), "i32"), p1, slot, cu, HK=w.HK, gate="scalar")
    o2 = gdr.recurrent_fwd(d["q"], d["k"], d["v"], g, beta, p2, slot, cu)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    check_state(host(p1, "f32"), host(p2, "f32"), "bf16", "f32")
