"""GPU parity of gdr_recurrent_fwd (the tokenwise recurrence over a ragged
batch, the state on chip across each sequence) against the fp64 oracle, its
agreement with the chunkwise prefill, and the in-kernel L2 normalisation of
q and k (the "gated_delta" Mojo page) on raw and fused-buffer inputs."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from helpers import check_out, check_state, host, oracle_run, to_device, widened

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RAGGED = (0, 1, 63, 64, 65, 130, 200)


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


def small(D, in_dtype, gate, rule, state_dtype="f32", zero_init=False, seqlens=RAGGED, seed=41):
    return synth.Workload(
        name="small", seqlens=tuple(seqlens), HK=2, HV=4, DK=D, DV=D, in_dtype=in_dtype,
        gate=gate, rule=rule, gate_shift=2.0 if gate != "channel" else 3.0,
        state_dtype=state_dtype, num_slots=9, zero_init=zero_init, seed=seed)


COMBOS = list(itertools.product([64, 128], ["bf16", "f32"], ["none", "scalar", "channel"],
                                ["delta", "linear"]))


@pytest.mark.parametrize("D,in_dtype,gate,rule", COMBOS,
                         ids=[f"d{d}-{i}-{g}-{r}" for d, i, g, r in COMBOS])
def test_recurrent_fwd_matches_oracle(D, in_dtype, gate, rule):
    gdr = _gdr()
    state_dtype = "bf16" if (D == 128 and gate == "scalar") else "f32"
    w = small(D, in_dtype, gate, rule, state_dtype)
    x = synth.generate(w)
    d = to_device(w, x)
    pool_before = d["pool"].clone()
    print(f"recurrent_fwd D={D} in={in_dtype} gate={gate} rule={rule} lens={RAGGED}", flush=True)
    o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                          d["cu_seqlens"], scale=D ** -0.5, rule=rule, gate=gate)
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], D ** -0.5)
    check_out(host(o, in_dtype), o_ref, in_dtype)
    pool = host(d["pool"], state_dtype)
    for s in x["slot_idx"]:
        check_state(pool[s], pool_ref[s], in_dtype, state_dtype)
    untouched = np.setdiff1d(np.arange(w.num_slots), x["slot_idx"])
    assert torch.equal(d["pool"][untouched], pool_before[untouched])


@pytest.mark.parametrize("zero_init", [True, False])
def test_recurrent_fwd_zero_init_and_bf16_output(zero_init):
    gdr = _gdr()
    w = small(128, "bf16", "scalar", "delta", zero_init=zero_init, seqlens=(100, 0, 7, 64))
    x = synth.generate(w)
    d = to_device(w, x)
    o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                          d["cu_seqlens"], zero_init=zero_init, out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], 128 ** -0.5)
    og = host(o, "bf16")
    assert np.all(np.abs(og - o_ref) <= 2.0 ** -8 * np.abs(o_ref) + 3e-3 * np.sqrt(np.mean(o_ref ** 2)))
    for s in x["slot_idx"]:
        check_state(host(d["pool"], "f32")[s], pool_ref[s], "bf16", "f32")


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_recurrent_fwd_equals_chunk_fwd(gate):
    """The two prefill schedules agree on the same ragged batch (outputs and
    final states), both within the gate of the oracle."""
    gdr = _gdr()
    w = small(128, "bf16", gate, "delta", seqlens=(300, 5, 129))
    x = synth.generate(w)
    d = to_device(w, x)
    p2 = d["pool"].clone()
    o1 = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                       d["cu_seqlens"])
    o2 = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], p2, d["slot_idx"],
                           d["cu_seqlens"])
    torch.cuda.synchronize()
    check_out(host(o2, "f32"), host(o1, "f32"), "bf16")
    for s in x["slot_idx"]:
        check_state(host(p2, "f32")[s], host(d["pool"], "f32")[s], "bf16", "f32")


def _raw_qk(x, w, rng):
    """Raw (un-normalised) keys and queries: the seeded unit vectors times a
    positive factor per token and key head, stored in the input dtype. The
    stored values are what both sides normalise."""
    out = {}
    for name in ("q", "k"):
        unit = synth.widen(x[name], w.in_dtype)
        f = rng.uniform(0.2, 6.0, size=unit.shape[:2] + (1,))
        raw = unit * f
        out[name] = synth.f64_to_bf16_bits(raw) if w.in_dtype == "bf16" else raw.astype(np.float32)
    return out


@pytest.mark.parametrize("D,in_dtype,gate", list(itertools.product([64, 128], ["bf16", "f32"],
                                                                    ["scalar", "channel"])))
def test_recurrent_fwd_l2norm_matches_oracle(D, in_dtype, gate):
    gdr = _gdr()
    w = small(D, in_dtype, gate, "delta", seed=43)
    x = synth.generate(w)
    raw = _raw_qk(x, w, np.random.default_rng(D + len(gate)))
    x.update(raw)
    d = to_device(w, x)
    print(f"recurrent_fwd l2norm D={D} in={in_dtype} gate={gate}", flush=True)
    o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                          d["cu_seqlens"], qk_l2norm=True)
    torch.cuda.synchronize()
    xw = widened(w, x)
    xw["q"] = oracle.l2_normalise_fp64(xw["q"])
    xw["k"] = oracle.l2_normalise_fp64(xw["k"])
    o_ref, pool_ref = oracle_run(w, xw, x["slot_idx"], x["cu_seqlens"], D ** -0.5)
    check_out(host(o, in_dtype), o_ref, in_dtype)
    for s in x["slot_idx"]:
        check_state(host(d["pool"], "f32")[s], pool_ref[s], in_dtype, "f32")


def test_recurrent_fwd_l2norm_on_a_fused_qkv_buffer():
    """q, k, v as views into one fused [T, 2 HK DK + HV DV] buffer (the
    channel layout of the Mojo page) with raw keys and queries: the result is
    bit-identical to the one from separate contiguous tensors."""
    gdr = _gdr()
    w = small(128, "bf16", "scalar", "delta", seqlens=(70, 33, 0, 129), seed=47)
    x = synth.generate(w)
    x.update(_raw_qk(x, w, np.random.default_rng(3)))
    d = to_device(w, x)
    T = w.T_total
    kd, vd = w.HK * w.DK, w.HV * w.DV
    fused = torch.cat([d["q"].reshape(T, kd), d["k"].reshape(T, kd), d["v"].reshape(T, vd)], 1)
    q = fused[:, :kd].view(T, w.HK, w.DK)
    k = fused[:, kd:2 * kd].view(T, w.HK, w.DK)
    v = fused[:, 2 * kd:].view(T, w.HV, w.DV)
    pool2 = d["pool"].clone()
    o1 = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                           d["cu_seqlens"], qk_l2norm=True)
    o2 = gdr.recurrent_fwd(q, k, v, d["g"], d["beta"], pool2, d["slot_idx"], d["cu_seqlens"],
                           qk_l2norm=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(d["pool"], pool2)


def test_recurrent_fwd_long_sequence_matches_oracle():
    """One 4096-token sequence (the length of the prefill benchmark's
    sequences), sampled heads recomputed by the oracle: the fp32 state held
    in registers for the whole sequence stays within the gate."""
    gdr = _gdr()
    w = synth.Workload(name="long", seqlens=(4096,), HK=2, HV=2, DK=128, DV=128, in_dtype="bf16",
                       gate="scalar", rule="delta", gate_shift=2.0, state_dtype="f32",
                       num_slots=1, zero_init=True, seed=53)
    x = synth.generate(w)
    d = to_device(w, x)
    o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                          d["cu_seqlens"], zero_init=True)
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], 128 ** -0.5)
    check_out(host(o, "bf16"), o_ref, "bf16")
    check_state(host(d["pool"], "f32")[0], pool_ref[0], "bf16", "f32")
