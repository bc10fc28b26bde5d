"""GPU parity of the HIP path (through the C ABI) against the fp64 oracle on
small seeded inputs that span several chunks, ragged tails, empty sequences,
grouped heads and every gate / rule / dtype combination."""
import itertools

import numpy as np
import pytest

import synth
from helpers import (check_out, check_state, host, oracle_run, to_device, widened)

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


def small_workload(D, in_dtype, gate, rule, state_dtype, zero_init, seqlens, HK=2, HV=4,
                   slots=9, seed=11):
    return synth.Workload(
        name="small", seqlens=tuple(seqlens), HK=HK, HV=HV, DK=D, DV=D, in_dtype=in_dtype,
        gate=gate, rule=rule, gate_shift=2.0 if gate != "channel" else 3.0,
        state_dtype=state_dtype, num_slots=slots, zero_init=zero_init, seed=seed)


RAGGED = (0, 1, 63, 64, 65, 130, 200)
COMBOS = list(itertools.product([64, 128], ["bf16", "f32"], ["none", "scalar", "channel"],
                                ["delta", "linear"]))


@pytest.mark.parametrize("D,in_dtype,gate,rule", COMBOS,
                         ids=[f"d{d}-{i}-{g}-{r}" for d, i, g, r in COMBOS])
def test_chunk_fwd_matches_oracle(D, in_dtype, gate, rule):
    gdr = _gdr()
    state_dtype = "bf16" if (D == 128 and gate == "scalar") else "f32"
    w = small_workload(D, in_dtype, gate, rule, state_dtype, zero_init=False, seqlens=RAGGED)
    x = synth.generate(w)
    d = to_device(w, x)
    pool_before = d["pool"].clone()
    scale = D ** -0.5
    print(f"chunk_fwd D={D} in={in_dtype} gate={gate} rule={rule} lens={RAGGED}", flush=True)
    o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                      d["cu_seqlens"], scale=scale, rule=rule, gate=gate)
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], scale)
    check_out(host(o, in_dtype), o_ref, in_dtype)
    pool = host(d["pool"], state_dtype)
    for n, s in enumerate(x["slot_idx"]):
        check_state(pool[s], pool_ref[s], in_dtype, state_dtype)
    untouched = np.setdiff1d(np.arange(w.num_slots), x["slot_idx"])
    assert torch.equal(d["pool"][untouched], pool_before[untouched])


CHUNK_SIZE_COMBOS = [(16, 64, "bf16", "scalar", "delta"), (16, 128, "f32", "channel", "delta"),
                     (16, 128, "bf16", "channel", "linear"), (16, 128, "bf16", "none", "linear"),
                     (32, 128, "bf16", "none", "delta"), (32, 64, "f32", "scalar", "linear"),
                     (32, 128, "bf16", "channel", "delta"), (32, 128, "bf16", "scalar", "delta")]


@pytest.mark.parametrize("C,D,in_dtype,gate,rule", CHUNK_SIZE_COMBOS,
                         ids=[f"c{c}-d{d}-{i}-{g}-{r}" for c, d, i, g, r in CHUNK_SIZE_COMBOS])
def test_chunk_sizes_16_and_32(C, D, in_dtype, gate, rule):
    """chunk_size 16 and 32 (the chunk lengths section 4 of "From Attention to
    Learned Memory" takes beside 64) compute the same recurrence: ragged
    sequences spanning several chunks of that length, ending in partial ones,
    match the oracle."""
    gdr = _gdr()
    state_dtype = "bf16" if (D == 128 and gate == "scalar") else "f32"
    w = small_workload(D, in_dtype, gate, rule, state_dtype, zero_init=False, seqlens=RAGGED)
    x = synth.generate(w)
    d = to_device(w, x)
    scale = D ** -0.5
    print(f"chunk_fwd C={C} D={D} in={in_dtype} gate={gate} rule={rule} lens={RAGGED}", flush=True)
    o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                      d["cu_seqlens"], scale=scale, rule=rule, gate=gate, chunk_size=C)
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], scale)
    check_out(host(o, in_dtype), o_ref, in_dtype)
    pool = host(d["pool"], state_dtype)
    for s in x["slot_idx"]:
        check_state(pool[s], pool_ref[s], in_dtype, state_dtype)


@pytest.mark.parametrize("zero_init", [True, False])
@pytest.mark.parametrize("gate,rule", [("scalar", "delta"), ("channel", "delta"), ("channel", "linear")])
def test_chunk_fwd_zero_init_and_bf16_output(zero_init, gate, rule):
    """bf16 outputs on ragged partial chunks (100 = 64 + 36 tokens, 7, an
    empty sequence), from the scalar-gate kernel and the channel-gate pair."""
    gdr = _gdr()
    w = small_workload(128, "bf16", gate, rule, "f32", zero_init, seqlens=(100, 0, 7, 64))
    x = synth.generate(w)
    d = to_device(w, x)
    print(f"chunk_fwd bf16 out gate={gate} rule={rule} zero_init={zero_init}", flush=True)
    o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                      d["cu_seqlens"], zero_init=zero_init, out_dtype=torch.bfloat16, rule=rule, gate=gate)
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], 128 ** -0.5)
    # a bf16 output carries its own rounding (2^-9 relative); gate it elementwise
    og = host(o, "bf16")
    assert np.all(np.abs(og - o_ref) <= 2.0 ** -8 * np.abs(o_ref) + 3e-3 * np.sqrt(np.mean(o_ref ** 2)))
    for s in x["slot_idx"]:
        check_state(host(d["pool"], "f32")[s], pool_ref[s], "bf16", "f32")


STEP_COMBOS = list(itertools.product([64, 128], ["bf16", "f32"], ["none", "scalar", "channel"],
                                     ["delta", "linear"], ["f32", "bf16"]))


@pytest.mark.parametrize("D,in_dtype,gate,rule,state_dtype", STEP_COMBOS,
                         ids=[f"d{d}-{i}-{g}-{r}-pool{s}" for d, i, g, r, s in STEP_COMBOS])
def test_recurrent_step_matches_oracle(D, in_dtype, gate, rule, state_dtype):
    """Three consecutive steps chained through the pool."""
    gdr = _gdr()
    N, steps = 6, 3
    w = small_workload(D, in_dtype, gate, rule, state_dtype, zero_init=False,
                       seqlens=(1,) * N, slots=10).replace(steps=steps)
    x = synth.generate(w)
    d = to_device(w, x)
    xw = widened(w, x)
    pool_ref = xw["pool"]
    scale = D ** -0.5
    print(f"recurrent_step D={D} in={in_dtype} gate={gate} rule={rule} pool={state_dtype}", flush=True)
    for s in range(steps):
        sl = slice(s * N, (s + 1) * N)
        o = gdr.recurrent_step(d["q"][sl], d["k"][sl], d["v"][sl],
                               None if d["g"] is None else d["g"][sl],
                               None if d["beta"] is None else d["beta"][sl],
                               d["pool"], d["slot_idx"], scale=scale, rule=rule, gate=gate)
        torch.cuda.synchronize()
        xs = {k: (None if v is None else v[sl]) for k, v in xw.items() if k != "pool"}
        xs["pool"] = pool_ref
        o_ref, pool_ref = oracle_run(w.replace(zero_init=False), xs, x["slot_idx"],
                                     np.arange(N + 1), scale)
        check_out(host(o, in_dtype), o_ref, in_dtype)
    pool = host(d["pool"], state_dtype)
    for s in x["slot_idx"]:
        check_state(pool[s], pool_ref[s], in_dtype, state_dtype, roundings=steps)
    untouched = np.setdiff1d(np.arange(w.num_slots), x["slot_idx"])
    np.testing.assert_array_equal(pool[untouched], xw["pool"][untouched])


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_chunk_equals_repeated_steps(gate):
    """The two schedules agree: one chunk_fwd over T tokens = T recurrent steps."""
    gdr = _gdr()
    N, T, D = 3, 150, 128
    w = small_workload(D, "bf16", gate, "delta", "f32", zero_init=False, seqlens=(T,) * N)
    x = synth.generate(w)
    d = to_device(w, x)
    pool0 = d["pool"].clone()
    o_chunk = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"],
                            d["slot_idx"], d["cu_seqlens"])
    pool_chunk = d["pool"].clone()
    d["pool"].copy_(pool0)
    outs = []
    for t in range(T):
        idx = torch.arange(N, device="cuda") * T + t
        outs.append(gdr.recurrent_step(d["q"][idx], d["k"][idx], d["v"][idx], d["g"][idx],
                                       d["beta"][idx], d["pool"], d["slot_idx"]))
    o_step = torch.stack(outs, 1).reshape(N * T, w.HV, D)
    torch.cuda.synchronize()
    ref = host(o_step, "f32")
    check_out(host(o_chunk, "f32"), ref, "bf16")
    for s in x["slot_idx"]:
        check_state(host(pool_chunk, "f32")[s], host(d["pool"], "f32")[s], "bf16", "f32")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("rows", [1, 2, 3, 6])
@pytest.mark.parametrize("rule", ["delta", "linear"])
def test_channel_gate_slices(D, rows, rule):
    """The channel-gate prefill (bf16 inputs) passes per-chunk records through
    the workspace in slices of `rows` flat chunks; the state crosses slice
    boundaries through the workspace's fp32 carry. The result of a workspace
    that holds 1, 2, 3 or 6 rows of records equals the oracle's, and equals
    the result with the preferred workspace (one slice here) bit for bit.
    The linear rule (GLA) takes the same records with T' = I and W = 0."""
    gdr = _gdr()
    w = small_workload(D, "bf16", "channel", rule, "f32", zero_init=False,
                       seqlens=(130, 0, 64, 1, 200), seed=23)
    x = synth.generate(w)
    d = to_device(w, x)
    pool_pref = d["pool"].clone()
    args = (d["q"], d["k"], d["v"], d["g"], d["beta"] if rule == "delta" else None)
    # record of one (chunk, head): W, Q^ and K_r^T fragments, T' and A^, gamma
    row = w.HV * ((3 * 4 * (D // 32) + 2 * 6) * 2048 + 4 * D)
    carry = w.N * w.HV * D * D * 4
    ws = torch.empty(carry + rows * row, dtype=torch.uint8, device="cuda")
    print(f"channel-gate slices D={D} rows={rows} rule={rule}", flush=True)
    o = gdr.chunk_fwd(*args, d["pool"], d["slot_idx"], d["cu_seqlens"], workspace=ws, rule=rule)
    o_pref = gdr.chunk_fwd(*args, pool_pref, d["slot_idx"], d["cu_seqlens"], rule=rule)
    torch.cuda.synchronize()
    assert torch.equal(o, o_pref)
    assert torch.equal(d["pool"], pool_pref)
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], D ** -0.5)
    check_out(host(o, "bf16"), o_ref, "bf16")
    for sl in x["slot_idx"]:
        check_state(host(d["pool"], "f32")[sl], pool_ref[sl], "bf16", "f32")


@pytest.mark.parametrize("N", [10, 17, 40])
def test_channel_gate_workgroup_rounds(N):
    """The channel-gate state kernel gives every workgroup 16 value columns
    (d = 128: 8 workgroups per (sequence, head)); 40, 68 and 160 heads need
    more workgroups than the device's 256 compute units hold at once, so they
    run in several rounds. Every batch matches the oracle."""
    gdr = _gdr()
    lens = tuple(int(x) for x in np.random.default_rng(N).integers(0, 140, size=N))
    w = small_workload(128, "bf16", "channel", "delta", "f32", zero_init=False, seqlens=lens,
                       HK=2, HV=4, slots=N + 3, seed=31 + N)
    x = synth.generate(w)
    d = to_device(w, x)
    print(f"channel-gate widths N={N} lens={lens}", flush=True)
    o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                      d["cu_seqlens"])
    torch.cuda.synchronize()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], 128 ** -0.5)
    check_out(host(o, "bf16"), o_ref, "bf16")
    for sl in x["slot_idx"]:
        check_state(host(d["pool"], "f32")[sl], pool_ref[sl], "bf16", "f32")


def test_fused_qkv_strides():
    """q, k, v may be views into one fused [T, 2 HK DK + HV DV] buffer (the
    channel layout of the Mojo gated_delta module)."""
    gdr = _gdr()
    w = small_workload(128, "bf16", "scalar", "delta", "f32", False, seqlens=(70, 33))
    x = synth.generate(w)
    d = to_device(w, x)
    T = w.T_total
    kd, vd = w.HK * w.DK, w.HV * w.DV
    fused = torch.cat([d["q"].reshape(T, kd), d["k"].reshape(T, kd), d["v"].reshape(T, vd)], 1)
    q = fused[:, :kd].view(T, w.HK, w.DK)
    k = fused[:, kd:2 * kd].view(T, w.HK, w.DK)
    v = fused[:, 2 * kd:].view(T, w.HV, w.DV)
    pool2 = d["pool"].clone()
    o1 = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                       d["cu_seqlens"])
    o2 = gdr.chunk_fwd(q, k, v, d["g"], d["beta"], pool2, d["slot_idx"], d["cu_seqlens"])
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(d["pool"], pool2)


def test_debug_checks_reject_bad_indices():
    gdr = _gdr()
    w = small_workload(64, "bf16", "scalar", "delta", "f32", False, seqlens=(5, 6))
    x = synth.generate(w)
    d = to_device(w, x)
    bad = d["slot_idx"].clone()
    bad[1] = bad[0]
    with pytest.raises(gdr.GdrError) as e:
        gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], bad,
                      d["cu_seqlens"], debug_checks=True)
    assert e.value.status == 5
    cu = d["cu_seqlens"].clone()
    cu[1] = 9   # beyond cu[2] = 11? keep monotone break explicit
    cu[2] = 8
    with pytest.raises(gdr.GdrError):
        gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                      cu, debug_checks=True)
    # valid indices pass and compute
    gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                  d["cu_seqlens"], debug_checks=True)
    torch.cuda.synchronize()
