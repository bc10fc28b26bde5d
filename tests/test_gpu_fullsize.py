"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times. The GPU computes every sequence and head; the fp64 oracle
recomputes a sample of (sequence, head) chains end to end and those outputs
and final states are compared under the same gate as the small tests."""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest

import synth
from helpers import check_out, check_state, host, to_device, widened
import oracle

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


def subset(w, x, heads):
    """Stored inputs of whole groups of value heads (and their key heads)."""
    heads = np.asarray(heads)
    ratio = w.HV // w.HK
    kh = np.unique(heads // ratio)
    assert ratio == 1 or len(heads) == len(kh) * ratio, "sample whole head groups"
    return dict(q=x["q"][:, kh], k=x["k"][:, kh], v=x["v"][:, heads],
                g=None if x["g"] is None else x["g"][:, heads],
                beta=None if x["beta"] is None else x["beta"][:, heads],
                pool=x["pool"][:, heads])


def run_prefill(gdr, w, d):
    o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                      d["cu_seqlens"], rule=w.rule, gate=w.gate, zero_init=w.zero_init,
                      chunk_size=w.chunk_size)
    torch.cuda.synchronize()
    return o


def check_sampled(w, x, o, pool_gpu, heads):
    xs = widened(w, subset(w, x, heads))
    o_ref, pool_ref = oracle.recurrent_fp64(
        xs["q"], xs["k"], xs["v"], xs["g"], xs["beta"], xs["pool"], x["slot_idx"],
        x["cu_seqlens"], scale=w.DK ** -0.5, rule=w.rule, gate=w.gate,
        zero_init=w.zero_init, state_dtype=w.state_dtype)
    og = host(o[:, torch.as_tensor(heads, device=o.device)], "f32")
    err, bound = check_out(og, o_ref, w.in_dtype)
    pg = host(pool_gpu, w.state_dtype)[:, heads]
    smargin = max(check_state(pg[s], pool_ref[s], w.in_dtype, w.state_dtype) for s in x["slot_idx"])
    print(f"MARGIN {w.name}: heads {list(heads)} o max|err| {err:.3e} <= {bound:.3e} "
          f"(err/bound {err / bound:.3f}); state max err/bound {smargin:.3f}", flush=True)


def test_gdr_fp32_t256_d64_all_outputs():
    gdr = _gdr()
    w = synth.workload("gdr_fp32_t256_h1_d64")
    x = synth.generate(w)
    d = to_device(w, x)
    print(f"launch {w.name}", flush=True)
    o = run_prefill(gdr, w, d)
    check_sampled(w, x, o, d["pool"], [0])


@pytest.mark.parametrize("name", ["gdn_prefill_b4_t4096_h16_d128", "la_prefill_b4_t4096_h16_d128"])
def test_gdn_prefill_b4_t4096_h16(name):
    gdr = _gdr()
    w = synth.workload(name)
    x = synth.generate(w)
    d = to_device(w, x)
    print(f"launch {w.name}", flush=True)
    o = run_prefill(gdr, w, d)
    assert torch.isfinite(o).all()
    check_sampled(w, x, o, d["pool"], [0, 9])


def test_ragged_gqa_prefill_bf16_pool():
    gdr = _gdr()
    w = synth.workload("ragged_gqa_prefill_n8_hk16_hv32_d128")
    x = synth.generate(w)
    d = to_device(w, x)
    pool0 = d["pool"].clone()
    print(f"launch {w.name} lens {w.seqlens}", flush=True)
    o = run_prefill(gdr, w, d)
    untouched = np.setdiff1d(np.arange(w.num_slots), x["slot_idx"])
    assert torch.equal(d["pool"][untouched], pool0[untouched])
    check_sampled(w, x, o, d["pool"], [0, 1, 30, 31])


def test_decode_n256_1000_steps():
    """The decode workload as bench.py times it: 1000 consecutive steps over the
    256-sequence fp32 pool, step s feeding token set s mod 64 (64 distinct
    sets of one new token per sequence). The full batch is checked against the
    oracle at each of the first 8 steps (every output) and after step 8 (every
    slot); a 16-sequence subset is followed for all 1000 steps (its outputs at
    every step and its final states), the oracle running each of its
    sequences as one 1000-token recurrence."""
    gdr = _gdr()
    w = synth.workload("decode_n256_hk16_hv32_d128")
    distinct, steps, full = 64, 1000, 8
    ws = w.replace(steps=distinct)
    x = synth.generate(ws)
    d = to_device(ws, x)
    xw = widened(ws, x)
    N = w.N
    sample = np.arange(0, N, 16)
    samp_t = torch.as_tensor(sample, device="cuda")
    outs_full = []
    outs_sample = torch.empty((steps, len(sample), w.HV, w.DV), dtype=torch.float32, device="cuda")
    pool_full = None
    print(f"launch {w.name}: {steps} steps", flush=True)
    for s in range(steps):
        sl = slice((s % distinct) * N, (s % distinct + 1) * N)
        o = gdr.recurrent_step(d["q"][sl], d["k"][sl], d["v"][sl], d["g"][sl], d["beta"][sl],
                               d["pool"], d["slot_idx"])
        outs_sample[s] = o[samp_t]
        if s < full:
            outs_full.append(o.clone())
        if s == full - 1:
            pool_full = d["pool"].clone()
    torch.cuda.synchronize()

    # Oracle runs split by sequence (each sequence's recurrence is separate)
    # over host threads; sequence n's state sits at local slot n.
    slots = x["slot_idx"]
    groups = np.array_split(np.arange(N), 16)

    def run_group(rows_of, grp, pool_grp, T):
        rows = np.concatenate([rows_of(n) for n in grp])
        return oracle.recurrent_fp64(
            xw["q"][rows], xw["k"][rows], xw["v"][rows], xw["g"][rows], xw["beta"][rows], pool_grp,
            np.arange(len(grp)), np.arange(len(grp) + 1) * T, scale=w.DK ** -0.5)

    # full batch, steps 1..8 (the pool holds fp32 after every step)
    pool_ref = xw["pool"][slots]
    worst = 0.0
    with ThreadPoolExecutor(16) as ex:
        for s in range(full):
            res = list(ex.map(lambda grp: run_group(lambda n: [s * N + n], grp, pool_ref[grp], 1), groups))
            o_ref = np.concatenate([r[0] for r in res])
            pool_ref = np.concatenate([r[1] for r in res])
            err, bound = check_out(host(outs_full[s], "f32"), o_ref, "bf16")
            worst = max(worst, err / bound)
        smargin = check_state(host(pool_full, "f32")[slots], pool_ref, "bf16", "f32")
        print(f"MARGIN {w.name} full batch steps 1-{full}: o max err/bound {worst:.3f}; "
              f"state (all {N} slots) err/bound {smargin:.3f}", flush=True)

        # the subset for all 1000 steps: sequence n sees token (s mod 64) * N + n
        # at step s, so each is one 1000-token recurrence
        pool0 = xw["pool"][slots]
        res = list(ex.map(lambda n: run_group(lambda m: (np.arange(steps) % distinct) * N + m, [n],
                                              pool0[[n]], steps), sample))
    o_ref = np.stack([r[0] for r in res], axis=1)           # [steps, 16, HV, DV]
    pool_sub = np.concatenate([r[1] for r in res])
    err, bound = check_out(host(outs_sample, "f32"), o_ref, "bf16")
    smargin = check_state(host(d["pool"], "f32")[slots[sample]], pool_sub, "bf16", "f32")
    print(f"MARGIN {w.name} {len(sample)} sequences x {steps} steps: o max|err| {err:.3e} <= {bound:.3e} "
          f"(err/bound {err / bound:.3f}); final state err/bound {smargin:.3f}", flush=True)


def test_kda_prefill_t131072_h32():
    gdr = _gdr()
    w = synth.workload("kda_prefill_t131072_h32_d128")
    x = synth.generate(w)
    d = to_device(w, x)
    print(f"launch {w.name}", flush=True)
    o = run_prefill(gdr, w, d)
    assert torch.isfinite(o).all()
    check_sampled(w, x, o, d["pool"], [5])


@pytest.mark.parametrize("name", ["gla_prefill_t131072_h32_d128", "mamba2_prefill_b4_t4096_h16_d128"])
def test_gated_linear_prefill(name):
    """The gated linear variants at the sizes bench.py --workload times: GLA
    (channel gate, through the KDA kernel pair with T' = I, W = 0) and the
    scalar-gated linear rule (Mamba-2; RetNet with a constant gate)."""
    gdr = _gdr()
    w = synth.workload(name)
    x = synth.generate(w)
    d = to_device(w, x)
    print(f"launch {w.name}", flush=True)
    o = run_prefill(gdr, w, d)
    assert torch.isfinite(o).all()
    check_sampled(w, x, o, d["pool"], [3] if w.N == 1 else [0, 11])


def test_short_prefill_n256_t16_recurrent_fwd():
    """The tokenwise schedule on the benchmark's short-prefill batch (256
    sequences of 16 tokens over the fp32 decode pool): two whole head groups
    recomputed by the oracle for every sequence; the chunkwise prefill on the
    same batch agrees with it."""
    gdr = _gdr()
    w = synth.workload("short_prefill_n256_t16_hk16_hv32_d128")
    x = synth.generate(w)
    d = to_device(w, x)
    pool2 = d["pool"].clone()
    print(f"launch {w.name} recurrent_fwd", flush=True)
    o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                          d["cu_seqlens"], rule=w.rule, gate=w.gate, zero_init=w.zero_init)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    check_sampled(w, x, o, d["pool"], [0, 1, 30, 31])
    print(f"launch {w.name} chunk_fwd", flush=True)
    o2 = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], pool2, d["slot_idx"],
                       d["cu_seqlens"], rule=w.rule, gate=w.gate, zero_init=w.zero_init)
    torch.cuda.synchronize()
    check_out(host(o, "f32"), host(o2, "f32"), w.in_dtype)
