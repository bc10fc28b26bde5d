"""GPU parity of Gated DeltaProduct ("Linear attention visualized", section
"Gated Delta Product (GDP)": n_h transitions per token, the decay once before
the first, the query after the last) in the tokenwise kernels, against the
fp64 oracle's delta_product_fp64."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from helpers import check_out, check_state, dev, host, widened

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RAGGED = (0, 1, 11, 40, 7)


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


def product_inputs(w, P):
    """Seeded inputs: q, g, pool, slots, cu_seqlens per real token from w;
    k, v, beta with P rows per token from the same recipe at P times the
    lengths (another seed)."""
    xr = synth.generate(w)
    xv = synth.generate(w.replace(seqlens=tuple(P * n for n in w.seqlens), seed=w.seed + 1000))
    x = dict(xr)
    x["k"], x["v"], x["beta"] = xv["k"], xv["v"], xv["beta"]
    return x


def to_dev(w, x):
    return {
        "q": dev(x["q"], w.in_dtype), "k": dev(x["k"], w.in_dtype), "v": dev(x["v"], w.in_dtype),
        "g": dev(x["g"], "f32"), "beta": dev(x["beta"], "f32"),
        "pool": dev(x["pool"], w.state_dtype), "slot_idx": dev(x["slot_idx"], "i32"),
        "cu_seqlens": dev(x["cu_seqlens"], "i32"),
    }


def reference(w, x, P, scale, l2=False):
    xw = widened(w, x)
    if l2:
        xw["q"] = oracle.l2_normalise_fp64(xw["q"])
        xw["k"] = oracle.l2_normalise_fp64(xw["k"])
    return oracle.delta_product_fp64(
        xw["q"], xw["k"], xw["v"], xw["g"], xw["beta"], xw["pool"], x["slot_idx"],
        x["cu_seqlens"], products=P, scale=scale, rule=w.rule, gate=w.gate,
        zero_init=w.zero_init, state_dtype=w.state_dtype)


def small(D, in_dtype, gate, rule, state_dtype="f32", seqlens=RAGGED, seed=61):
    return synth.Workload(
        name="small", seqlens=tuple(seqlens), HK=2, HV=4, DK=D, DV=D, in_dtype=in_dtype,
        gate=gate, rule=rule, gate_shift=2.0 if gate != "channel" else 3.0,
        state_dtype=state_dtype, num_slots=7, zero_init=False, seed=seed)


COMBOS = [(P, D, i, g, r) for P, D, i, g, r in itertools.product(
    [2, 3], [64, 128], ["bf16", "f32"], ["none", "scalar", "channel"], ["delta", "linear"])
    if not (r == "linear" and g == "none" and P == 3)]


@pytest.mark.parametrize("P,D,in_dtype,gate,rule", COMBOS,
                         ids=[f"p{P}-d{D}-{i}-{g}-{r}" for P, D, i, g, r in COMBOS])
def test_recurrent_fwd_products_match_oracle(P, D, in_dtype, gate, rule):
    gdr = _gdr()
    state_dtype = "bf16" if (D == 128 and gate == "scalar") else "f32"
    w = small(D, in_dtype, gate, rule, state_dtype)
    x = product_inputs(w, P)
    d = to_dev(w, x)
    before = d["pool"].clone()
    print(f"recurrent_fwd products={P} D={D} in={in_dtype} gate={gate} rule={rule}", flush=True)
    o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"] if rule == "delta" else None,
                          d["pool"], d["slot_idx"], d["cu_seqlens"], scale=D ** -0.5, rule=rule,
                          gate=gate, products=P)
    torch.cuda.synchronize()
    o_ref, pool_ref = reference(w, x, P, D ** -0.5)
    check_out(host(o, in_dtype), o_ref, in_dtype)
    pool = host(d["pool"], state_dtype)
    for s in x["slot_idx"]:
        check_state(pool[s], pool_ref[s], in_dtype, state_dtype)
    untouched = np.setdiff1d(np.arange(w.num_slots), x["slot_idx"])
    assert torch.equal(d["pool"][untouched], before[untouched])


@pytest.mark.parametrize("P", [2, 4])
@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_recurrent_step_products_match_oracle(P, gate):
    """Six chained decode steps, each token with P transitions."""
    gdr = _gdr()
    steps = 6
    w = synth.Workload(name="dec", seqlens=(1,) * 5, HK=2, HV=4, DK=128, DV=128, in_dtype="bf16",
                       gate=gate, rule="delta", gate_shift=2.0, state_dtype="f32", num_slots=8,
                       zero_init=False, steps=steps, seed=71)
    x = product_inputs(w, P)
    d = to_dev(w, x)
    xw = widened(w, x)
    N = w.N
    pool_ref = xw["pool"]
    print(f"recurrent_step products={P} gate={gate}", flush=True)
    for s in range(steps):
        sq, sk = slice(s * N, (s + 1) * N), slice(s * N * P, (s + 1) * N * P)
        o = gdr.recurrent_step(d["q"][sq], d["k"][sk], d["v"][sk], d["g"][sq], d["beta"][sk],
                               d["pool"], d["slot_idx"], products=P)
        torch.cuda.synchronize()
        o_ref, pool_ref = oracle.delta_product_fp64(
            xw["q"][sq], xw["k"][sk], xw["v"][sk], xw["g"][sq], xw["beta"][sk], pool_ref,
            x["slot_idx"], np.arange(N + 1), products=P, scale=128 ** -0.5, gate=gate,
            state_dtype="f64")
        check_out(host(o, "f32"), o_ref, "bf16")
    pool = host(d["pool"], "f32")
    for sl in x["slot_idx"]:
        check_state(pool[sl], pool_ref[sl], "bf16", "f32")


def test_recurrent_fwd_products_with_l2norm():
    gdr = _gdr()
    P = 2
    w = small(128, "bf16", "scalar", "delta", seqlens=(9, 33, 0), seed=63)
    x = product_inputs(w, P)
    rng = np.random.default_rng(5)
    for name in ("q", "k"):
        raw = synth.widen(x[name], "bf16") * rng.uniform(0.3, 4.0, size=x[name].shape[:2] + (1,))
        x[name] = synth.f64_to_bf16_bits(raw)
    d = to_dev(w, x)
    o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                          d["cu_seqlens"], products=P, qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, pool_ref = reference(w, x, P, 128 ** -0.5, l2=True)
    check_out(host(o, "bf16"), o_ref, "bf16")
    for s in x["slot_idx"]:
        check_state(host(d["pool"], "f32")[s], pool_ref[s], "bf16", "f32")


def test_one_product_is_the_plain_recurrence():
    """products=1 is bit-identical to the call without it."""
    gdr = _gdr()
    w = small(128, "bf16", "scalar", "delta", seqlens=(50, 3))
    x = synth.generate(w)
    d = to_dev(w, x)
    p2 = d["pool"].clone()
    o1 = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                           d["cu_seqlens"])
    o2 = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], p2, d["slot_idx"],
                           d["cu_seqlens"], products=1)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(d["pool"], p2)


CHUNK_COMBOS = [
    # (P, D, in_dtype, gate, rule): the warp-specialised kernel (bf16, no or
    # scalar gate) and the general kernel (fp32 inputs, the channel gate)
    (2, 128, "bf16", "scalar", "delta"), (3, 128, "bf16", "scalar", "delta"),
    (3, 64, "bf16", "none", "delta"), (2, 128, "bf16", "scalar", "linear"),
    (3, 128, "bf16", "channel", "delta"), (2, 64, "bf16", "channel", "linear"),
    (3, 64, "f32", "scalar", "delta"), (2, 128, "f32", "channel", "delta"),
    (4, 128, "f32", "none", "linear"),
]


@pytest.mark.parametrize("P,D,in_dtype,gate,rule", CHUNK_COMBOS,
                         ids=[f"p{P}-d{D}-{i}-{g}-{r}" for P, D, i, g, r in CHUNK_COMBOS])
def test_chunk_fwd_products_match_oracle(P, D, in_dtype, gate, rule):
    """GDP as GDN over the virtual sequence of substeps, chunk by chunk (the
    page's construction), with tokens whose substeps straddle chunk ends."""
    gdr = _gdr()
    state_dtype = "bf16" if gate == "none" else "f32"
    w = small(D, in_dtype, gate, rule, state_dtype, seqlens=(0, 1, 40, 70, 129), seed=67)
    x = product_inputs(w, P)
    d = to_dev(w, x)
    before = d["pool"].clone()
    print(f"chunk_fwd products={P} D={D} in={in_dtype} gate={gate} rule={rule}", flush=True)
    o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"] if rule == "delta" else None,
                      d["pool"], d["slot_idx"], d["cu_seqlens"], scale=D ** -0.5, rule=rule,
                      gate=gate, products=P)
    torch.cuda.synchronize()
    o_ref, pool_ref = reference(w, x, P, D ** -0.5)
    check_out(host(o, "f32"), o_ref, in_dtype)
    pool = host(d["pool"], state_dtype)
    for s in x["slot_idx"]:
        check_state(pool[s], pool_ref[s], in_dtype, state_dtype)
    untouched = np.setdiff1d(np.arange(w.num_slots), x["slot_idx"])
    assert torch.equal(d["pool"][untouched], before[untouched])


@pytest.mark.parametrize("out_dtype", ["f32", "bf16"])
def test_chunk_fwd_products_equal_recurrent_fwd(out_dtype):
    gdr = _gdr()
    P = 2
    w = small(128, "bf16", "scalar", "delta", seqlens=(100, 33, 64), seed=69)
    x = product_inputs(w, P)
    d = to_dev(w, x)
    p2 = d["pool"].clone()
    od = torch.float32 if out_dtype == "f32" else torch.bfloat16
    o1 = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                       d["cu_seqlens"], products=P, out_dtype=od)
    o2 = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], p2, d["slot_idx"],
                           d["cu_seqlens"], products=P, out_dtype=od)
    torch.cuda.synchronize()
    a, b = host(o1, "f32"), host(o2, "f32")
    if out_dtype == "f32":
        check_out(a, b, "bf16")
    else:
        # each side rounds its fp32 result to bf16: two values that straddle
        # a rounding midpoint land one bf16 step (2^-7 of the value) apart
        r = np.sqrt(np.mean(b * b))
        assert np.all(np.abs(a - b) <= 2.0 ** -7 * np.abs(b) + 3e-3 * r)
    for s in x["slot_idx"]:
        check_state(host(d["pool"], "f32")[s], host(p2, "f32")[s], "bf16", "f32")


@pytest.mark.parametrize("HK,HV", [(1, 8), (3, 6)])
@pytest.mark.parametrize("entry", ["chunk_fwd", "recurrent_fwd"])
def test_products_head_layouts(HK, HV, entry):
    """Gated DeltaProduct (two transitions per token) with eight value heads
    per key head and with an odd number of key heads, on the warp-specialised
    prefill and the tokenwise recurrence."""
    gdr = _gdr()
    P, D = 2, 128
    w = synth.Workload(name="small", seqlens=(1, 40, 0, 97), HK=HK, HV=HV, DK=D, DV=D, in_dtype="bf16",
                       gate="scalar", rule="delta", gate_shift=2.0, state_dtype="f32", num_slots=6,
                       zero_init=False, seed=66 + HV)
    x = product_inputs(w, P)
    d = to_dev(w, x)
    print(f"{entry} products={P} HK={HK} HV={HV}", flush=True)
    o = getattr(gdr, entry)(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                            d["cu_seqlens"], scale=D ** -0.5, rule="delta", gate="scalar", products=P)
    torch.cuda.synchronize()
    o_ref, pool_ref = reference(w, x, P, D ** -0.5)
    check_out(host(o, "bf16"), o_ref, "bf16")
    pool = host(d["pool"], "f32")
    for s in x["slot_idx"]:
        check_state(pool[s], pool_ref[s], "bf16", "f32")
