"""GPU parity of gdr_linear_chunk_bwd and gdr_gated_linear_chunk_bwd
(gradients of causal linear attention, plain or with a scalar gate, "From
Attention to Learned Memory", section "Backward: reverse the boundary scan,
then differentiate each chunk") against the fp64 oracle: its chunk-free
linear_attention_grads_fp64 for the plain rule with one value head per key
head, and its tokenwise recurrent_grads_fp64 (reverse mode through the
recurrence, pinned separately) for gates and grouped key heads.

Tolerance: as the forward outputs for the plain rule; for the gated and
grouped cases fp32 inputs max|err| <= 1e-4 * max(1, RMS of the reference)
(the gradients, dg above all, sum over up to a few hundred tokens, so their
scale grows past 1) and bf16 inputs 3e-3 * RMS."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from helpers import check_out, dev, host, rms

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RAGGED = (0, 1, 63, 64, 65, 130, 200)


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


def inputs(w):
    """Seeded q, k, v, pool of the workload and an upstream gradient dO drawn
    like v (another seed)."""
    x = synth.generate(w)
    x["do"] = synth.generate(w.replace(seed=w.seed + 500))["v"]
    return x


def run(gdr, w, x, out_dtype=torch.float32):
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v", "do")}
    pool = dev(x["pool"], w.state_dtype)
    before = pool.clone()
    g = gdr.linear_chunk_bwd(d["q"], d["k"], d["v"], d["do"], pool, dev(x["slot_idx"], "i32"),
                             dev(x["cu_seqlens"], "i32"), zero_init=w.zero_init, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(pool, before), "the backward must not write the pool"
    return g


def reference(w, x, heads=None):
    wid = lambda n: synth.widen(x[n], w.in_dtype)
    q, k, v, do = wid("q"), wid("k"), wid("v"), wid("do")
    pool = synth.widen(x["pool"], w.state_dtype)
    if heads is not None:
        q, k, v, do, pool = q[:, heads], k[:, heads], v[:, heads], do[:, heads], pool[:, heads]
    return oracle.linear_attention_grads_fp64(q, k, v, do, pool, x["slot_idx"], x["cu_seqlens"],
                                              scale=w.DK ** -0.5, zero_init=w.zero_init)


def small(D, in_dtype, zero_init, state_dtype="f32", seqlens=RAGGED, seed=81):
    return synth.Workload(name="small", seqlens=tuple(seqlens), HK=3, HV=3, DK=D, DV=D,
                          in_dtype=in_dtype, gate="none", rule="linear", gate_shift=2.0,
                          state_dtype=state_dtype, num_slots=9, zero_init=zero_init, seed=seed)


COMBOS = list(itertools.product([64, 128], ["bf16", "f32"], [True, False]))


@pytest.mark.parametrize("D,in_dtype,zero_init", COMBOS,
                         ids=[f"d{D}-{i}-{'zero' if z else 'pool'}" for D, i, z in COMBOS])
def test_linear_backward_matches_oracle(D, in_dtype, zero_init):
    gdr = _gdr()
    w = small(D, in_dtype, zero_init, state_dtype="bf16" if D == 64 else "f32")
    x = inputs(w)
    print(f"linear_chunk_bwd D={D} in={in_dtype} zero_init={zero_init} lens={RAGGED}", flush=True)
    dq, dk, dv = run(gdr, w, x)
    ref = reference(w, x)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_out(host(got, "f32"), want, in_dtype, what=name)


def test_linear_backward_bf16_gradients():
    gdr = _gdr()
    w = small(128, "bf16", False, seqlens=(100, 7, 64))
    x = inputs(w)
    got = run(gdr, w, x, out_dtype=torch.bfloat16)
    for g, want in zip(got, reference(w, x)):
        a = host(g, "bf16")
        r = np.sqrt(np.mean(want ** 2))
        assert np.all(np.abs(a - want) <= 2.0 ** -8 * np.abs(want) + 3e-3 * r)


def test_linear_backward_full_size_headline_shapes():
    """The linear-attention shapes of the prefill benchmark (4 x 4096 tokens,
    16 heads, d = 128), two heads recomputed by the oracle."""
    gdr = _gdr()
    w = synth.workload("la_prefill_b4_t4096_h16_d128")
    x = inputs(w)
    print(f"launch {w.name} backward", flush=True)
    dq, dk, dv = run(gdr, w, x)
    assert all(torch.isfinite(t).all() for t in (dq, dk, dv))
    heads = [0, 9]
    ref = reference(w, x, heads)
    hh = torch.as_tensor(heads, device=dq.device)
    for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
        check_out(host(got[:, hh], "f32"), want, "bf16", what=name)


def test_linear_backward_on_fused_qkv_views():
    """q, k, v as views into one fused [T, 3 H D] buffer (token strides of
    3 H D): the gradients equal those from separate contiguous tensors."""
    gdr = _gdr()
    w = small(128, "bf16", False, seqlens=(90, 0, 33, 130), seed=83)
    x = inputs(w)
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v", "do")}
    pool = dev(x["pool"], w.state_dtype)
    slot, cu = dev(x["slot_idx"], "i32"), dev(x["cu_seqlens"], "i32")
    T, HD = w.T_total, w.HK * w.DK
    fused = torch.cat([d["q"].reshape(T, HD), d["k"].reshape(T, HD), d["v"].reshape(T, HD)], 1)
    q, k, v = (fused[:, i * HD:(i + 1) * HD].view(T, w.HK, w.DK) for i in range(3))
    a = gdr.linear_chunk_bwd(d["q"], d["k"], d["v"], d["do"], pool, slot, cu)
    b = gdr.linear_chunk_bwd(q, k, v, d["do"], pool, slot, cu)
    torch.cuda.synchronize()
    for ga, gb in zip(a, b):
        assert torch.equal(ga, gb)


# --- scalar gate and grouped key heads ---------------------------------------

def check(got, want, in_dtype, what):
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    r = rms(want)
    bound = 1e-4 * max(1.0, r) if in_dtype == "f32" else 3e-3 * r
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= bound, f"{what}: max|err| {err:.3e} > {bound:.3e} (rms {r:.3e})"


def run_gated(gdr, w, x, out_dtype=torch.float32):
    """(dq, dk, dv, dg | None) as host fp32 arrays."""
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v", "do")}
    pool = dev(x["pool"], w.state_dtype)
    before = pool.clone()
    g = dev(x["g"], "f32") if w.gate == "scalar" else None
    out = gdr.linear_chunk_bwd(d["q"], d["k"], d["v"], d["do"], pool, dev(x["slot_idx"], "i32"),
                               dev(x["cu_seqlens"], "i32"), g=g, zero_init=w.zero_init, out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert torch.equal(pool, before), "the backward must not write the pool"
    assert len(out) == (4 if g is not None else 3)
    res = [host(t, "f32") for t in out]
    return res + [None] * (4 - len(res))


def reference_rec(w, x, kheads=None, seqs=None):
    """Oracle gradients through the tokenwise recurrence; kheads keeps whole
    key-head groups (their value heads), seqs a subset of the sequences."""
    wid = lambda n: synth.widen(x[n], w.in_dtype)
    q, k, v, do = wid("q"), wid("k"), wid("v"), wid("do")
    pool = synth.widen(x["pool"], w.state_dtype)
    g = x["g"] if w.gate == "scalar" else None
    cu, slots = x["cu_seqlens"], x["slot_idx"]
    if kheads is not None:
        G = w.HV // w.HK
        vh = [hk * G + j for hk in kheads for j in range(G)]
        q, k, v, do, pool = q[:, kheads], k[:, kheads], v[:, vh], do[:, vh], pool[:, vh]
        g = None if g is None else g[:, vh]
    if seqs is not None:
        rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs])
        q, k, v, do = q[rows], k[rows], v[rows], do[rows]
        g = None if g is None else g[rows]
        cu = np.concatenate([[0], np.cumsum([cu[n + 1] - cu[n] for n in seqs])])
        slots = slots[list(seqs)]
    r = oracle.recurrent_grads_fp64(q, k, v, g, None, do, pool, slots, cu, scale=w.DK ** -0.5,
                                    rule="linear", gate=w.gate, zero_init=w.zero_init)
    return [r["dq"], r["dk"], r["dv"], r["dg"]]


def small_gated(D, in_dtype, gate, HK, HV, zero_init=False, seqlens=RAGGED, seed=87):
    return synth.Workload(name="small", seqlens=tuple(seqlens), HK=HK, HV=HV, DK=D, DV=D,
                          in_dtype=in_dtype, gate=gate, rule="linear", gate_shift=2.0,
                          state_dtype="bf16" if D == 64 else "f32", num_slots=9, zero_init=zero_init,
                          seed=seed)


HEADS = [("scalar", 3, 3), ("scalar", 2, 4), ("none", 2, 4)]
GCOMBOS = [(D, i, gt, hk, hv) for D in (64, 128) for i in ("bf16", "f32") for gt, hk, hv in HEADS]


@pytest.mark.parametrize("D,in_dtype,gate,HK,HV", GCOMBOS,
                         ids=[f"d{D}-{i}-{g}-hk{hk}-hv{hv}" for D, i, g, hk, hv in GCOMBOS])
def test_gated_grouped_linear_backward_matches_oracle(D, in_dtype, gate, HK, HV):
    gdr = _gdr()
    w = small_gated(D, in_dtype, gate, HK, HV)
    x = inputs(w)
    print(f"linear_chunk_bwd D={D} in={in_dtype} gate={gate} HK={HK} HV={HV} lens={RAGGED}", flush=True)
    got = run_gated(gdr, w, x)
    for name, a, b in zip(("dq", "dk", "dv", "dg"), got, reference_rec(w, x)):
        if b is None:
            assert a is None
            continue
        check(a, b, in_dtype, name)


@pytest.mark.parametrize("in_dtype", ["bf16", "f32"])
def test_gated_linear_backward_zero_init(in_dtype):
    gdr = _gdr()
    w = small_gated(128, in_dtype, "scalar", 2, 4, zero_init=True, seqlens=(70, 0, 129), seed=88)
    x = inputs(w)
    print(f"gated linear_chunk_bwd zero_init in={in_dtype}", flush=True)
    for name, a, b in zip(("dq", "dk", "dv", "dg"), run_gated(gdr, w, x), reference_rec(w, x)):
        check(a, b, in_dtype, name)


def test_gated_linear_backward_bf16_gradients():
    gdr = _gdr()
    w = small_gated(128, "bf16", "scalar", 2, 4, seqlens=(100, 7, 64), seed=89)
    x = inputs(w)
    print("gated linear_chunk_bwd bf16 gradients", flush=True)
    got = run_gated(gdr, w, x, out_dtype=torch.bfloat16)
    ref = reference_rec(w, x)
    for name, a, want in zip(("dq", "dk", "dv"), got, ref):
        r = np.sqrt(np.mean(want ** 2))
        assert np.all(np.abs(a - want) <= 2.0 ** -8 * np.abs(want) + 3e-3 * r), name
    check(got[3], ref[3], "bf16", "dg")   # dg stays fp32


def test_gated_linear_backward_on_fused_qkv_views():
    """Gated and grouped, with q, k, v as views into one fused buffer: the
    gradients equal those from separate contiguous tensors."""
    gdr = _gdr()
    w = small_gated(128, "bf16", "scalar", 2, 2, seqlens=(90, 0, 33, 130), seed=90)
    x = inputs(w)
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v", "do")}
    pool = dev(x["pool"], w.state_dtype)
    g = dev(x["g"], "f32")
    slot, cu = dev(x["slot_idx"], "i32"), dev(x["cu_seqlens"], "i32")
    T, HD = w.T_total, w.HK * w.DK
    fused = torch.cat([d["q"].reshape(T, HD), d["k"].reshape(T, HD), d["v"].reshape(T, HD)], 1)
    q, k, v = (fused[:, i * HD:(i + 1) * HD].view(T, w.HK, w.DK) for i in range(3))
    print("gated linear_chunk_bwd on fused views", flush=True)
    a = gdr.linear_chunk_bwd(d["q"], d["k"], d["v"], d["do"], pool, slot, cu, g=g)
    b = gdr.linear_chunk_bwd(q, k, v, d["do"], pool, slot, cu, g=g)
    torch.cuda.synchronize()
    for ga, gb in zip(a, b):
        assert torch.equal(ga, gb)


def test_gated_linear_backward_full_size_headline_shapes():
    """The gated prefill benchmark's shapes (4 x 4096 tokens, 16 heads,
    d = 128) under the linear rule; two heads of one sequence recomputed by
    the oracle."""
    gdr = _gdr()
    w = synth.workload("gdn_prefill_b4_t4096_h16_d128").replace(rule="linear")
    x = inputs(w)
    print(f"launch {w.name} gated linear backward", flush=True)
    got = run_gated(gdr, w, x)
    heads, seqs = [0, 9], [2]
    cu = x["cu_seqlens"]
    rows = np.arange(cu[2], cu[3])
    for name, a, b in zip(("dq", "dk", "dv", "dg"), got, reference_rec(w, x, heads, seqs)):
        check(a[rows][:, heads], b, "bf16", name)


def test_gated_linear_backward_full_size_ragged_grouped():
    """The ragged grouped-head prefill's shapes (8 sequences of 512 to 16384
    tokens, 16 key and 32 value heads, a bf16 pool) under the linear rule;
    one key-head group of the shortest sequence recomputed by the oracle."""
    gdr = _gdr()
    w = synth.workload("ragged_gqa_prefill_n8_hk16_hv32_d128").replace(rule="linear")
    x = inputs(w)
    print(f"launch {w.name} gated linear backward", flush=True)
    got = run_gated(gdr, w, x)
    cu = x["cu_seqlens"]
    n = int(np.argmin(np.diff(cu)))
    rows = np.arange(cu[n], cu[n + 1])
    kh = [5]
    G = w.HV // w.HK
    vh = [kh[0] * G + j for j in range(G)]
    ref = reference_rec(w, x, kh, [n])
    for name, a, b, hh in zip(("dq", "dk", "dv", "dg"), got, ref, (kh, kh, vh, vh)):
        check(a[rows][:, hh], b, "bf16", name)


LDEGEN = list(itertools.product(["zero_k", "forget", "zero_g"], ["bf16", "f32"]))


@pytest.mark.parametrize("kind,in_dtype", LDEGEN, ids=["-".join(c) for c in LDEGEN])
def test_gated_linear_backward_degenerate_cases(kind, in_dtype):
    """The gated linear backward (scalar gate, grouped key heads) on zero keys
    for every other token, complete forgetting (log-decay -60 per token) and a
    gate of exactly zero. Under complete forgetting the exact dg is of order
    e^{-60} times the other gradients, while the kernels form it as
    q.dq - k.dk (a difference of terms of the gradients' own scale, summed
    over the tokens after it): it is checked against fp32's absolute bound at
    that scale, 1e-4 times the scale of dk."""
    gdr = _gdr()
    w = small_gated(128, in_dtype, "scalar", 2, 4, seed=88)
    x = inputs(w)
    if kind == "zero_k":
        k = np.array(x["k"], copy=True)
        k[::2] = 0
        x["k"] = k
    else:
        x["g"] = np.full_like(x["g"], -60.0 if kind == "forget" else 0.0)
    print(f"linear_chunk_bwd degenerate {kind} in={in_dtype}", flush=True)
    got = run_gated(gdr, w, x)
    ref = reference_rec(w, x)
    for name, a, b in zip(("dq", "dk", "dv", "dg"), got, ref):
        if name == "dg" and kind == "forget":
            assert np.all(np.isfinite(a))
            assert float(np.max(np.abs(a - b))) <= 1e-4 * max(1.0, rms(ref[1]))
            continue
        check(a, b, in_dtype, name)
