"""GPU parity of gdr_chunk_bwd (the chunkwise gradients of the gated delta
rule, gate none or scalar: the boundary scan of "From Attention to Learned
Memory", section "Backward: reverse the boundary scan, then differentiate each
chunk", over the chunk equations of "You Could Have Come Up With Kimi Delta
Attention", section 6) against the fp64 oracle's recurrent_grads_fp64 (the
tokenwise recurrence differentiated, pinned by finite differences of the
forward oracle).

Tolerance as for the tokenwise backward: fp32 inputs max|err| <= 1e-4 *
max(1, RMS of the reference), bf16 inputs 3e-3 * RMS (the oracle widens the
same rounded inputs; the kernels compute in fp32)."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from helpers import dev, host, rms

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RAGGED = (0, 1, 63, 64, 65, 130, 7)   # empty, one token, either side of a chunk, two chunks + 2


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


def check(got, want, in_dtype, what):
    err = float(np.max(np.abs(got - want))) if want.size else 0.0
    r = rms(want)
    bound = 1e-4 * max(1.0, r) if in_dtype == "f32" else 3e-3 * r
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    assert err <= bound, f"{what}: max|err| {err:.3e} > {bound:.3e} (rms {r:.3e})"
    return err / bound if bound else 0.0


def inputs(w):
    x = synth.generate(w)
    x["do"] = synth.generate(w.replace(seed=w.seed + 500))["v"]
    return x


def run(gdr, w, x, fn="chunk_bwd", out_dtype=torch.float32, **kw):
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v", "do")}
    pool = dev(x["pool"], w.state_dtype)
    before = pool.clone()
    g = dev(x["g"], "f32") if w.gate != "none" else None
    beta = dev(x["beta"], "f32")
    out = getattr(gdr, fn)(d["q"], d["k"], d["v"], g, beta, d["do"], pool, dev(x["slot_idx"], "i32"),
                           dev(x["cu_seqlens"], "i32"), gate=w.gate, zero_init=w.zero_init, out_dtype=out_dtype,
                           **kw)
    torch.cuda.synchronize()
    assert torch.equal(pool, before), "the backward must not write the pool"
    return {n: None if t is None else host(t, "f32") for n, t in out.items()}


def reference(w, x, kheads=None, seqs=None):
    """Oracle gradients; kheads keeps whole key-head groups (their value
    heads), seqs a subset of the sequences."""
    wid = lambda n: synth.widen(x[n], w.in_dtype)
    q, k, v, do = wid("q"), wid("k"), wid("v"), wid("do")
    pool = synth.widen(x["pool"], w.state_dtype)
    g = x["g"] if w.gate != "none" else None
    beta = x["beta"]
    cu, slots = x["cu_seqlens"], x["slot_idx"]
    if kheads is not None:
        G = w.HV // w.HK
        vh = [hk * G + j for hk in kheads for j in range(G)]
        q, k, v, do, pool, beta = q[:, kheads], k[:, kheads], v[:, vh], do[:, vh], pool[:, vh], beta[:, vh]
        g = None if g is None else g[:, vh]
    if seqs is not None:
        rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs])
        q, k, v, do, beta = q[rows], k[rows], v[rows], do[rows], beta[rows]
        g = None if g is None else g[rows]
        cu = np.concatenate([[0], np.cumsum([cu[n + 1] - cu[n] for n in seqs])])
        slots = slots[list(seqs)]
    return oracle.recurrent_grads_fp64(q, k, v, g, beta, do, pool, slots, cu, scale=w.DK ** -0.5,
                                       rule="delta", gate=w.gate, zero_init=w.zero_init)


def small(D, in_dtype, gate, zero_init=False, HK=2, HV=4, seqlens=RAGGED, seed=95, gate_shift=2.0):
    return synth.Workload(name="small", seqlens=tuple(seqlens), HK=HK, HV=HV, DK=D, DV=D,
                          in_dtype=in_dtype, gate=gate, rule="delta", gate_shift=gate_shift,
                          state_dtype="bf16" if D == 64 else "f32", num_slots=11, zero_init=zero_init, seed=seed)


NAMES = ("dq", "dk", "dv", "dbeta", "dg", "dstate0")


def compare(got, ref, w, names=NAMES):
    for n in names:
        if ref[n] is None:
            assert got[n] is None, n
            continue
        check(got[n], ref[n], w.in_dtype, n)


COMBOS = list(itertools.product([64, 128], ["bf16", "f32"], ["none", "scalar"]))


@pytest.mark.parametrize("D,in_dtype,gate", COMBOS, ids=[f"d{D}-{i}-{g}" for D, i, g in COMBOS])
def test_chunk_bwd_matches_oracle(D, in_dtype, gate):
    gdr = _gdr()
    w = small(D, in_dtype, gate)
    x = inputs(w)
    print(f"chunk_bwd D={D} in={in_dtype} gate={gate} lens={RAGGED}", flush=True)
    compare(run(gdr, w, x), reference(w, x), w)


@pytest.mark.parametrize("gate", ["none", "scalar"])
def test_chunk_bwd_zero_init_and_one_head_group(gate):
    gdr = _gdr()
    w = small(128, "f32", gate, zero_init=True, HK=3, HV=3, seqlens=(129, 0, 64), seed=96)
    x = inputs(w)
    print(f"chunk_bwd zero_init HK=HV=3 gate={gate}", flush=True)
    compare(run(gdr, w, x), reference(w, x), w)


def test_chunk_bwd_four_value_heads_per_key_head():
    gdr = _gdr()
    w = small(64, "bf16", "scalar", HK=1, HV=4, seqlens=(150, 64, 1), seed=94)
    x = inputs(w)
    print("chunk_bwd HK=1 HV=4", flush=True)
    compare(run(gdr, w, x), reference(w, x), w)


def test_chunk_bwd_all_sequences_empty():
    """Sequences of no tokens: nothing to differentiate but the initial
    states, whose gradient is zero (the final state's is taken as zero)."""
    gdr = _gdr()
    w = small(128, "bf16", "scalar", seqlens=(0, 0, 0), seed=92)
    x = inputs(w)
    print("chunk_bwd empty batch", flush=True)
    got = run(gdr, w, x)
    assert got["dq"].shape[0] == 0 and got["dv"].shape[0] == 0
    assert np.array_equal(got["dstate0"], np.zeros_like(got["dstate0"]))


def test_chunk_bwd_with_debug_checks():
    """GDR_FLAG_DEBUG_CHECKS validates the index arrays on the device first;
    the gradients are unchanged."""
    gdr = _gdr()
    w = small(64, "bf16", "scalar", seed=91)
    x = inputs(w)
    print("chunk_bwd debug checks", flush=True)
    a, b = run(gdr, w, x), run(gdr, w, x, debug_checks=True)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


def test_chunk_bwd_strong_gate():
    """A strong decay (g = -softplus(x + 2): about -2.1 per token, spans of
    -130 over a chunk): every factor stays an exponential of a non-positive
    number."""
    gdr = _gdr()
    w = small(128, "f32", "scalar", seqlens=(100, 64, 3), seed=97, gate_shift=-2.0)
    x = inputs(w)
    print("chunk_bwd strong gate", flush=True)
    compare(run(gdr, w, x), reference(w, x), w)


@pytest.mark.parametrize("HK,HV", [(2, 4), (3, 3)])
def test_chunk_bwd_bf16_gradients_and_no_dstate(HK, HV):
    """bf16 dq, dk, dv: summed over each key head's group (HV > HK) or
    written by the gradient kernel itself (HV == HK)."""
    gdr = _gdr()
    w = small(128, "bf16", "scalar", HK=HK, HV=HV, seqlens=(33, 5, 64), seed=98)
    x = inputs(w)
    print(f"chunk_bwd bf16 gradients, dstate0 off, HK={HK} HV={HV}", flush=True)
    got = run(gdr, w, x, out_dtype=torch.bfloat16, dstate0=False)
    assert got["dstate0"] is None
    ref = reference(w, x)
    for n in ("dq", "dk", "dv"):
        want = ref[n]
        assert np.all(np.abs(got[n] - want) <= 2.0 ** -8 * np.abs(want) + 3e-3 * rms(want)), n
    compare(got, ref, w, names=("dbeta", "dg"))


def test_chunk_bwd_is_deterministic():
    """Two calls give bit-identical gradients (no summation order depends on
    which wave finishes first)."""
    gdr = _gdr()
    w = small(128, "bf16", "scalar", seed=93)
    x = inputs(w)
    print("chunk_bwd twice", flush=True)
    a, b = run(gdr, w, x), run(gdr, w, x)
    for n in NAMES:
        assert np.array_equal(a[n], b[n]), n


def test_chunk_bwd_on_fused_qkv_views():
    """q, k, v as views into one fused [T, (2 HK + HV) D] buffer: the same
    gradients, bit for bit, as from contiguous tensors."""
    gdr = _gdr()
    w = small(128, "bf16", "scalar", seqlens=(90, 0, 33, 130), seed=90)
    x = inputs(w)
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v", "do")}
    pool = dev(x["pool"], w.state_dtype)
    g, beta = dev(x["g"], "f32"), dev(x["beta"], "f32")
    slot, cu = dev(x["slot_idx"], "i32"), dev(x["cu_seqlens"], "i32")
    T, KD, VD = w.T_total, w.HK * w.DK, w.HV * w.DV
    fused = torch.cat([d["q"].reshape(T, KD), d["k"].reshape(T, KD), d["v"].reshape(T, VD)], 1)
    q = fused[:, :KD].view(T, w.HK, w.DK)
    k = fused[:, KD:2 * KD].view(T, w.HK, w.DK)
    v = fused[:, 2 * KD:].view(T, w.HV, w.DV)
    print("chunk_bwd on fused views", flush=True)
    a = gdr.chunk_bwd(d["q"], d["k"], d["v"], g, beta, d["do"], pool, slot, cu, gate="scalar")
    b = gdr.chunk_bwd(q, k, v, g, beta, d["do"], pool, slot, cu, gate="scalar")
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(a[n], b[n]), n


def test_chunk_bwd_agrees_with_tokenwise():
    """Both backwards of the same call, fp32 inputs: equal to fp32
    rounding."""
    gdr = _gdr()
    w = small(64, "f32", "scalar", seed=99)
    x = inputs(w)
    print("chunk_bwd vs recurrent_bwd", flush=True)
    a, b = run(gdr, w, x), run(gdr, w, x, fn="recurrent_bwd")
    for n in NAMES:
        assert np.max(np.abs(a[n] - b[n])) <= 2e-4 * max(1.0, rms(b[n])), n


def test_chunk_bwd_full_size_gdn_shapes():
    """The Gated DeltaNet prefill's shapes (4 x 4096 tokens, 16 heads,
    d = 128); two heads of one sequence recomputed by the oracle."""
    gdr = _gdr()
    w = synth.workload("gdn_prefill_b4_t4096_h16_d128")
    x = inputs(w)
    print(f"launch {w.name} chunk_bwd", flush=True)
    got = run(gdr, w, x)
    heads, n = [3, 12], 1
    cu = x["cu_seqlens"]
    rows = np.arange(cu[n], cu[n + 1])
    ref = reference(w, x, heads, [n])
    for name in ("dq", "dk", "dv", "dbeta", "dg"):
        check(got[name][rows][:, heads], ref[name], "bf16", name)
    check(got["dstate0"][n][heads], ref["dstate0"][0], "bf16", "dstate0")


def test_chunk_bwd_full_size_ragged_grouped():
    """The ragged grouped-head prefill's shapes (8 sequences, 16 key and 32
    value heads, bf16 pool); one key-head group of the shortest sequence
    recomputed by the oracle."""
    gdr = _gdr()
    w = synth.workload("ragged_gqa_prefill_n8_hk16_hv32_d128")
    x = inputs(w)
    print(f"launch {w.name} chunk_bwd", flush=True)
    got = run(gdr, w, x)
    cu = x["cu_seqlens"]
    n = int(np.argmin(np.diff(cu)))
    rows = np.arange(cu[n], cu[n + 1])
    kh = [7]
    G = w.HV // w.HK
    vh = [kh[0] * G + j for j in range(G)]
    ref = reference(w, x, kh, [n])
    for name, hh in (("dq", kh), ("dk", kh), ("dv", vh), ("dbeta", vh), ("dg", vh)):
        check(got[name][rows][:, hh], ref[name], "bf16", name)
    check(got["dstate0"][n][vh], ref["dstate0"][0], "bf16", "dstate0")


def _degenerate(x, kind):
    """Inputs with one degenerate feature of the update imposed: beta = 0 (no
    write: dv is exactly zero), beta = 1, zero keys on every other token,
    complete forgetting (log-decay -60 per token) or a gate of exactly zero."""
    x = dict(x)
    if kind == "beta0":
        x["beta"] = np.zeros_like(x["beta"])
    elif kind == "beta1":
        x["beta"] = np.ones_like(x["beta"])
    elif kind == "zero_k":
        k = np.array(x["k"], copy=True)
        k[::2] = 0
        x["k"] = k
    elif kind == "forget":
        x["g"] = np.full_like(x["g"], -60.0)
    elif kind == "zero_g":
        x["g"] = np.zeros_like(x["g"])
    return x


DEGEN = list(itertools.product(["beta0", "beta1", "zero_k", "forget", "zero_g"], ["bf16", "f32"],
                               ["chunk_bwd", "recurrent_bwd"]))


@pytest.mark.parametrize("kind,in_dtype,fn", DEGEN, ids=["-".join(c) for c in DEGEN])
def test_backward_degenerate_cases(kind, in_dtype, fn):
    """Both delta-rule backwards on the update's degenerate cases (scalar
    gate, ragged grouped batch). Under complete forgetting the log-decays'
    and the initial states' gradients are of order e^{-60} times the others:
    they are checked against an absolute bound of 1e-6 times the scale of the
    key gradients, below which fp32 cannot resolve them."""
    gdr = _gdr()
    w = small(128, in_dtype, "scalar", seed=97)
    x = _degenerate(inputs(w), kind)
    print(f"{fn} degenerate {kind} in={in_dtype}", flush=True)
    got, ref = run(gdr, w, x, fn=fn), reference(w, x)
    tiny = ("dg", "dstate0") if kind == "forget" else ()
    compare(got, ref, w, names=tuple(n for n in NAMES if n not in tiny))
    for n in tiny:
        assert np.all(np.isfinite(got[n])), n
        err = float(np.max(np.abs(got[n] - ref[n])))
        assert err <= 1e-6 * max(1.0, rms(ref["dk"])), f"{n}: max|err| {err:.3e}"
    if kind == "beta0":
        assert not np.any(got["dv"]), "beta = 0: dv must be exactly zero"


@pytest.mark.parametrize("HK,HV", [(1, 8), (3, 6), (5, 5)])
def test_chunk_bwd_head_layouts(HK, HV):
    """Eight value heads per key head (the group sums of dq and dk over eight
    heads), an odd number of key heads, and five heads with one value head
    each (the direct dq/dk write), against the oracle."""
    gdr = _gdr()
    w = small(64, "bf16", "scalar", HK=HK, HV=HV, seqlens=(70, 0, 129), seed=98 + HV)
    x = inputs(w)
    print(f"chunk_bwd HK={HK} HV={HV}", flush=True)
    compare(run(gdr, w, x), reference(w, x), w)
