"""GPU parity of gdr_recurrent_bwd (gradients of the gated delta and gated
linear rules: the recurrence of "You Could Have Come Up With Kimi Delta
Attention", recurrent form, and the gated variants of "Linear attention
visualized", differentiated in reverse mode) against the fp64 oracle's
recurrent_grads_fp64.

Tolerance: fp32 inputs, max|err| <= 1e-4 * max(1, RMS of the reference) (the
gradients sum over up to a few hundred tokens, so their scale grows past 1);
bf16 inputs, 3e-3 * RMS as for the forward outputs (the oracle widens the same
rounded inputs, so only fp32 arithmetic separates the two)."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from helpers import dev, host, rms

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RAGGED = (0, 1, 7, 8, 9, 17, 64, 100)   # empty, one token, either side of the 8-token blocks


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


def inputs(w):
    x = synth.generate(w)
    x["do"] = synth.generate(w.replace(seed=w.seed + 500))["v"]
    return x


def run(gdr, w, x, out_dtype=torch.float32, **kw):
    d = {n: dev(x[n], w.in_dtype) for n in ("q", "k", "v", "do")}
    pool = dev(x["pool"], w.state_dtype)
    before = pool.clone()
    g = dev(x["g"], "f32") if w.gate != "none" else None
    beta = dev(x["beta"], "f32") if w.rule == "delta" else None
    out = gdr.recurrent_bwd(d["q"], d["k"], d["v"], g, beta, d["do"], pool, dev(x["slot_idx"], "i32"),
                            dev(x["cu_seqlens"], "i32"), rule=w.rule, gate=w.gate, zero_init=w.zero_init,
                            out_dtype=out_dtype, **kw)
    torch.cuda.synchronize()
    assert torch.equal(pool, before), "the backward must not write the pool"
    return {n: None if t is None else host(t, "f32") for n, t in out.items()}


def reference(w, x, heads=None, seqs=None):
    wid = lambda n: synth.widen(x[n], w.in_dtype)
    q, k, v, do = wid("q"), wid("k"), wid("v"), wid("do")
    pool = synth.widen(x["pool"], w.state_dtype)
    g = x["g"] if w.gate != "none" else None
    beta = x["beta"] if w.rule == "delta" else None
    cu, slots = x["cu_seqlens"], x["slot_idx"]
    if heads is not None:   # value heads of whole key-head groups
        G = w.HV // w.HK
        kh = sorted({h // G for h in heads})
        vh = [hk * G + j for hk in kh for j in range(G)]
        q, k = q[:, kh], k[:, kh]
        v, do, pool = v[:, vh], do[:, vh], pool[:, vh]
        g = None if g is None else g[:, vh]
        beta = None if beta is None else beta[:, vh]
    if seqs is not None:
        rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs])
        q, k, v, do = q[rows], k[rows], v[rows], do[rows]
        g = None if g is None else g[rows]
        beta = None if beta is None else beta[rows]
        lens = [cu[n + 1] - cu[n] for n in seqs]
        cu = np.concatenate([[0], np.cumsum(lens)])
        slots = slots[list(seqs)]
    return oracle.recurrent_grads_fp64(q, k, v, g, beta, do, pool, slots, cu, scale=w.DK ** -0.5,
                                       rule=w.rule, gate=w.gate, zero_init=w.zero_init)


def small(D, in_dtype, rule, gate, zero_init=False, state_dtype="f32", HK=2, HV=4, seqlens=RAGGED, seed=91):
    return synth.Workload(name="small", seqlens=tuple(seqlens), HK=HK, HV=HV, DK=D, DV=D,
                          in_dtype=in_dtype, gate=gate, rule=rule, gate_shift=2.0,
                          state_dtype=state_dtype, num_slots=11, zero_init=zero_init, seed=seed)


def compare(got, ref, w, names=("dq", "dk", "dv", "dbeta", "dg", "dstate0")):
    for n in names:
        if ref[n] is None:
            assert got[n] is None, n
            continue
        check(got[n], ref[n], w.in_dtype, n)


COMBOS = list(itertools.product([64, 128], ["bf16", "f32"], ["delta", "linear"], ["none", "scalar", "channel"]))


@pytest.mark.parametrize("D,in_dtype,rule,gate", COMBOS, ids=[f"d{D}-{i}-{r}-{g}" for D, i, r, g in COMBOS])
def test_recurrent_bwd_matches_oracle(D, in_dtype, rule, gate):
    gdr = _gdr()
    w = small(D, in_dtype, rule, gate, state_dtype="bf16" if D == 64 else "f32")
    x = inputs(w)
    print(f"recurrent_bwd D={D} in={in_dtype} {rule} {gate} lens={RAGGED}", flush=True)
    compare(run(gdr, w, x), reference(w, x), w)


@pytest.mark.parametrize("gate", ["scalar", "channel"])
def test_recurrent_bwd_zero_init(gate):
    gdr = _gdr()
    w = small(128, "f32", "delta", gate, zero_init=True)
    x = inputs(w)
    print(f"recurrent_bwd zero_init {gate}", flush=True)
    compare(run(gdr, w, x), reference(w, x), w)


def test_recurrent_bwd_bf16_gradients_and_no_dstate():
    gdr = _gdr()
    w = small(128, "bf16", "delta", "scalar", seqlens=(33, 5, 64))
    x = inputs(w)
    print("recurrent_bwd bf16 gradients, dstate0 off", flush=True)
    got = run(gdr, w, x, out_dtype=torch.bfloat16, dstate0=False)
    assert got["dstate0"] is None
    ref = reference(w, x)
    for n in ("dq", "dk", "dv"):   # one more bf16 rounding of the result
        r = rms(ref[n])
        assert np.max(np.abs(got[n] - ref[n]) - 2.0 ** -8 * np.abs(ref[n])) <= 3e-3 * r, n
    compare(got, ref, w, names=("dbeta", "dg"))


def test_recurrent_bwd_one_value_head_per_key_head():
    gdr = _gdr()
    w = small(128, "bf16", "delta", "channel", HK=3, HV=3, seqlens=(20, 41))
    x = inputs(w)
    print("recurrent_bwd HK = HV = 3", flush=True)
    compare(run(gdr, w, x), reference(w, x), w)


def test_recurrent_bwd_fused_qkv_strides_are_bit_identical():
    """q, k, v as views into one token-major buffer give the same bits as
    contiguous copies."""
    gdr = _gdr()
    w = small(128, "bf16", "delta", "scalar", seqlens=(30, 3, 50))
    x = inputs(w)
    print("recurrent_bwd fused qkv", flush=True)
    base = run(gdr, w, x)
    T = w.T_total
    q, k, v = (dev(x[n], "bf16") for n in ("q", "k", "v"))
    buf = torch.cat([q.reshape(T, -1), k.reshape(T, -1), v.reshape(T, -1)], dim=1).contiguous()
    qkd, vd = w.HK * w.DK, w.HV * w.DV
    qv = buf[:, :qkd].view(T, w.HK, w.DK)
    kv = buf[:, qkd:2 * qkd].view(T, w.HK, w.DK)
    vv = buf[:, 2 * qkd:2 * qkd + vd].view(T, w.HV, w.DV)
    out = gdr.recurrent_bwd(qv, kv, vv, dev(x["g"], "f32"), dev(x["beta"], "f32"), dev(x["do"], "bf16"),
                            dev(x["pool"], w.state_dtype), dev(x["slot_idx"], "i32"), dev(x["cu_seqlens"], "i32"),
                            rule="delta", gate="scalar")
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dbeta", "dg", "dstate0"):
        assert np.array_equal(host(out[n], "f32"), base[n]), n


def test_recurrent_bwd_linear_agrees_with_chunk_backward():
    """The plain linear rule through the tokenwise backward and through the
    chunkwise linear-attention backward (three chunk passes) agree."""
    gdr = _gdr()
    w = small(128, "f32", "linear", "none", HK=3, HV=3, seqlens=(70, 0, 130))
    x = inputs(w)
    print("recurrent_bwd vs linear_chunk_bwd", flush=True)
    got = run(gdr, w, x)
    d = {n: dev(x[n], "f32") for n in ("q", "k", "v", "do")}
    dq, dk, dv = gdr.linear_chunk_bwd(d["q"], d["k"], d["v"], d["do"], dev(x["pool"], "f32"),
                                      dev(x["slot_idx"], "i32"), dev(x["cu_seqlens"], "i32"))
    torch.cuda.synchronize()
    for n, t in (("dq", dq), ("dk", dk), ("dv", dv)):
        check(got[n], host(t, "f32"), "f32", n)


def test_recurrent_bwd_headline_shapes_sampled():
    """The prefill headline's shapes (4 x 4096 tokens, 16 heads, d = 128, bf16,
    scalar gate, delta rule) at full size; two heads recomputed by the oracle
    over two whole sequences."""
    gdr = _gdr()
    w = synth.WORKLOADS["gdn_prefill_b4_t4096_h16_d128"]
    x = inputs(w)
    print("recurrent_bwd headline shapes", flush=True)
    got = run(gdr, w, x)
    heads, seqs = [3, 12], [0, 3]
    ref = reference(w, x, heads=heads, seqs=seqs)
    cu = x["cu_seqlens"]
    rows = np.concatenate([np.arange(cu[n], cu[n + 1]) for n in seqs])
    for i, h in enumerate(heads):
        check(got["dq"][rows][:, h], ref["dq"][:, i], w.in_dtype, "dq")
        check(got["dk"][rows][:, h], ref["dk"][:, i], w.in_dtype, "dk")
        check(got["dv"][rows][:, h], ref["dv"][:, i], w.in_dtype, "dv")
        check(got["dbeta"][rows][:, h], ref["dbeta"][:, i], w.in_dtype, "dbeta")
        check(got["dg"][rows][:, h], ref["dg"][:, i], w.in_dtype, "dg")
        check(got["dstate0"][seqs][:, h], ref["dstate0"][:, i], w.in_dtype, "dstate0")


def test_recurrent_bwd_debug_checks_reject_bad_indices():
    """GDR_FLAG_DEBUG_CHECKS verifies cu_seqlens and slot_idx on the device
    before the walk is launched; valid indices pass and compute."""
    gdr = _gdr()
    w = small(64, "bf16", "delta", "scalar", seqlens=(5, 6))
    x = inputs(w)
    print("recurrent_bwd debug checks", flush=True)
    d = {n: dev(x[n], "bf16") for n in ("q", "k", "v", "do")}
    g, beta, pool = dev(x["g"], "f32"), dev(x["beta"], "f32"), dev(x["pool"], w.state_dtype)
    slots, cu = dev(x["slot_idx"], "i32"), dev(x["cu_seqlens"], "i32")
    call = lambda s, c: gdr.recurrent_bwd(d["q"], d["k"], d["v"], g, beta, d["do"], pool, s, c,
                                          debug_checks=True)
    bad = slots.clone()
    bad[1] = bad[0]
    with pytest.raises(gdr.GdrError) as e:
        call(bad, cu)
    assert e.value.status == 5
    badcu = cu.clone()
    badcu[1] = 9
    badcu[2] = 8
    with pytest.raises(gdr.GdrError) as e:
        call(slots, badcu)
    assert e.value.status == 5
    got = call(slots, cu)
    torch.cuda.synchronize()
    ref = reference(w, x)
    check(host(got["dk"], "f32"), ref["dk"], "bf16", "dk")
