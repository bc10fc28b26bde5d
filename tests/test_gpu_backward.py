"""GPU parity of gdr_linear_chunk_bwd (gradients of causal linear attention,
"From Attention to Learned Memory", section "Backward: reverse the boundary
scan, then differentiate each chunk") against the fp64 oracle's
linear_attention_grads_fp64, under the same gate as the forward outputs."""
import itertools

import numpy as np
import pytest

import oracle
import synth
from helpers import check_out, dev, host

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
