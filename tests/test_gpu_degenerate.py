"""Degenerate cases of the update, on every forward entry point, against the
fp64 recurrence:

* beta = 0: the delta rule writes nothing, the state only decays;
* beta = 1: the write replaces the value stored under the key outright (for a
  unit key; "From Attention to Learned Memory", the delta rule's write as a
  correction of the current prediction);
* zero keys on every other token: such a token neither reads from nor writes
  to the state (its prediction is zero and so is its outer product);
* complete forgetting: a log-decay of -60 per token (per channel for the
  channel gate), so that e^{G_i - G_j} underflows to zero two tokens apart:
  the state is all but wiped before every write and each output reads little
  more than its own token's write ("You Could Have Come Up With Kimi Delta
  Attention", the gate as forgetting applied before the write);
* a gate of exactly zero: the same recurrence as no gate.

The chunked prefill at chunk sizes 64 and 16, the tokenwise recurrence and the
one-token step all take each case, for the scalar and the channel gate and
both input dtypes, on a ragged batch with grouped key heads."""
import itertools

import numpy as np
import pytest

import synth
from helpers import check_out, check_state, host, oracle_run, to_device, widened

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RAGGED = (0, 1, 63, 64, 65, 130, 200)
KINDS = ("beta0", "beta1", "zero_k", "forget", "zero_g")
GATES = ("scalar", "channel")
DTYPES = ("bf16", "f32")


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


def _degenerate(x: dict, kind: str) -> dict:
    """The workload's inputs with one degenerate feature imposed (storage
    form: bf16 arrays are bit patterns, for which 0 is +0.0)."""
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


def _workload(seqlens, D, in_dtype, gate, seed):
    return synth.Workload(name="degenerate", seqlens=seqlens, HK=2, HV=4, DK=D, DV=D, in_dtype=in_dtype,
                          gate=gate, rule="delta", gate_shift=2.0 if gate == "scalar" else 3.0,
                          state_dtype="f32", num_slots=max(len(seqlens), 1) + 2,
                          zero_init=False, seed=seed)


def _check(w, x, d, o, cu, scale):
    in_dtype = w.in_dtype
    assert torch.isfinite(o).all()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], cu, scale)
    err, bound = check_out(host(o, in_dtype), o_ref, in_dtype)
    pool = host(d["pool"], "f32")
    smargin = max(check_state(pool[s], pool_ref[s], in_dtype, "f32") for s in x["slot_idx"])
    return err / bound, smargin


ENTRIES = ("chunk64", "chunk16", "recurrent")
CASES = list(itertools.product(KINDS, GATES, DTYPES, ENTRIES))


@pytest.mark.parametrize("kind,gate,in_dtype,entry", CASES, ids=["-".join(c) for c in CASES])
def test_degenerate_prefill(kind, gate, in_dtype, entry):
    gdr = _gdr()
    D = 128
    w = _workload(RAGGED, D, in_dtype, gate, seed=61)
    x = _degenerate(synth.generate(w), kind)
    d = to_device(w, x)
    scale = D ** -0.5
    print(f"degenerate {kind}: {entry} gate={gate} in={in_dtype}", flush=True)
    if entry == "recurrent":
        o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                              d["cu_seqlens"], scale=scale, rule="delta", gate=gate)
    else:
        o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                          d["cu_seqlens"], scale=scale, rule="delta", gate=gate,
                          chunk_size=64 if entry == "chunk64" else 16)
    torch.cuda.synchronize()
    om, sm = _check(w, x, d, o, x["cu_seqlens"], scale)
    print(f"MARGIN degenerate {kind} {entry} {gate} {in_dtype}: o err/bound {om:.3f}, "
          f"state err/bound {sm:.3f}", flush=True)


STEP_CASES = list(itertools.product(KINDS, GATES, DTYPES))


@pytest.mark.parametrize("kind,gate,in_dtype", STEP_CASES, ids=["-".join(c) for c in STEP_CASES])
def test_degenerate_step(kind, gate, in_dtype):
    """The one-token step over a batch of 24 sequences (one token each)."""
    gdr = _gdr()
    D, N = 128, 24
    w = _workload((1,) * N, D, in_dtype, gate, seed=62)
    x = _degenerate(synth.generate(w), kind)
    d = to_device(w, x)
    scale = D ** -0.5
    print(f"degenerate {kind}: step gate={gate} in={in_dtype}", flush=True)
    o = gdr.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                           scale=scale, rule="delta", gate=gate)
    torch.cuda.synchronize()
    _check(w, x, d, o, np.arange(N + 1), scale)


def test_zero_keys_leave_state_untouched_by_writes():
    """With every key zero and no gate, every prediction is zero and every
    write is a zero outer product: each slot comes back bit for bit, and the
    outputs are the queries read against the untouched initial states."""
    gdr = _gdr()
    D = 128
    w = synth.Workload(name="zero_keys", seqlens=(1, 64, 130), HK=2, HV=4, DK=D, DV=D, in_dtype="bf16",
                       gate="none", rule="delta", gate_shift=0.0, state_dtype="f32", num_slots=5,
                       zero_init=False, seed=63)
    x = synth.generate(w)
    x["k"] = np.zeros_like(x["k"])
    d = to_device(w, x)
    before = d["pool"].clone()
    print("degenerate: all keys zero, chunk_fwd", flush=True)
    o = gdr.chunk_fwd(d["q"], d["k"], d["v"], None, d["beta"], d["pool"], d["slot_idx"], d["cu_seqlens"],
                      rule="delta", gate="none")
    torch.cuda.synchronize()
    assert torch.equal(d["pool"], before)
    om, _ = _check(w, x, d, o, x["cu_seqlens"], D ** -0.5)
    print(f"MARGIN zero keys: o err/bound {om:.3f}", flush=True)
