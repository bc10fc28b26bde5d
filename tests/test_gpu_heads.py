"""Head layouts beyond the usual two value heads per key head: one head, one
key head shared by eight value heads, odd key-head counts and ratios 1, 4 and
2 on them. The workgroup grids put all workgroups of one (sequence, key head)
on one XCD and pad the last round of XCDs; these layouts exercise that
mapping (and the key-head index h / (HV / HK)) on every forward entry point,
against the fp64 recurrence (the Mojo "gated_delta" page: value heads share a
key head in groups)."""
import itertools

import numpy as np
import pytest

import synth
from helpers import check_out, check_state, host, oracle_run, to_device, widened

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

LAYOUTS = [(1, 1), (1, 8), (3, 3), (3, 12), (5, 10)]
ENTRIES = [("chunk", "bf16", "scalar"), ("chunk", "f32", "scalar"), ("chunk", "bf16", "channel"),
           ("recurrent", "bf16", "scalar"), ("step", "bf16", "channel")]
CASES = list(itertools.product(LAYOUTS, ENTRIES))


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


@pytest.mark.parametrize("layout,entry", CASES,
                         ids=[f"hk{hk}-hv{hv}-{e}-{i}-{g}" for (hk, hv), (e, i, g) in CASES])
def test_head_layouts_match_oracle(layout, entry):
    gdr = _gdr()
    HK, HV = layout
    kind, in_dtype, gate = entry
    D = 64
    seqlens = (1,) * 5 if kind == "step" else (1, 70, 0, 130)
    w = synth.Workload(name="heads", seqlens=seqlens, HK=HK, HV=HV, DK=D, DV=D, in_dtype=in_dtype, gate=gate,
                       rule="delta", gate_shift=2.0 if gate == "scalar" else 3.0, state_dtype="f32",
                       num_slots=len(seqlens) + 2, zero_init=False, seed=71 + HK + HV)
    x = synth.generate(w)
    d = to_device(w, x)
    scale = D ** -0.5
    print(f"heads HK={HK} HV={HV}: {kind} in={in_dtype} gate={gate}", flush=True)
    if kind == "chunk":
        o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                          d["cu_seqlens"], scale=scale, rule="delta", gate=gate)
    elif kind == "recurrent":
        o = gdr.recurrent_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                              d["cu_seqlens"], scale=scale, rule="delta", gate=gate)
    else:
        o = gdr.recurrent_step(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                               scale=scale, rule="delta", gate=gate)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    cu = np.arange(len(seqlens) + 1) if kind == "step" else x["cu_seqlens"]
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], cu, scale)
    check_out(host(o, in_dtype), o_ref, in_dtype)
    pool = host(d["pool"], "f32")
    for s in range(w.num_slots):
        if s in set(int(v) for v in x["slot_idx"]):
            check_state(pool[s], pool_ref[s], in_dtype, "f32")
        else:
            # slots no sequence names come back bit for bit
            assert np.array_equal(pool[s], synth.widen(x["pool"], "f32")[s]), f"slot {s} was written"
