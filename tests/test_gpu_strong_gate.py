"""Channel gates (KDA's delta rule, GLA's linear rule) strong enough that the
in-chunk decay of a channel leaves the fp32 range: shift -2 (a channel decays
by about e^-135 over a 64-token chunk), shift -6 (about e^-96 over 16 tokens,
beyond the span the factored diagonal blocks take, so those blocks are summed
pair by pair), and a mixed gate whose channels alternate between almost no
decay (shift 6) and that extreme one. Every output and touched slot is
compared with the fp64 recurrence; no value may be non-finite. Strong
per-channel forgetting is what the channel gate is for ("You Could Have Come
Up With Kimi Delta Attention", section 4); the chunked form takes it through
16-token sub-blocks (section 5's table, section 6)."""
import itertools

import numpy as np
import pytest

import synth
from helpers import check_out, check_state, host, oracle_run, to_device, widened

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

RAGGED = (0, 1, 63, 64, 65, 130, 200)
GATES = {"strong": dict(gate_shift=-2.0), "extreme": dict(gate_shift=-6.0),
         "mixed": dict(gate_shift=0.0, channel_shifts=(6.0, -6.0, 6.0, 6.0, -2.0, -6.0))}
CASES = list(itertools.product([64, 128], ["bf16", "f32"], ["delta", "linear"], sorted(GATES)))


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


@pytest.mark.parametrize("D,in_dtype,rule,gate", CASES, ids=[f"d{d}-{i}-{r}-{g}" for d, i, r, g in CASES])
def test_strong_channel_gate_matches_oracle(D, in_dtype, rule, gate):
    gdr = _gdr()
    w = synth.Workload(name="strong", seqlens=RAGGED, HK=2, HV=4, DK=D, DV=D, in_dtype=in_dtype,
                       gate="channel", rule=rule, state_dtype="f32", num_slots=9, zero_init=False,
                       seed=31, **GATES[gate])
    x = synth.generate(w)
    d = to_device(w, x)
    print(f"chunk_fwd strong gate {gate}: D={D} in={in_dtype} rule={rule} "
          f"min g {float(x['g'].min()):.1f}", flush=True)
    o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                      d["cu_seqlens"], scale=D ** -0.5, rule=rule, gate="channel")
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], D ** -0.5)
    err, bound = check_out(host(o, in_dtype), o_ref, in_dtype)
    pool = host(d["pool"], "f32")
    smargin = max(check_state(pool[s], pool_ref[s], in_dtype, "f32") for s in x["slot_idx"])
    print(f"MARGIN strong gate {gate} D={D} {in_dtype} {rule}: o err/bound {err / bound:.3f}, "
          f"state err/bound {smargin:.3f}", flush=True)


@pytest.mark.parametrize("gate", sorted(GATES))
def test_strong_channel_gate_long_sequence(gate):
    """One 4096-token sequence at the KDA workload's head shape (d = 128, bf16),
    so that many chunks carry the state through strongly decayed channels."""
    gdr = _gdr()
    w = synth.Workload(name="strong_long", seqlens=(4096,), HK=2, HV=2, DK=128, DV=128, in_dtype="bf16",
                       gate="channel", rule="delta", state_dtype="f32", num_slots=1, zero_init=True,
                       seed=32, **GATES[gate])
    x = synth.generate(w)
    d = to_device(w, x)
    print(f"chunk_fwd strong gate {gate}: 4096 tokens", flush=True)
    o = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                      d["cu_seqlens"], rule="delta", gate="channel", zero_init=True)
    torch.cuda.synchronize()
    assert torch.isfinite(o).all()
    o_ref, pool_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], 128 ** -0.5)
    check_out(host(o, "bf16"), o_ref, "bf16")
    check_state(host(d["pool"], "f32")[0], pool_ref[0], "bf16", "f32")
