"""gdr_chunk_fwd_noalloc (the prefill with the library's static device scratch
instead of a caller workspace) against gdr_chunk_fwd on the same inputs, on
two calls in a row, the second smaller than the first; then a call that
needs no workspace, and a call whose minimum workspace exceeds the scratch
(rejected on the host before anything is enqueued)."""
import numpy as np
import pytest

import synth
from helpers import check_out, check_state, host, oracle_run, to_device, widened

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _gdr():
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    return gdr


def _workload(seqlens, HV, gate, seed):
    return synth.Workload(name="noalloc", seqlens=tuple(seqlens), HK=HV // 2, HV=HV, DK=128, DV=128,
                          in_dtype="bf16", gate=gate, rule="delta", gate_shift=3.0, state_dtype="f32",
                          num_slots=len(seqlens) + 2, zero_init=False, seed=seed)


def _both(gdr, w):
    """Run the workload through both entry points (each on a fresh pool);
    return their outputs and pools, and the oracle's."""
    x = synth.generate(w)
    d = to_device(w, x)
    pool_a, pool_b = d["pool"].clone(), d["pool"].clone()
    print(f"noalloc: lens {w.seqlens} HV {w.HV} gate {w.gate}", flush=True)
    o_a = gdr.chunk_fwd(d["q"], d["k"], d["v"], d["g"], d["beta"], pool_a, d["slot_idx"],
                        d["cu_seqlens"], gate=w.gate)
    o_b = gdr.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], pool_b, d["slot_idx"],
                                d["cu_seqlens"], gate=w.gate)
    torch.cuda.synchronize()
    o_ref, p_ref = oracle_run(w, widened(w, x), x["slot_idx"], x["cu_seqlens"], w.DK ** -0.5)
    return x, (host(o_a, "f32"), host(pool_a, "f32")), (host(o_b, "f32"), host(pool_b, "f32")), (o_ref, p_ref)


@pytest.mark.parametrize("gate", ["channel", "scalar"])
def test_noalloc_matches_chunk_fwd_on_two_calls(gate):
    gdr = _gdr()
    for seqlens, HV, seed in (((700, 64, 1300, 0), 4, 21), ((100, 37), 2, 22)):
        w = _workload(seqlens, HV, gate, seed)
        x, (o_a, p_a), (o_b, p_b), (o_ref, p_ref) = _both(gdr, w)
        # the allocation-free call against the workspace call, and both
        # against the oracle, under the bf16-input gate
        check_out(o_b, o_a, "bf16")
        check_out(o_b, o_ref, "bf16")
        for s in x["slot_idx"]:
            check_state(p_b[s], p_a[s], "bf16", "f32")
            check_state(p_b[s], p_ref[s], "bf16", "f32")
        untouched = np.setdiff1d(np.arange(w.num_slots), x["slot_idx"])
        assert np.array_equal(p_b[untouched], synth.widen(x["pool"], "f32")[untouched])


def test_noalloc_rejects_calls_beyond_its_scratch():
    gdr = _gdr()
    # 64 one-token sequences x 64 value heads: the fp32 state carry alone is
    # 64 * 64 * 128 * 128 * 4 bytes = 256 MiB, more than the 64 MiB scratch
    w = synth.Workload(name="big", seqlens=(1,) * 64, HK=64, HV=64, DK=128, DV=128, in_dtype="bf16",
                       gate="channel", rule="delta", gate_shift=3.0, state_dtype="f32", num_slots=64,
                       zero_init=True, seed=23)
    x = synth.generate(w)
    d = to_device(w, x)
    pool0 = d["pool"].clone()
    with pytest.raises(gdr.GdrError, match="scratch"):
        gdr.chunk_fwd_noalloc(d["q"], d["k"], d["v"], d["g"], d["beta"], d["pool"], d["slot_idx"],
                              d["cu_seqlens"], gate="channel", zero_init=True)
    torch.cuda.synchronize()
    assert torch.equal(d["pool"], pool0)
