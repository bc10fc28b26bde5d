"""The seeded input generator is deterministic and block-consistent."""
import numpy as np

import synth


def test_deterministic_and_block_consistent():
    w = synth.workload("gdr_fp32_t256_h1_d64")
    a = synth.generate(w)
    b = synth.generate(w, threads=1)
    for key in ("q", "k", "v", "beta", "g", "pool"):
        np.testing.assert_array_equal(a[key], b[key])
    part = synth.generate(w, t0=100, t1=160)
    for key in ("q", "k", "v", "beta", "g"):
        np.testing.assert_array_equal(part[key], a[key][100:160])


def test_shapes_and_ranges():
    w = synth.workload("ragged_gqa_prefill_n8_hk16_hv32_d128")
    assert w.N == 8 and all(512 <= n <= 16384 for n in w.seqlens)
    x = synth.generate(w.replace(seqlens=(5, 3)), heads=np.array([6, 7]))
    assert x["q"].shape == (8, 1, 128) and x["q"].dtype == np.uint16
    assert x["v"].shape == (8, 2, 128)
    qn = np.linalg.norm(synth.widen(x["q"], "bf16"), axis=-1)
    assert np.all(np.abs(qn - 1) < 1e-2)
    assert np.all(x["g"] <= 0) and np.all((x["beta"] > 0) & (x["beta"] < 1))
    assert len(np.unique(x["slot_idx"])) == 2
    assert x["pool"].shape == (64, 32, 128, 128)


def test_bf16_cast_round_trip():
    rng = np.random.default_rng(0)
    x = rng.standard_normal(1000)
    b = synth.f64_to_bf16_bits(x)
    y = synth.bf16_bits_to_f64(b)
    assert np.all(np.abs(y - x) <= np.abs(x) * 2 ** -8)


def test_channel_shift_pattern():
    """Per-channel gate shifts repeat over the key channels; a single shift
    draws the same values as a pattern of that one shift."""
    import numpy as np
    import synth
    base = synth.Workload(name="t", seqlens=(40,), HK=1, HV=2, DK=64, DV=64, in_dtype="bf16",
                          gate="channel", rule="delta", gate_shift=1.0, state_dtype="f32",
                          num_slots=1, zero_init=True, seed=3)
    g1 = synth.generate(base)["g"]
    g2 = synth.generate(base.replace(channel_shifts=(1.0,)))["g"]
    assert np.array_equal(g1, g2)
    g3 = synth.generate(base.replace(channel_shifts=(8.0, -8.0)))["g"]
    assert g3.shape == g1.shape and np.all(g3 <= 0)
    assert g3[:, :, 0::2].mean() > -0.01 and g3[:, :, 1::2].mean() < -7.0
