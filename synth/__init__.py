"""Seeded synthetic workloads for the gated delta rule forward pass.

This module only draws random inputs and casts them to their storage types.
It holds none of the method's arithmetic: no decay, no delta write, no read.
Both the fp64 oracle (through tests and the bench's CPU leg) and the HIP path
consume exactly the arrays produced here.

Recipe (the same for every workload):
  * each tensor (q, k, v, beta-logits, g-logits) is drawn in blocks of 4096
    tokens, block b from SeedSequence([seed, tensor id, b]); initial
    states slot by slot from SeedSequence([seed, 98, slot]) and slot indices
    from SeedSequence([seed, 99]);
  * draws are fp32 N(0, 1);
  * q, k are L2-normalised over the key dimension (norm accumulated in fp64),
    then cast to bf16 (round to nearest even) when the workload's input type
    is bf16;
  * v ~ N(0, 1), cast the same way;
  * beta = sigmoid(N(0, 1)) and g = -softplus(N(0, 1) - shift) in fp32
    (g = log alpha <= 0; channel gates draw one value per key channel, with
    one shift for every channel or a repeating pattern of per-channel shifts);
  * initial states ~ N(0, 0.02^2) cast to the pool's storage type; slot indices
    are a seeded choice of distinct slots.
Any token range reproduces the values of the whole tensor.

bf16 arrays are carried as numpy ``uint16`` bit patterns; ``widen`` turns any
stored array into float64 exactly.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass
from typing import Dict, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "widen",
           "f64_to_bf16_bits", "bf16_bits_to_f64", "HEADLINE", "CONFIGS", "GDN"]


@dataclass(frozen=True)
class Workload:
    """Shape, types and structure of one synthetic workload."""
    name: str
    seqlens: tuple            # tokens per sequence (decode: 1 each)
    HK: int
    HV: int
    DK: int
    DV: int
    in_dtype: str             # "f32" | "bf16" for q, k, v
    gate: str                 # "none" | "scalar" | "channel"
    rule: str                 # "delta" | "linear"
    gate_shift: float         # g = -softplus(x - shift)
    state_dtype: str          # "f32" | "bf16" pool storage
    num_slots: int
    zero_init: bool           # S0 = 0 instead of the pool's contents
    chunk_size: int = 64
    steps: int = 1            # decode: consecutive steps (fresh token each)
    seed: int = 0
    description: str = ""
    channel_shifts: tuple = ()  # channel gate: shift of key channel c is channel_shifts[c % len]
                                # (empty: gate_shift for every channel)

    @property
    def N(self) -> int:
        return len(self.seqlens)

    @property
    def T_total(self) -> int:
        return int(sum(self.seqlens))

    def cu_seqlens(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seqlens)]).astype(np.int32)

    def replace(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


def _ragged_lengths(seed: int, n: int, lo: int, hi: int) -> tuple:
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 0xA11])))
    return tuple(int(x) for x in rng.integers(lo, hi + 1, size=n))


# The five workloads. Sizes follow the pages' configurations; names say what
# each one is.
WORKLOADS: Dict[str, Workload] = {}


def _reg(w: Workload) -> Workload:
    WORKLOADS[w.name] = w
    return w


_reg(Workload(
    name="gdr_fp32_t256_h1_d64", seqlens=(256,), HK=1, HV=1, DK=64, DV=64,
    in_dtype="f32", gate="scalar", rule="delta", gate_shift=0.0,
    state_dtype="f32", num_slots=1, zero_init=True, seed=1,
    description="gated delta rule, 1 sequence x 1 head, T=256, d=64, fp32, S0=0"))
_reg(Workload(
    name="gdn_prefill_b4_t4096_h16_d128", seqlens=(4096,) * 4, HK=16, HV=16,
    DK=128, DV=128, in_dtype="bf16", gate="scalar", rule="delta", gate_shift=2.0,
    state_dtype="f32", num_slots=4, zero_init=True, seed=2,
    description="Gated DeltaNet chunkwise prefill, B=4, T=4096, H=16, d=128, bf16 in"))
_reg(Workload(
    name="la_prefill_b4_t4096_h16_d128", seqlens=(4096,) * 4, HK=16, HV=16,
    DK=128, DV=128, in_dtype="bf16", gate="none", rule="linear", gate_shift=2.0,
    state_dtype="f32", num_slots=4, zero_init=True, seed=2,
    description="the same shapes in linear-attention mode (alpha=1, no delta)"))
_reg(Workload(
    name="ragged_gqa_prefill_n8_hk16_hv32_d128",
    seqlens=_ragged_lengths(3, 8, 512, 16384), HK=16, HV=32, DK=128, DV=128,
    in_dtype="bf16", gate="scalar", rule="delta", gate_shift=2.0,
    state_dtype="bf16", num_slots=64, zero_init=False, seed=3,
    description="ragged varlen GQA prefill, 8 sequences of U{512..16384} tokens, "
                "bf16 pool [64,32,128,128]"))
_reg(Workload(
    name="decode_n256_hk16_hv32_d128", seqlens=(1,) * 256, HK=16, HV=32, DK=128,
    DV=128, in_dtype="bf16", gate="scalar", rule="delta", gate_shift=2.0,
    state_dtype="f32", num_slots=256, zero_init=False, steps=1000, seed=4,
    description="recurrent decode step, 256 sequences x 1 token, fp32 pool "
                "[256,32,128,128], 1000 consecutive steps"))
_reg(Workload(
    name="kda_prefill_t131072_h32_d128", seqlens=(131072,), HK=32, HV=32, DK=128,
    DV=128, in_dtype="bf16", gate="channel", rule="delta", gate_shift=3.0,
    state_dtype="f32", num_slots=1, zero_init=True, seed=5,
    description="KDA long-context prefill, T=131072, H=32, d=128, per-key-channel gate"))

_reg(Workload(
    name="short_prefill_n256_t16_hk16_hv32_d128", seqlens=(16,) * 256, HK=16, HV=32, DK=128,
    DV=128, in_dtype="bf16", gate="scalar", rule="delta", gate_shift=2.0,
    state_dtype="f32", num_slots=256, zero_init=False, seed=6,
    description="short ragged prefill over the decode pool: 256 sequences x 16 tokens, fp32 "
                "pool [256,32,128,128] (the tokenwise schedule's case: state I/O dominates)"))

_reg(Workload(
    name="gla_prefill_t131072_h32_d128", seqlens=(131072,), HK=32, HV=32, DK=128,
    DV=128, in_dtype="bf16", gate="channel", rule="linear", gate_shift=3.0,
    state_dtype="f32", num_slots=1, zero_init=True, seed=7,
    description="GLA (channel-gated linear attention) on the KDA workload's shapes"))
_reg(Workload(
    name="mamba2_prefill_b4_t4096_h16_d128", seqlens=(4096,) * 4, HK=16, HV=16, DK=128,
    DV=128, in_dtype="bf16", gate="scalar", rule="linear", gate_shift=2.0,
    state_dtype="f32", num_slots=4, zero_init=True, seed=8,
    description="scalar-gated linear attention (Mamba-2; RetNet with a constant gate) on the "
                "headline prefill's shapes"))

# The five configurations of the pages' workloads, in order.
CONFIGS = ("gdr_fp32_t256_h1_d64", "gdn_prefill_b4_t4096_h16_d128",
           "ragged_gqa_prefill_n8_hk16_hv32_d128", "decode_n256_hk16_hv32_d128",
           "kda_prefill_t131072_h32_d128")
# The workload the throughput figure is quoted on: the largest configuration
# (7.5 GB of algorithmic traffic per call).
HEADLINE = "kda_prefill_t131072_h32_d128"
# The Gated DeltaNet prefill on which the gradient, product and linear-mode
# legs are measured.
GDN = "gdn_prefill_b4_t4096_h16_d128"


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w


# ----------------------------------------------------------------------------
# storage casts (input preparation only)
# ----------------------------------------------------------------------------

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE) bit patterns as uint16 (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = u >> 16
    r &= 1
    r += 0x7FFF
    r += u          # no overflow for finite inputs
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f64(b: np.ndarray) -> np.ndarray:
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def widen(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored array (uint16 bits for bf16, float32 for f32) -> float64, exactly."""
    if dtype == "bf16":
        return bf16_bits_to_f64(a)
    return np.asarray(a, dtype=np.float64)


def _cast(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f64_to_bf16_bits(x)
    if dtype == "f32":
        return x.astype(np.float32)
    raise ValueError(dtype)


# ----------------------------------------------------------------------------
# generation
# ----------------------------------------------------------------------------

_TENSORS = {"q": 1, "k": 2, "v": 3, "beta": 4, "g": 5}
BLOCK = 4096   # tokens per independently seeded block


def _block(w: Workload, seed: int, name: str, b: int, T: int):
    """Stored values of tensor `name` for token block b (tokens b*BLOCK ...)."""
    n = min(BLOCK, T - b * BLOCK)
    rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, _TENSORS[name], b])))
    HK, HV, DK, DV = w.HK, w.HV, w.DK, w.DV
    f32 = np.float32
    if name in ("q", "k"):
        x = rng.standard_normal((n, HK, DK), dtype=f32)
        x /= np.sqrt(np.sum(np.square(x, dtype=np.float64), axis=-1, keepdims=True)).astype(f32)
        return _cast(x, w.in_dtype)
    if name == "v":
        return _cast(rng.standard_normal((n, HV, DV), dtype=f32), w.in_dtype)
    if name == "beta":
        b_ = rng.standard_normal((n, HV), dtype=f32)
        return (1.0 / (1.0 + np.exp(-b_))).astype(f32)
    x = rng.standard_normal((n, HV, DK) if w.gate == "channel" else (n, HV), dtype=f32)
    if w.gate == "channel" and w.channel_shifts:
        shifts = np.resize(np.asarray(w.channel_shifts, dtype=f32), DK)
        z = x - shifts
    else:
        z = x - f32(w.gate_shift)
    return (-(np.maximum(z, f32(0)) + np.log1p(np.exp(-np.abs(z))))).astype(f32)


def generate(w: Workload, seed: Optional[int] = None, t0: int = 0,
             t1: Optional[int] = None, heads: Optional[np.ndarray] = None,
             threads: Optional[int] = None) -> dict:
    """Draw the workload's token inputs for tokens [t0, t1) plus its extras.

    Returns a dict with q, k [T, HK, DK], v [T, HV, DV] in storage form, beta
    [T, HV] fp32 (None for the linear rule), g [T, HV] or [T, HV, DK] fp32 (None
    for gate "none"), pool [num_slots, HV, DK, DV] in storage form, slot_idx
    [N] int32 and cu_seqlens [N+1] int32. Decode workloads with ``steps`` > 1
    lay the steps out as consecutive token blocks of N tokens.
    Each tensor is drawn in blocks of BLOCK tokens, block b from its own
    stream SeedSequence([seed, tensor, b]), so any token range reproduces the
    values of the whole tensor and blocks can be drawn in parallel.
    ``heads`` optionally keeps only some value heads (and the key heads they
    read) of the returned token arrays.
    """
    from concurrent.futures import ThreadPoolExecutor
    import os

    seed = w.seed if seed is None else seed
    T = w.T_total * w.steps
    t1 = T if t1 is None else t1
    assert 0 <= t0 <= t1 <= T
    names = ["q", "k", "v"]
    if w.rule == "delta":
        names.append("beta")
    if w.gate != "none":
        names.append("g")
    b0, b1 = t0 // BLOCK, (t1 + BLOCK - 1) // BLOCK
    jobs = [(nm, b) for nm in names for b in range(b0, b1)]
    threads = threads or min(16, os.cpu_count() or 1)
    with ThreadPoolExecutor(max_workers=threads) as ex:
        parts = list(ex.map(lambda j: _block(w, seed, j[0], j[1], T), jobs))
    res = {"beta": None, "g": None}
    HK, HV, DK, DV = w.HK, w.HV, w.DK, w.DV
    empty = {"q": (0, HK, DK), "k": (0, HK, DK), "v": (0, HV, DV), "beta": (0, HV),
             "g": (0, HV, DK) if w.gate == "channel" else (0, HV)}
    for nm in names:
        blocks = [p for (n_, _), p in zip(jobs, parts) if n_ == nm]
        if blocks:
            full = np.concatenate(blocks, axis=0) if len(blocks) > 1 else blocks[0]
            res[nm] = full[t0 - b0 * BLOCK:t1 - b0 * BLOCK]
        else:
            dt = np.float32 if nm in ("beta", "g") or w.in_dtype == "f32" else np.uint16
            res[nm] = np.zeros(empty[nm], dt)

    if heads is not None:
        heads = np.asarray(heads)
        ratio = HV // HK
        kh = np.unique(heads // ratio)
        res["q"] = res["q"][:, kh]
        res["k"] = res["k"][:, kh]
        res["v"] = res["v"][:, heads]
        if res["beta"] is not None:
            res["beta"] = res["beta"][:, heads]
        if res["g"] is not None:
            res["g"] = res["g"][:, heads]

    ex_rng = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 99])))
    slot_idx = ex_rng.choice(w.num_slots, size=w.N, replace=False).astype(np.int32)
    if w.zero_init:
        res["pool"] = _cast(np.zeros((w.num_slots, HV, DK, DV), np.float32), w.state_dtype)
    else:
        def slot_state(sl):
            r = np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, 98, sl])))
            x = r.standard_normal((HV, DK, DV), dtype=np.float32)
            x *= np.float32(0.02)
            return _cast(x, w.state_dtype)
        with ThreadPoolExecutor(max_workers=threads) as ex:
            res["pool"] = np.stack(list(ex.map(slot_state, range(w.num_slots))))
    res["slot_idx"] = slot_idx
    res["cu_seqlens"] = w.cu_seqlens()
    return res
