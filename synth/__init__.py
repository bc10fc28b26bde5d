"""Seeded synthetic workloads for the gated delta rule forward pass.

This module only draws random inputs and casts them to their storage types.
It holds none of the method's arithmetic: no decay, no delta write, no read.
Both the fp64 oracle (through tests and the bench's CPU leg) and the HIP path
consume exactly the arrays produced here.

Recipe (the same for every workload):
  * one ``numpy.random.SeedSequence(seed)`` spawns one child stream per tensor,
    in the order q, k, v, beta-logits, g-logits, extras;
  * q, k ~ N(0, 1) per token and head, L2-normalised over the key dimension in
    fp64, then cast (fp64 -> fp32 -> bf16, round to nearest even) when the
    workload's input type is bf16;
  * v ~ N(0, 1), cast the same way;
  * beta = sigmoid(N(0, 1)) and g = -softplus(N(0, 1) - shift) in fp64, then
    rounded to fp32 (g = log alpha <= 0; channel gates draw one value per key
    channel);
  * initial states ~ N(0, 0.02^2) cast to the pool's storage type; slot indices
    are a seeded choice of distinct slots.
Draws go token-major, so generating a token range in blocks yields the same
values as one draw of the whole range.

bf16 arrays are carried as numpy ``uint16`` bit patterns; ``widen`` turns any
stored array into float64 exactly.
"""
from __future__ import annotations

import dataclasses
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

__all__ = ["Workload", "WORKLOADS", "workload", "generate", "widen",
           "f64_to_bf16_bits", "bf16_bits_to_f64", "HEADLINE"]


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

# The prefill workload the throughput figure is quoted on.
HEADLINE = "gdn_prefill_b4_t4096_h16_d128"


def workload(name: str, **overrides) -> Workload:
    w = WORKLOADS[name]
    return w.replace(**overrides) if overrides else w


# ----------------------------------------------------------------------------
# storage casts (input preparation only)
# ----------------------------------------------------------------------------

def f64_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp64 -> fp32 (RNE) -> bf16 (RNE) bit patterns as uint16 (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


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

_STREAMS = ("q", "k", "v", "beta", "g", "extra")


def _streams(seed: int):
    ss = np.random.SeedSequence(seed)
    return {name: np.random.Generator(np.random.PCG64(c))
            for name, c in zip(_STREAMS, ss.spawn(len(_STREAMS)))}


def _skip_normals(rng: np.random.Generator, count: int, block: int = 1 << 22):
    while count > 0:
        n = min(count, block)
        rng.standard_normal(n)
        count -= n


def generate(w: Workload, seed: Optional[int] = None, t0: int = 0,
             t1: Optional[int] = None, heads: Optional[np.ndarray] = None,
             block_tokens: int = 8192) -> dict:
    """Draw the workload's token inputs for tokens [t0, t1) plus its extras.

    Returns a dict with q, k [T, HK, DK], v [T, HV, DV] in storage form, beta
    [T, HV] fp32 (None for the linear rule), g [T, HV] or [T, HV, DK] fp32 (None
    for gate "none"), pool [num_slots, HV, DK, DV] in storage form, slot_idx
    [N] int32 and cu_seqlens [N+1] int32. Decode workloads with ``steps`` > 1
    lay the steps out as consecutive token blocks of N tokens.
    ``heads`` optionally keeps only some value heads (and the key heads they
    read) of the returned token arrays; draws still cover every head so the
    values equal those of the full tensors.
    """
    seed = w.seed if seed is None else seed
    T = w.T_total * w.steps
    t1 = T if t1 is None else t1
    assert 0 <= t0 <= t1 <= T
    rs = _streams(seed)
    HK, HV, DK, DV = w.HK, w.HV, w.DK, w.DV
    per_tok = {"q": HK * DK, "k": HK * DK, "v": HV * DV, "beta": HV,
               "g": HV * (DK if w.gate == "channel" else 1)}
    for name in per_tok:
        _skip_normals(rs[name], t0 * per_tok[name])

    out = {n: [] for n in per_tok}
    t = t0
    while t < t1:
        n = min(block_tokens, t1 - t)
        for name in ("q", "k"):
            x = rs[name].standard_normal((n, HK, DK))
            x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
            out[name].append(_cast(x, w.in_dtype))
        out["v"].append(_cast(rs["v"].standard_normal((n, HV, DV)), w.in_dtype))
        b = rs["beta"].standard_normal((n, HV))
        out["beta"].append((1.0 / (1.0 + np.exp(-b))).astype(np.float32))
        if w.gate == "channel":
            x = rs["g"].standard_normal((n, HV, DK))
        else:
            x = rs["g"].standard_normal((n, HV))
        z = x - w.gate_shift
        softplus = np.maximum(z, 0.0) + np.log1p(np.exp(-np.abs(z)))
        out["g"].append((-softplus).astype(np.float32))
        t += n
    res = {n: (np.concatenate(v, axis=0) if v else None) for n, v in out.items()}
    if res["q"] is None:
        res["q"] = _cast(np.zeros((0, HK, DK)), w.in_dtype)
        res["k"] = _cast(np.zeros((0, HK, DK)), w.in_dtype)
        res["v"] = _cast(np.zeros((0, HV, DV)), w.in_dtype)
        res["beta"] = np.zeros((0, HV), np.float32)
        res["g"] = np.zeros((0, HV) + ((DK,) if w.gate == "channel" else ()), np.float32)
    if w.rule == "linear":
        res["beta"] = None
    if w.gate == "none":
        res["g"] = None

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

    ex = rs["extra"]
    slot_idx = ex.choice(w.num_slots, size=w.N, replace=False).astype(np.int32)
    if w.zero_init:
        pool = np.zeros((w.num_slots, HV, DK, DV))
    else:
        pool = 0.02 * ex.standard_normal((w.num_slots, HV, DK, DV))
    res["pool"] = _cast(pool, w.state_dtype)
    res["slot_idx"] = slot_idx
    res["cu_seqlens"] = w.cu_seqlens()
    return res
