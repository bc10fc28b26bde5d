#!/usr/bin/env python3
"""Benchmark of the gated delta rule forward pass on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one gdr_chunk_fwd call (the whole prefill path: loads, gate sums,
Gram matrices, triangular solve, corrected values, outputs, state scan and
write-back) over the workload's full batch, with inputs already resident in
HBM. For workloads under 1 GB three copies of the inputs/outputs are used in
rotation so that no step reads what the previous one left in the 256 MB
last-level cache. The decode
path is timed alongside: 1000 consecutive gdr_recurrent_step launches over
the 256-sequence decode workload, each step with a new token per sequence
(64 distinct token sets in rotation; the state pool carries over). The
ragged tokenwise recurrence (gdr_recurrent_fwd) is timed on 256 sequences of
16 tokens over the same fp32 pool, with gdr_chunk_fwd on that batch beside it.

Prints one JSON line. `value` is prefill tokens per second for one layer (all
heads) on the largest configuration, the KDA long-context prefill (T = 131072,
32 heads, per-key-channel gate); `roofline` describes its prefill call against
HBM bandwidth (its binding roofline), with its MFMA fraction alongside;
`configs` holds the same figures for each of the five configurations (and
configuration 2's linear-attention run), the decode step's as steps/s and HBM
fraction; `linear_backward` and `gdn_backward` time the gradients on the
Gated DeltaNet batch (`gdn_chunk_backward` the delta rule's chunkwise),
`gated_linear_backward` those of gated linear attention
on the ragged grouped-head batch (chunkwise, the tokenwise backward beside it); `recurrent_fwd` the tokenwise recurrence on a short
batch; `delta_product` the chunkwise prefill of Gated DeltaProduct (2
transitions per token); `speculative` a 4-token verify window per sequence and
the fold of its accepted prefix on the decode pool; `cpu_baseline` times the
fp64 oracle on bounded samples on the host's cores.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
MFMA_BF16_PEAK_TFLOPS = 2500.0  # dense bf16/fp16 MFMA
PROFILES = os.path.join(ROOT, "profiles")
CSRC = os.path.join(ROOT, "gated_delta_rule_gdr_amd", "csrc")
STEP_SRC = [os.path.join(CSRC, "recurrent_step.hip"), os.path.join(CSRC, "gdr_internal.h")]
RECUR_SRC = [os.path.join(CSRC, "recurrent_fwd.hip"), os.path.join(CSRC, "gdr_internal.h")]
CBWD_SRC = [os.path.join(CSRC, "chunk_bwd.hip"), os.path.join(CSRC, "chunk_fwd_ws.hip"),
            os.path.join(CSRC, "chunk_common.h"), os.path.join(CSRC, "gdr_internal.h")]
RBWD_SRC = [os.path.join(CSRC, "recurrent_bwd.hip"), os.path.join(CSRC, "recurrent_bwd.h"),
            os.path.join(CSRC, "gdr_internal.h")]


def prefill_kernel(w: synth.Workload):
    """(kernel name, its source files) of the prefill kernel(s) the library
    runs for this workload: the warp-specialised kernel for bf16 inputs
    without a channel gate; for bf16 inputs with the channel gate (KDA's
    delta rule, GLA's linear rule) the prep and state kernel pair (timed
    together, as one call);
    the general kernel otherwise (the dispatch in gdr_api.hip and
    chunk_fwd.hip)."""
    common = [os.path.join(CSRC, "chunk_common.h"), os.path.join(CSRC, "gdr_internal.h")]
    if w.in_dtype == "bf16" and w.gate != "channel":
        return "chunk_fwd_ws_kernel", [os.path.join(CSRC, "chunk_fwd_ws.hip")] + common
    if w.in_dtype == "bf16":
        return "kda_prep_kernel+kda_state_kernel", [os.path.join(CSRC, "chunk_fwd_kda.hip")] + common
    return "chunk_fwd_kernel", [os.path.join(CSRC, "chunk_fwd.hip")] + common


# ----------------------------------------------------------------------------
# algorithmic work (per launch)
# ----------------------------------------------------------------------------

def _isz(dtype: str) -> int:
    return 2 if dtype == "bf16" else 4


def prefill_bytes(w: synth.Workload, out_dtype="f32") -> int:
    """q, k (per key head), v, g, beta read once; o written once; the state
    read at sequence starts (unless zero-initialised) and written at ends."""
    T, ie = w.T_total, _isz(w.in_dtype)
    b = 2 * T * w.HK * w.DK * ie + T * w.HV * w.DV * ie
    if w.gate == "scalar":
        b += T * w.HV * 4
    elif w.gate == "channel":
        b += T * w.HV * w.DK * 4
    if w.rule == "delta":
        b += T * w.HV * 4
    b += T * w.HV * w.DV * _isz(out_dtype)
    st = w.N * w.HV * w.DK * w.DV * _isz(w.state_dtype)
    b += st if w.zero_init else 2 * st
    return b


def prefill_flops(w: synth.Workload, C=64) -> int:
    """Dense C x C tiles, no recompute (per token and value head):
    delta 4C(dk + dv) + 6 dk dv, linear 2C(dk + dv) + 4 dk dv."""
    if w.rule == "delta":
        per = 4 * C * (w.DK + w.DV) + 6 * w.DK * w.DV
    else:
        per = 2 * C * (w.DK + w.DV) + 4 * w.DK * w.DV
    return per * w.T_total * w.HV


def step_bytes(w: synth.Workload, out_dtype="f32") -> int:
    N, ie = w.N, _isz(w.in_dtype)
    b = 2 * N * w.HV * w.DK * w.DV * _isz(w.state_dtype)
    b += 2 * N * w.HK * w.DK * ie + N * w.HV * w.DV * ie
    b += N * w.HV * 4 * (2 if w.rule == "delta" else 1)
    b += N * w.HV * w.DV * _isz(out_dtype)
    return b


def source_hash(srcs) -> str:
    """First 16 hex digits of the sha256 of the kernel's source files, in order."""
    h = hashlib.sha256()
    for path in srcs:
        h.update(open(path, "rb").read())
    return h.hexdigest()[:16]


def committed_traffic(kernel: str, workload: str, srcs):
    """HBM bytes per launch from the committed rocprofv3 --pmc summary, or
    None if there is none or the kernel sources changed since it was taken."""
    path = os.path.join(PROFILES, f"{kernel}_{workload}_pmc.md")
    if not os.path.exists(path):
        return None
    text = open(path).read()
    m = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    h = re.search(r"source_sha256_16:\s*([0-9a-f]+)", text)
    if not m or not h or h.group(1) != source_hash(srcs):
        return None
    return float(m.group(1))


# ----------------------------------------------------------------------------
# GPU legs
# ----------------------------------------------------------------------------

def _dev(x, dtype, device):
    import torch
    if x is None:
        return None
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16).to(device)
    if dtype == "i32":
        return torch.from_numpy(np.ascontiguousarray(x, dtype=np.int32)).to(device)
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(device)


def bench_prefill(w: synth.Workload, steps: int, warmup: int, copies: int = 0):
    import torch
    import gated_delta_rule_gdr_amd as gdr
    gdr.load()
    dev = torch.device("cuda", 0)
    if copies <= 0:
        # rotate copies only where one call's inputs could stay in the 256 MB
        # last-level cache between calls
        copies = 3 if prefill_bytes(w) < (1 << 30) else 1
    x = synth.generate(w)
    sets = []
    for _ in range(copies):
        sets.append(dict(
            q=_dev(x["q"], w.in_dtype, dev), k=_dev(x["k"], w.in_dtype, dev),
            v=_dev(x["v"], w.in_dtype, dev), g=_dev(x["g"], "f32", dev),
            beta=_dev(x["beta"], "f32", dev), pool=_dev(x["pool"], w.state_dtype, dev),
            o=torch.empty((w.T_total, w.HV, w.DV), dtype=torch.float32, device=dev)))
    slot = _dev(x["slot_idx"], "i32", dev)
    cu = _dev(x["cu_seqlens"], "i32", dev)
    del x

    def run(i):
        s = sets[i % copies]
        gdr.chunk_fwd(s["q"], s["k"], s["v"], s["g"], s["beta"], s["pool"], slot, cu,
                      rule=w.rule, gate=w.gate, zero_init=w.zero_init, o=s["o"],
                      chunk_size=w.chunk_size)

    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        ev[i][0].record(stream)
        run(i)
        ev[i][1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kms = [a.elapsed_time(b) for a, b in ev]
    return wall / steps, float(np.mean(kms)), float(np.median(kms))


def bench_decode(w: synth.Workload, steps: int, warmup: int = 10):
    import torch
    import gated_delta_rule_gdr_amd as gdr
    dev = torch.device("cuda", 0)
    distinct = min(steps, 64)      # distinct token sets, used in rotation
    ws = w.replace(steps=distinct)
    x = synth.generate(ws)
    N = w.N
    q = _dev(x["q"], w.in_dtype, dev)
    k = _dev(x["k"], w.in_dtype, dev)
    v = _dev(x["v"], w.in_dtype, dev)
    g = _dev(x["g"], "f32", dev)
    beta = _dev(x["beta"], "f32", dev)
    pool = _dev(x["pool"], w.state_dtype, dev)
    slot = _dev(x["slot_idx"], "i32", dev)
    o = torch.empty((N, w.HV, w.DV), dtype=torch.float32, device=dev)
    del x

    def run(s):
        s %= distinct
        sl = slice(s * N, (s + 1) * N)
        gdr.recurrent_step(q[sl], k[sl], v[sl], g[sl], beta[sl], pool, slot, o=o,
                           rule=w.rule, gate=w.gate)

    for s in range(warmup):
        run(s)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    e0.record(stream)
    for s in range(steps):
        run(s)
    e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    kernel_ms = e0.elapsed_time(e1) / steps
    # For comparison, the same pool streamed in place by torch's elementwise
    # multiply: each element read and written once, as by the step.
    for _ in range(3):
        pool.mul_(1.0)
    reps = 20
    e0.record(stream)
    for _ in range(reps):
        pool.mul_(1.0)
    e1.record(stream)
    torch.cuda.synchronize()
    return wall / steps, kernel_ms, e0.elapsed_time(e1) / reps


def bench_recurrent_fwd(w: synth.Workload, steps: int, warmup: int = 5):
    """Mean kernel time (ms) of gdr_recurrent_fwd and of gdr_chunk_fwd on the
    same ragged batch, each call updating the pool in place."""
    import torch
    import gated_delta_rule_gdr_amd as gdr
    dev = torch.device("cuda", 0)
    x = synth.generate(w)
    a = dict(q=_dev(x["q"], w.in_dtype, dev), k=_dev(x["k"], w.in_dtype, dev),
             v=_dev(x["v"], w.in_dtype, dev), g=_dev(x["g"], "f32", dev),
             beta=_dev(x["beta"], "f32", dev), pool=_dev(x["pool"], w.state_dtype, dev),
             slot_idx=_dev(x["slot_idx"], "i32", dev), cu_seqlens=_dev(x["cu_seqlens"], "i32", dev))
    o = torch.empty((w.T_total, w.HV, w.DV), dtype=torch.float32, device=dev)
    del x
    stream = torch.cuda.current_stream(dev)
    out = {}
    for name, fn in (("recurrent_fwd", gdr.recurrent_fwd), ("chunk_fwd", gdr.chunk_fwd)):
        def run():
            fn(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["slot_idx"],
               a["cu_seqlens"], rule=w.rule, gate=w.gate, zero_init=w.zero_init, o=o)
        for _ in range(warmup):
            run()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) / steps
    return out


def product_bytes(w: synth.Workload, P: int, out_dtype="f32") -> int:
    """Gated DeltaProduct over w's batch with P transitions per token: q and
    g once per token, k, v and beta once per substep, o per token, the state
    read (unless zero-initialised) and written."""
    T, ie = w.T_total, _isz(w.in_dtype)
    b = T * w.HK * w.DK * ie + P * T * w.HK * w.DK * ie + P * T * w.HV * w.DV * ie
    b += T * w.HV * 4 if w.gate == "scalar" else 0
    b += P * T * w.HV * 4 if w.rule == "delta" else 0
    b += T * w.HV * w.DV * _isz(out_dtype)
    st = w.N * w.HV * w.DK * w.DV * _isz(w.state_dtype)
    return b + (st if w.zero_init else 2 * st)


def bench_product(w: synth.Workload, P: int, steps: int, warmup: int = 3):
    """Mean kernel time (ms) of gdr_chunk_fwd with P transitions per token on
    w's batch: q, g from w; k, v, beta from the same recipe at P times the
    lengths (another seed)."""
    import torch
    import gated_delta_rule_gdr_amd as gdr
    dev = torch.device("cuda", 0)
    xr = synth.generate(w)
    xv = synth.generate(w.replace(seqlens=tuple(P * n for n in w.seqlens), seed=w.seed + 1000))
    a = dict(q=_dev(xr["q"], w.in_dtype, dev), k=_dev(xv["k"], w.in_dtype, dev),
             v=_dev(xv["v"], w.in_dtype, dev), g=_dev(xr["g"], "f32", dev),
             beta=_dev(xv["beta"], "f32", dev), pool=_dev(xr["pool"], w.state_dtype, dev),
             slot_idx=_dev(xr["slot_idx"], "i32", dev), cu_seqlens=_dev(xr["cu_seqlens"], "i32", dev))
    o = torch.empty((w.T_total, w.HV, w.DV), dtype=torch.float32, device=dev)
    del xr, xv

    def run():
        gdr.chunk_fwd(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["slot_idx"],
                      a["cu_seqlens"], rule=w.rule, gate=w.gate, zero_init=w.zero_init, o=o,
                      products=P)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_linear_bwd(w: synth.Workload, steps: int, warmup: int = 3):
    """Mean time (ms) of gdr_linear_chunk_bwd (w.gate "none") or
    gdr_gated_linear_chunk_bwd (w.gate "scalar") on w's batch (all of its
    kernels: the gate shifts, input reversals or head repeats, three chunkwise
    passes, the output reversals, group sums and the gate's gradient), with a
    workspace allocated once."""
    import torch
    import gated_delta_rule_gdr_amd as gdr
    dev = torch.device("cuda", 0)
    x = synth.generate(w)
    do = synth.generate(w.replace(seed=w.seed + 500))["v"]
    a = dict(q=_dev(x["q"], w.in_dtype, dev), k=_dev(x["k"], w.in_dtype, dev),
             v=_dev(x["v"], w.in_dtype, dev), do=_dev(do, w.in_dtype, dev),
             pool=_dev(x["pool"], w.state_dtype, dev), slot_idx=_dev(x["slot_idx"], "i32", dev),
             cu_seqlens=_dev(x["cu_seqlens"], "i32", dev),
             g=_dev(x["g"], "f32", dev) if w.gate == "scalar" else None)
    del x, do
    L = gdr.load()
    ws = None

    def run():
        return gdr.linear_chunk_bwd(a["q"], a["k"], a["v"], a["do"], a["pool"], a["slot_idx"],
                                    a["cu_seqlens"], g=a["g"], zero_init=w.zero_init, workspace=ws)
    run()
    import ctypes
    args, _ = gdr._prepare(a["q"], a["k"], a["v"], a["g"], None, a["pool"], a["slot_idx"],
                           a["cu_seqlens"], None, None, "linear", w.gate, w.zero_init, False, 64,
                           torch.float32)
    ws = torch.empty(L.gdr_linear_chunk_bwd_workspace_bytes(ctypes.byref(args)), dtype=torch.uint8,
                     device=dev)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps


def bench_recurrent_bwd(w: synth.Workload, steps: int, warmup: int = 2, entry: str = "recurrent_bwd"):
    """Mean time (ms) of gdr_recurrent_bwd (the checkpointing walk and the
    reduction of the partial sums) or, with entry "chunk_bwd", of
    gdr_chunk_bwd (the forward walk, the reverse maps, the reverse walk, the
    per-chunk gradients and the group sums) on w's batch, with a workspace
    allocated once; also its workspace bytes."""
    import ctypes
    import torch
    import gated_delta_rule_gdr_amd as gdr
    dev = torch.device("cuda", 0)
    x = synth.generate(w)
    do = synth.generate(w.replace(seed=w.seed + 500))["v"]
    a = dict(q=_dev(x["q"], w.in_dtype, dev), k=_dev(x["k"], w.in_dtype, dev),
             v=_dev(x["v"], w.in_dtype, dev), do=_dev(do, w.in_dtype, dev),
             g=_dev(x["g"], "f32", dev) if w.gate != "none" else None,
             beta=_dev(x["beta"], "f32", dev) if w.rule == "delta" else None,
             pool=_dev(x["pool"], w.state_dtype, dev), slot_idx=_dev(x["slot_idx"], "i32", dev),
             cu_seqlens=_dev(x["cu_seqlens"], "i32", dev))
    del x, do
    L = gdr.load()
    args, _ = gdr._prepare(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["slot_idx"],
                           a["cu_seqlens"], None, None, w.rule, w.gate, w.zero_init, False, 64,
                           torch.float32)
    nbytes = getattr(L, "gdr_" + entry + "_workspace_bytes")(ctypes.byref(args))
    ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    kw = dict(rule=w.rule) if entry == "recurrent_bwd" else {}

    def run():
        return getattr(gdr, entry)(a["q"], a["k"], a["v"], a["g"], a["beta"], a["do"], a["pool"], a["slot_idx"],
                                   a["cu_seqlens"], gate=w.gate, zero_init=w.zero_init, workspace=ws, **kw)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, nbytes


def bench_speculative(w: synth.Workload, window: int, steps: int, warmup: int = 3):
    """Mean time (ms) of one verify of `window` draft tokens per sequence
    plus the fold of a seeded accepted prefix, on the decode workload's pool."""
    import torch
    import gated_delta_rule_gdr_amd as gdr
    dev = torch.device("cuda", 0)
    ww = w.replace(seqlens=(window,) * w.N, steps=1)
    x = synth.generate(ww)
    a = dict(q=_dev(x["q"], w.in_dtype, dev), k=_dev(x["k"], w.in_dtype, dev),
             v=_dev(x["v"], w.in_dtype, dev), g=_dev(x["g"], "f32", dev),
             beta=_dev(x["beta"], "f32", dev), pool=_dev(x["pool"], w.state_dtype, dev),
             slot_idx=_dev(x["slot_idx"], "i32", dev), cu_seqlens=_dev(x["cu_seqlens"], "i32", dev))
    rng = np.random.default_rng(11)
    acc = torch.from_numpy(rng.integers(0, window + 1, size=w.N).astype(np.int32)).to(dev)
    del x
    o = torch.empty((w.N * window, w.HV, w.DV), dtype=torch.float32, device=dev)

    def run():
        _, ring = gdr.verify_ring(a["q"], a["k"], a["v"], a["g"], a["beta"], a["pool"], a["slot_idx"],
                                  a["cu_seqlens"], o=o)
        gdr.state_fold(ring, acc, a["pool"], a["slot_idx"], a["cu_seqlens"], HK=w.HK, gate=w.gate)
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / steps, float(acc.float().mean())


# ----------------------------------------------------------------------------
# CPU leg: the fp64 oracle on a bounded sample
# ----------------------------------------------------------------------------

def _oracle_args(w: synth.Workload, x: dict) -> dict:
    return dict(q=synth.widen(x["q"], w.in_dtype), k=synth.widen(x["k"], w.in_dtype),
                v=synth.widen(x["v"], w.in_dtype),
                g=None if x["g"] is None else x["g"].astype(np.float64),
                beta=None if x["beta"] is None else x["beta"].astype(np.float64),
                pool=synth.widen(x["pool"], w.state_dtype))


_ORACLE_JOB = {}


def _oracle_heads(kh):
    """Worker: the oracle over key heads kh (and their value heads) of the
    batch in _ORACLE_JOB (inherited from the parent when the pool forks)."""
    import oracle
    w, x, a = _ORACLE_JOB["w"], _ORACLE_JOB["x"], _ORACLE_JOB["a"]
    ratio = w.HV // w.HK
    heads = (kh[:, None] * ratio + np.arange(ratio)[None, :]).ravel()
    t0 = time.perf_counter()
    oracle.recurrent_fp64(a["q"][:, kh], a["k"][:, kh], a["v"][:, heads],
                          None if a["g"] is None else a["g"][:, heads],
                          None if a["beta"] is None else a["beta"][:, heads],
                          a["pool"][:, heads], x["slot_idx"], x["cu_seqlens"],
                          scale=w.DK ** -0.5, rule=w.rule, gate=w.gate, zero_init=w.zero_init,
                          state_dtype=w.state_dtype)
    return time.perf_counter() - t0


def _time_oracle(w: synth.Workload, x: dict, procs: int) -> float:
    """Wall time of the fp64 oracle over x's batch with `procs` host
    processes: the key heads (with the value heads that read them) are split
    into `procs` groups that run side by side, each head's recurrence being
    separate. BLAS is held to one thread per process. Forks, so it must run
    before anything in this process touches the GPU."""
    import multiprocessing as mp
    from threadpoolctl import threadpool_limits
    _ORACLE_JOB.update(w=w, x=x, a=_oracle_args(w, x))
    groups = [gr for gr in np.array_split(np.arange(w.HK), min(procs, w.HK)) if len(gr)]
    with threadpool_limits(1):
        t0 = time.perf_counter()
        if len(groups) == 1:
            _oracle_heads(groups[0])
        else:
            with mp.get_context("fork").Pool(len(groups)) as pool:
                pool.map(_oracle_heads, groups)
        el = time.perf_counter() - t0
    _ORACLE_JOB.clear()
    return el


def cpu_baseline(w: synth.Workload, budget_s: float = 8.0):
    """The fp64 oracle on the host cores, on bounded samples (about 30 s of
    CPU work in all): the headline workload's first tokens of every
    sequence for all heads, timed with one process and with one process per
    core (at most 16, the host share of one GPU); samples of the other
    configurations beside it, each with the time the whole configuration
    would take at the sampled rate (the oracle's cost is linear in tokens x
    heads). Runs before the GPU is touched (it forks)."""
    affinity = len(os.sched_getaffinity(0))
    cores = min(affinity, 16)

    def sample(wl: synth.Workload, threads: int, budget: float):
        tok, lens = 32, np.asarray(wl.seqlens)
        while True:
            sl = tuple(int(n) for n in np.minimum(lens, tok))
            ws = wl.replace(seqlens=sl, steps=1)
            el = _time_oracle(ws, synth.generate(ws), threads)
            if el > budget / 3 or tok >= lens.max():
                return ws, el
            tok = min(int(lens.max()), tok * 4)

    ws, el1 = sample(w, 1, budget_s)
    elm = _time_oracle(ws, synth.generate(ws), cores)
    full_tok = w.T_total
    out = {"value": ws.T_total / elm, "unit": "tokens/s/layer", "cores": cores, "kind": "oracle",
           "sample": f"fp64 tokenwise recurrence of {w.name}: the first {ws.seqlens[0]} tokens of each of its "
                     f"{w.N} sequence(s), all {w.HV} value heads, the heads split over {cores} "
                     f"processes (one per core; the host shows {affinity}) in {elm:.2f} s",
           "single_thread": {"value": ws.T_total / el1, "seconds": el1},
           "full_config_estimate_s": full_tok / (ws.T_total / elm),
           "configs": {}}
    for name in synth.CONFIGS:
        wl = synth.workload(name)
        if name == w.name:
            continue
        if wl.steps > 1:
            # decode: one step of the whole batch
            x = synth.generate(wl.replace(steps=1))
            el = _time_oracle(wl.replace(steps=1), x, cores)
            out["configs"][name] = {"steps_per_s": 1.0 / el, "unit": "decode steps/s (256 sequences)",
                                    "sample": "one step of the full batch", "seconds": el,
                                    "full_config_estimate_s": wl.steps * el}
            continue
        ws2, el = sample(wl, cores, budget_s / 2)
        rate = ws2.T_total / el
        out["configs"][name] = {"tokens_per_s": rate, "unit": "tokens/s/layer",
                                "sample": f"first {max(ws2.seqlens)} tokens of each sequence, {ws2.T_total} "
                                          f"tokens in all", "seconds": el,
                                "full_config_estimate_s": wl.T_total / rate}
    return out


# ----------------------------------------------------------------------------

def prefill_leg(w: synth.Workload, steps: int, warmup: int) -> dict:
    """Time gdr_chunk_fwd on w (fp32 outputs): tokens/s, the kernel's HBM and
    MFMA fractions, and the committed counter traffic."""
    step_s, kernel_ms, kernel_med = bench_prefill(w, steps, warmup)
    nbytes = prefill_bytes(w)
    nflops = prefill_flops(w, w.chunk_size)
    kname, ksrcs = prefill_kernel(w)
    achieved = nbytes / (kernel_ms * 1e-3) / 1e9
    return {"workload": w.name, "tokens": w.T_total, "tokens_per_s": w.T_total / step_s,
            "ms_per_step": step_s * 1e3, "kernel": kname, "kernel_ms_mean": kernel_ms,
            "kernel_ms_median": kernel_med, "algorithmic_bytes": nbytes, "algorithmic_flops": nflops,
            "hbm_gbs": achieved, "hbm_frac": achieved / HBM_PEAK_GBS,
            "mfma_tflops": nflops / (kernel_ms * 1e-3) / 1e12,
            "mfma_frac": nflops / (kernel_ms * 1e-3) / 1e12 / MFMA_BF16_PEAK_TFLOPS,
            "traffic": committed_traffic(kname, w.name, ksrcs)}


def decode_leg(steps: int) -> dict:
    dw = synth.workload("decode_n256_hk16_hv32_d128")
    d_step, d_kernel, d_rmw = bench_decode(dw, steps)
    db = step_bytes(dw)
    pool_bytes = 2 * dw.num_slots * dw.HV * dw.DK * dw.DV * (2 if dw.state_dtype == "bf16" else 4)
    return {"workload": dw.name, "steps": steps, "steps_per_s": 1.0 / d_step,
            "us_per_step": d_step * 1e6, "kernel": "recurrent_step_kernel",
            "kernel_us_per_step": d_kernel * 1e3, "algorithmic_bytes_per_step": db,
            "hbm_gbs": db / (d_kernel * 1e-3) / 1e9,
            "hbm_frac": db / (d_kernel * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": committed_traffic("recurrent_step_kernel", dw.name, STEP_SRC),
            # torch's in-place multiply over the whole pool (read + write), the
            # same stream without the step's arithmetic: a reference for the
            # rate an in-place state stream reaches on this device
            "pool_inplace_stream_us": d_rmw * 1e3,
            "pool_inplace_stream_gbs": pool_bytes / (d_rmw * 1e-3) / 1e9}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default=synth.HEADLINE)
    ap.add_argument("--decode-steps", type=int, default=1000)
    ap.add_argument("--no-configs", action="store_true",
                    help="time only --workload (no other configuration legs)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--recurrent-steps", type=int, default=50)
    ap.add_argument("--no-recurrent", action="store_true")
    ap.add_argument("--product-steps", type=int, default=20)
    ap.add_argument("--no-linear", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--backward-steps", type=int, default=10)
    ap.add_argument("--no-speculative", action="store_true")
    ap.add_argument("--no-product", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run plain device copies of a known size (scales the HBM "
                         "byte counters of a profiler run) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print(json.dumps({"error": "the library and this benchmark run on one GPU; the gated delta rule "
                                   "shards by (sequence, head) with no communication and "
                                   "multi-GPU runs are not part of it"}))
        sys.exit(2)

    w = synth.workload(args.workload)
    # the CPU leg forks worker processes, so it runs before the GPU is touched
    cpu = None if (args.no_cpu_baseline or args.calibrate_copy) else cpu_baseline(w)

    import torch
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}))
        sys.exit(1)

    if args.calibrate_copy:
        nbytes = 512 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibration": "device copy", "bytes_read_per_copy": nbytes,
                          "bytes_written_per_copy": nbytes, "copies": 3}), flush=True)
        return

    torch.cuda.synchronize()
    head = prefill_leg(w, args.steps, args.warmup)
    result = {
        "metric": "prefill tokens/s/layer + decode steps/s; % MFMA peak / % HBM BW",
        "value": head["tokens_per_s"],
        "unit": "tokens/s/layer",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded; q,k L2-normalised N(0,1), v N(0,1), beta=sigmoid(N(0,1)), "
                "g=-softplus(N(0,1)-shift))",
        "config": {"workload": w.name, "batch": w.N, "seq_len": int(max(w.seqlens)),
                   "tokens": w.T_total, "key_heads": w.HK, "value_heads": w.HV,
                   "head_dim": w.DK, "chunk": w.chunk_size, "gate": w.gate, "rule": w.rule,
                   "in_dtype": w.in_dtype, "out_dtype": "f32", "state_dtype": w.state_dtype},
        "roofline": {"bound": "hbm", "achieved": head["hbm_gbs"], "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": head["hbm_frac"], "traffic": head["traffic"],
                     "kernel": head["kernel"], "kernel_ms_mean": head["kernel_ms_mean"],
                     "kernel_ms_median": head["kernel_ms_median"],
                     "algorithmic_bytes": head["algorithmic_bytes"],
                     "algorithmic_flops": head["algorithmic_flops"],
                     "mfma_tflops": head["mfma_tflops"], "mfma_frac": head["mfma_frac"]},
    }
    if not args.no_configs:
        # every configuration of the pages' workloads (the headline's numbers
        # repeated under its name), and configuration 2's linear-attention run
        legs = {}
        for name in synth.CONFIGS:
            if name == w.name:
                legs[name] = head
            elif synth.workload(name).steps > 1:
                if not args.no_decode:
                    legs[name] = decode_leg(args.decode_steps)
            else:
                legs[name] = prefill_leg(synth.workload(name), args.steps, args.warmup)
        if not args.no_linear:
            legs["la_prefill_b4_t4096_h16_d128"] = prefill_leg(
                synth.workload("la_prefill_b4_t4096_h16_d128"), args.steps, args.warmup)
        result["configs"] = legs
        if "decode_n256_hk16_hv32_d128" in legs:
            result["decode"] = legs["decode_n256_hk16_hv32_d128"]
    if not args.no_recurrent:
        rw = synth.workload("short_prefill_n256_t16_hk16_hv32_d128")
        t = bench_recurrent_fwd(rw, args.recurrent_steps)
        rb = prefill_bytes(rw)
        result["recurrent_fwd"] = {
            "workload": rw.name, "steps": args.recurrent_steps,
            "kernel_us": t["recurrent_fwd"] * 1e3,
            "tokens_per_s": rw.T_total / (t["recurrent_fwd"] * 1e-3),
            "algorithmic_bytes": rb,
            "hbm_gbs": rb / (t["recurrent_fwd"] * 1e-3) / 1e9,
            "hbm_frac": rb / (t["recurrent_fwd"] * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "traffic": committed_traffic("recurrent_fwd_kernel", rw.name, RECUR_SRC),
            "chunk_fwd_kernel_us_same_batch": t["chunk_fwd"] * 1e3}
    if not args.no_backward:
        # gradients of the linear-attention mode (dq, dk, dv from dO)
        bw = synth.workload("la_prefill_b4_t4096_h16_d128")
        bt = bench_linear_bwd(bw, args.steps)
        T, HD = bw.T_total, bw.HV * bw.DK
        bb = 4 * T * HD * _isz(bw.in_dtype) + 3 * T * HD * 4   # q, k, v, dO read; dq, dk, dv fp32
        bf = 3 * prefill_flops(bw, bw.chunk_size)                # one linear pass per gradient
        result["linear_backward"] = {
            "workload": bw.name, "steps": args.steps, "ms": bt, "tokens_per_s": T / (bt * 1e-3),
            "algorithmic_bytes": bb, "hbm_gbs": bb / (bt * 1e-3) / 1e9,
            "hbm_frac": bb / (bt * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_flops": bf, "mfma_tflops": bf / (bt * 1e-3) / 1e12}
        # gradients of gated linear attention (dq, dk, dv, dg) on the ragged
        # grouped-head batch, chunkwise, and tokenwise beside it
        lw = synth.workload("ragged_gqa_prefill_n8_hk16_hv32_d128").replace(rule="linear")
        lt = bench_linear_bwd(lw, args.steps)
        lrt, _ = bench_recurrent_bwd(lw, args.backward_steps)
        T, HKD, HVD = lw.T_total, lw.HK * lw.DK, lw.HV * lw.DV
        # q, k, v, dO, g and the initial states read; dq, dk, dv, dg written (fp32)
        sb = lw.N * lw.HV * lw.DK * lw.DV
        lb = ((2 * HKD + 2 * HVD) * T * _isz(lw.in_dtype) + T * lw.HV * 4 + sb * _isz(lw.state_dtype)
              + (2 * HKD + HVD) * T * 4 + T * lw.HV * 4)
        lf = 3 * prefill_flops(lw, lw.chunk_size)   # one linear pass per gradient
        result["gated_linear_backward"] = {
            "workload": lw.name + " (linear rule)", "steps": args.steps, "ms": lt,
            "tokens_per_s": T / (lt * 1e-3), "algorithmic_bytes": lb, "hbm_gbs": lb / (lt * 1e-3) / 1e9,
            "hbm_frac": lb / (lt * 1e-3) / 1e9 / HBM_PEAK_GBS, "algorithmic_flops": lf,
            "mfma_tflops": lf / (lt * 1e-3) / 1e12, "tokenwise_ms_same_batch": lrt}
        # gradients of the gated delta rule on the GDN batch (tokenwise)
        gw = synth.workload(synth.GDN)
        gt, gws = bench_recurrent_bwd(gw, args.backward_steps)
        T, HD, HVT = gw.T_total, gw.HV * gw.DK, gw.T_total * gw.HV
        # q, k, v, dO, g, beta and the initial states read; dq, dk, dv, dbeta,
        # dg and the initial state's gradient written (fp32)
        sb = gw.N * gw.HV * gw.DK * gw.DV
        gb = (4 * T * HD * _isz(gw.in_dtype) + 2 * HVT * 4 + sb * _isz(gw.state_dtype)
              + 3 * T * HD * 4 + 2 * HVT * 4 + sb * 4)
        result["gdn_backward"] = {
            "workload": gw.name, "steps": args.backward_steps, "ms": gt, "tokens_per_s": T / (gt * 1e-3),
            "algorithmic_bytes": gb, "hbm_gbs": gb / (gt * 1e-3) / 1e9,
            "hbm_frac": gb / (gt * 1e-3) / 1e9 / HBM_PEAK_GBS, "workspace_bytes": gws,
            "traffic": committed_traffic("recurrent_bwd_kernel+recurrent_bwd_reduce_kernel", gw.name, RBWD_SRC)}
        # the same gradients chunkwise (forward walk, reverse maps, reverse
        # walk, per-chunk gradients, group sums)
        ct, cws = bench_recurrent_bwd(gw, args.steps, entry="chunk_bwd")
        result["gdn_chunk_backward"] = {
            "workload": gw.name, "steps": args.steps, "ms": ct, "tokens_per_s": T / (ct * 1e-3),
            "algorithmic_bytes": gb, "hbm_gbs": gb / (ct * 1e-3) / 1e9,
            "hbm_frac": gb / (ct * 1e-3) / 1e9 / HBM_PEAK_GBS, "workspace_bytes": cws,
            "speedup_vs_tokenwise": gt / ct, "traffic": committed_traffic("chunk_bwd", gw.name, CBWD_SRC)}
    if not args.no_product:
        pw, P = synth.workload(synth.GDN), 2
        pt = bench_product(pw, P, args.product_steps)
        pb = product_bytes(pw, P)
        result["delta_product"] = {
            "workload": pw.name, "products": P, "steps": args.product_steps,
            "kernel_ms": pt, "tokens_per_s": pw.T_total / (pt * 1e-3),
            "algorithmic_bytes": pb, "hbm_gbs": pb / (pt * 1e-3) / 1e9,
            "hbm_frac": pb / (pt * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "mfma_tflops": prefill_flops(pw.replace(seqlens=tuple(P * n for n in pw.seqlens)),
                                         pw.chunk_size) / (pt * 1e-3) / 1e12,
            "traffic": committed_traffic("chunk_fwd_ws_kernel", "gdp_nh2_prefill_b4_t4096_h16_d128",
                                         prefill_kernel(pw)[1])}
    if not args.no_speculative and "decode" in result:
        # speculative decoding: verify 4 draft tokens per sequence, fold the
        # accepted prefix (the decode workload's pool and heads)
        sw_ = synth.workload("decode_n256_hk16_hv32_d128")
        sp_ms, mean_acc = bench_speculative(sw_, 4, 50)
        result["speculative"] = {
            "workload": sw_.name, "window": 4, "mean_accepted": mean_acc, "ms_per_window": sp_ms,
            "accepted_tokens_per_s": sw_.N * mean_acc / (sp_ms * 1e-3),
            "decode_steps_same_tokens_ms": result["decode"]["kernel_us_per_step"] * 1e-3 * mean_acc}
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
