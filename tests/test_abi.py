"""The C ABI library loads, exports what include/gdr.h declares, and rejects
malformed arguments on the host before touching the GPU (no compute here)."""
import ctypes
import os
import re
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "gdr.h")


def _lib():
    import gated_delta_rule_gdr_amd as gdr
    if not os.path.exists(gdr.lib_path):
        pytest.fail("libgdr.so is not built (python -m gated_delta_rule_gdr_amd.build)")
    return gdr, gdr.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(gdr_[a-z_0-9]+)\s*\(",
                                 text, re.M)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    assert names == sorted(["gdr_abi_version", "gdr_chunk_fwd_workspace_bytes", "gdr_chunk_fwd",
                            "gdr_recurrent_step", "gdr_recurrent_fwd", "gdr_status_string",
                            "gdr_last_error", "gdr_linear_chunk_bwd_workspace_bytes",
                            "gdr_linear_chunk_bwd", "gdr_ring_record_elements",
                            "gdr_ring_record_stride", "gdr_verify_ring", "gdr_state_fold",
                            "gdr_recurrent_bwd_workspace_bytes", "gdr_recurrent_bwd",
                            "gdr_chunk_fwd_noalloc", "gdr_gated_linear_chunk_bwd",
                            "gdr_chunk_bwd_workspace_bytes", "gdr_chunk_bwd"])


def test_library_exports_every_declared_symbol():
    gdr, L = _lib()
    out = subprocess.run(["nm", "-D", "--defined-only", gdr.lib_path], capture_output=True,
                         text=True, check=True).stdout
    exported = set(re.findall(r"\bT\s+(gdr_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(L, name)
    assert L.gdr_abi_version() == gdr.ABI_VERSION == 7


def test_args_struct_matches_header_field_order():
    import gated_delta_rule_gdr_amd as gdr
    text = open(HEADER).read()
    body = text[text.index("typedef struct gdr_args {") + 25:text.index("} gdr_args;")]
    body = re.sub(r"/\*.*?\*/", "", body, flags=re.S)
    fields = []
    for decl in body.split(";"):
        for part in decl.split(","):
            ids = re.findall(r"\w+", part)
            if ids:
                fields.append(ids[-1])
    names = [f[0] for f in gdr.Args._fields_]
    assert fields == names


def _valid_args(gdr):
    a = gdr.Args()
    a.q = a.k = a.v = 0x1000
    a.o = 0x900000
    a.g, a.beta = 0x2000, 0x3000
    a.state_pool = 0x4000000
    a.slot_idx, a.cu_seqlens = 0x5000, 0x6000
    a.q_stride_t = a.k_stride_t = 2 * 128
    a.v_stride_t = 4 * 128
    a.in_dtype, a.out_dtype, a.state_dtype = 1, 0, 0
    a.num_slots = 4
    a.N, a.HK, a.HV, a.DK, a.DV = 2, 2, 4, 128, 128
    a.T_total = 8
    a.scale = 128 ** -0.5
    a.chunk_size = 64
    a.rule, a.gate, a.flags = 0, 1, 0
    return a


CASES = [
    ("HV % HK", dict(HV=3), 1),
    ("bad head dim", dict(DK=96, DV=96), 2),
    ("DK != DV", dict(DV=64), 2),
    ("chunk size", dict(chunk_size=48), 2),
    ("null beta (delta)", dict(beta=None), 1),
    ("null g (gated)", dict(g=None), 1),
    ("null q", dict(q=None), 1),
    ("null pool", dict(state_pool=None), 1),
    ("null cu_seqlens", dict(cu_seqlens=None), 1),
    ("short stride", dict(q_stride_t=100), 1),
    ("too few slots", dict(num_slots=1), 1),
    ("unknown dtype", dict(in_dtype=7), 1),
    ("unknown rule", dict(rule=5), 1),
    ("unknown gate", dict(gate=9), 1),
    ("unknown flag", dict(flags=0x80), 1),
    ("nan scale", dict(scale=float("nan")), 1),
    ("negative N", dict(N=-1), 1),
    ("o aliases q", dict(o=0x1000 + 64), 1),
    ("o aliases pool", dict(o=0x4000000 + 4096), 1),
    ("misaligned q", dict(q=0x1008), 1),
    ("misaligned g", dict(g=0x2004), 1),
    ("misaligned pool", dict(state_pool=0x4000008), 1),
    ("negative products", dict(products=-1), 1),
    ("too many products", dict(products=9), 1),
    ("stride not 16 bytes", dict(k_stride_t=2 * 128 + 4), 1),
]


@pytest.mark.parametrize("name,change,status", CASES, ids=[c[0] for c in CASES])
def test_chunk_fwd_rejects_on_host(name, change, status):
    gdr, L = _lib()
    a = _valid_args(gdr)
    for k, v in change.items():
        setattr(a, k, v)
    s = L.gdr_chunk_fwd(ctypes.byref(a), None, 0, None)
    assert s == status, (name, L.gdr_last_error())
    assert L.gdr_last_error().decode()


def test_l2norm_flag_only_for_the_ragged_recurrence():
    gdr, L = _lib()
    a = _valid_args(gdr)
    a.flags = gdr.FLAG_QK_L2NORM
    assert L.gdr_chunk_fwd(ctypes.byref(a), None, 0, None) == 2
    b = _valid_args(gdr)
    b.T_total = 2
    b.flags = gdr.FLAG_QK_L2NORM
    assert L.gdr_recurrent_step(ctypes.byref(b), None) == 2
    c = _valid_args(gdr)
    c.flags = 0x80
    assert L.gdr_recurrent_fwd(ctypes.byref(c), None) == 1   # unknown bit
    d = _valid_args(gdr)
    d.cu_seqlens = None
    assert L.gdr_recurrent_fwd(ctypes.byref(d), None) == 1   # ragged batch needs offsets


def test_recurrent_step_rejects_on_host():
    gdr, L = _lib()
    a = _valid_args(gdr)
    assert L.gdr_recurrent_step(ctypes.byref(a), None) == 1   # T_total != N
    a.T_total = 2
    a.HV = 3
    assert L.gdr_recurrent_step(ctypes.byref(a), None) == 1
    assert L.gdr_recurrent_step(None, None) == 1


def test_empty_batch_is_a_no_op():
    gdr, L = _lib()
    a = _valid_args(gdr)
    a.N, a.T_total = 0, 0
    a.q = a.k = a.v = a.o = a.state_pool = a.slot_idx = a.cu_seqlens = None
    assert L.gdr_chunk_fwd(ctypes.byref(a), None, 0, None) == 0
    assert L.gdr_recurrent_step(ctypes.byref(a), None) == 0
    assert L.gdr_recurrent_fwd(ctypes.byref(a), None) == 0
    assert L.gdr_chunk_fwd_workspace_bytes(ctypes.byref(a)) == 0


def test_channel_gate_workspace_on_host():
    """bf16 inputs with the channel gate pass per-chunk records through the
    workspace: the preferred size is the fp32 carry of
    every (sequence, head) plus whole rows of (chunk, head) records, and a
    missing, short or misaligned workspace is rejected before any launch."""
    gdr, L = _lib()
    a = _valid_args(gdr)
    assert L.gdr_chunk_fwd_workspace_bytes(ctypes.byref(a)) == 0   # scalar gate: fused
    a.gate = 2
    carry = a.N * a.HV * 128 * 128 * 4
    record = 3 * 16 * 2048 + 2 * 6 * 2048 + 4 * 128   # W, Q, K_r^T; T', A; gamma
    flat = (a.T_total + 63) // 64 + a.N
    want = carry + flat * a.HV * record
    assert L.gdr_chunk_fwd_workspace_bytes(ctypes.byref(a)) == want
    assert L.gdr_chunk_fwd(ctypes.byref(a), None, 0, None) == 3
    assert L.gdr_chunk_fwd(ctypes.byref(a), 0x10000000, carry + a.HV * record - 1, None) == 3
    assert L.gdr_chunk_fwd(ctypes.byref(a), 0x10000010, want, None) == 1
    a.rule = 1   # GLA's linear rule takes the same records (T' = I, W = 0)
    assert L.gdr_chunk_fwd_workspace_bytes(ctypes.byref(a)) == want
    a.products = 2   # Gated DeltaProduct runs fused on the general kernel
    assert L.gdr_chunk_fwd_workspace_bytes(ctypes.byref(a)) == 0


def test_status_strings():
    gdr, L = _lib()
    for s in range(6):
        assert L.gdr_status_string(s).decode()
    assert L.gdr_status_string(0) == b"ok"


def test_binding_fails_loudly_without_library(tmp_path, monkeypatch):
    import gated_delta_rule_gdr_amd as gdr
    monkeypatch.setattr(gdr, "lib_path", str(tmp_path / "missing.so"))
    monkeypatch.setattr(gdr, "_lib", None)
    with pytest.raises(ImportError):
        gdr.load()


def test_binding_checks_product_rows():
    """k, v and beta must carry T * products rows (checked before any call)."""
    import torch
    import gated_delta_rule_gdr_amd as gdr
    T, P = 4, 2
    q = torch.zeros(T, 1, 64)
    k = torch.zeros(T, 1, 64)
    v = torch.zeros(T * P, 1, 64)
    beta = torch.zeros(T * P, 1)
    pool = torch.zeros(1, 1, 64, 64)
    with pytest.raises(ValueError, match="T \\* products"):
        gdr.recurrent_fwd(q, k, v, None, beta, pool, torch.zeros(1, dtype=torch.int32),
                          torch.tensor([0, T], dtype=torch.int32), gate="none", products=P)



def test_linear_backward_rejects_on_host():
    """The backward covers the linear rule, plain (gdr_linear_chunk_bwd) or
    with a scalar gate (gdr_gated_linear_chunk_bwd), with grouped key heads;
    it checks its outputs, their overlaps and the workspace before any
    launch."""
    gdr, L = _lib()
    a = _valid_args(gdr)
    a.rule, a.gate, a.HV, a.beta, a.g = 1, 0, 2, None, None
    a.v_stride_t = 2 * 128
    need = L.gdr_linear_chunk_bwd_workspace_bytes(ctypes.byref(a))
    rows = a.T_total * 2 * 128
    assert need >= a.N * 2 * 128 * 128 * 4 + a.N * 4   # bf16: scratch pool and slots only
    a.in_dtype = 0                                     # fp32 inputs: reversed copies as well
    assert L.gdr_linear_chunk_bwd_workspace_bytes(ctypes.byref(a)) >= 4 * rows * 4 + rows * 4 + need
    a.in_dtype = 1
    dout, dq, dk, dv, dg, ws = 0x7000000, 0x8000000, 0x8100000, 0x8200000, 0x8300000, 0x10000000
    call = lambda aa, **kw: L.gdr_linear_chunk_bwd(
        ctypes.byref(aa), kw.get("dout", dout), kw.get("dq", dq), kw.get("dk", dk), kw.get("dv", dv),
        kw.get("ws", ws), kw.get("wsb", need), None)
    gcall = lambda aa, **kw: L.gdr_gated_linear_chunk_bwd(
        ctypes.byref(aa), kw.get("dout", dout), kw.get("dq", dq), kw.get("dk", dk), kw.get("dv", dv),
        kw.get("dg", dg), kw.get("ws", ws), kw.get("wsb", need), None)
    assert call(a, ws=None) == 3                      # no workspace
    assert call(a, wsb=need - 1) == 3                 # short workspace
    assert call(a, ws=ws + 16) == 1                   # misaligned workspace
    assert call(a, dk=None) == 1
    assert call(a, dv=dq + 64) == 1                   # outputs overlap
    assert call(a, dq=0x1000) == 1                    # dq overlaps q
    assert call(a, dout=dout + 4) == 1                # misaligned dout
    assert gcall(a) == 2                              # the gated entry wants a gate
    b = _valid_args(gdr)                              # delta rule, scalar gate
    assert L.gdr_linear_chunk_bwd_workspace_bytes(ctypes.byref(b)) == 0
    assert call(b) == 2
    assert gcall(b) == 2
    # grouped heads (HV = 2 HK): q and k repeated per value head, fp32 dq, dk
    # per value head
    a.HV, a.v_stride_t = 4, 4 * 128
    grouped = L.gdr_linear_chunk_bwd_workspace_bytes(ctypes.byref(a))
    vrows = a.T_total * 4 * 128
    assert grouped >= need + 2 * vrows * 2 + 2 * vrows * 4
    assert call(a, wsb=grouped - 1) == 3
    assert call(a, dq=dv + 64, wsb=grouped) == 1      # dq overlaps dv
    # the scalar gate: the plain entry refuses it (it has no dg), the gated
    # one checks dg
    a.gate, a.g = 1, 0x2000
    gated = L.gdr_linear_chunk_bwd_workspace_bytes(ctypes.byref(a))
    assert gated >= grouped + 2 * a.T_total * 4 * 4
    assert call(a, wsb=gated) == 2
    assert gcall(a, dg=None, wsb=gated) == 1
    assert gcall(a, dg=dg + 2, wsb=gated) == 1        # misaligned dg
    assert gcall(a, dg=0x2000 + 4, wsb=gated) == 1    # dg overlaps g
    assert gcall(a, dg=dv, wsb=gated) == 1            # dg overlaps dv
    assert gcall(a, wsb=gated - 1) == 3
    a.gate = 2                                        # channel gate
    assert L.gdr_linear_chunk_bwd_workspace_bytes(ctypes.byref(a)) == 0
    assert gcall(a, wsb=gated) == 2
    a.gate, a.products = 1, 2                         # several transitions per token
    assert gcall(a, wsb=gated) == 2


def test_chunk_backward_rejects_on_host():
    """gdr_chunk_bwd takes the delta rule with gate NONE or SCALAR (the
    tokenwise backward's other checks apply too) and checks its workspace
    before any launch."""
    gdr, L = _lib()
    a = _valid_args(gdr)                              # delta rule, scalar gate, HV = 2 HK
    need = L.gdr_chunk_bwd_workspace_bytes(ctypes.byref(a))
    flat = (a.T_total + 63) // 64 + a.N
    mat = flat * a.HV * 128 * 128 * 4
    rows = a.T_total * a.HV * 128 * 4
    assert need >= 4 * mat + 2 * rows
    dout, dq, dk, dv, db, dg, ds, ws = (0x7000000, 0x8000000, 0x8100000, 0x8200000, 0x8300000, 0x8400000,
                                        0x9000000, 0x10000000)
    call = lambda aa, **kw: L.gdr_chunk_bwd(
        ctypes.byref(aa), dout, dq, dk, dv, kw.get("db", db), kw.get("dg", dg), ds, kw.get("ws", ws),
        kw.get("wsb", need), None)
    assert call(a, ws=None) == 3
    assert call(a, wsb=need - 1) == 3
    assert call(a, ws=ws + 16) == 1
    assert call(a, db=None) == 1                      # dbeta is required for the delta rule
    assert call(a, dg=None) == 1                      # dg is required for a gated call
    b = _valid_args(gdr)
    b.rule, b.beta = 1, None                          # the linear rule has its own chunkwise backward
    assert L.gdr_chunk_bwd_workspace_bytes(ctypes.byref(b)) == 0
    assert call(b) == 2
    c = _valid_args(gdr)
    c.gate = 2                                        # channel gate
    assert L.gdr_chunk_bwd_workspace_bytes(ctypes.byref(c)) == 0
    assert call(c) == 2


def test_recurrent_backward_rejects_on_host():
    """The tokenwise backward takes any rule and gate; it checks the gradients'
    buffers, their overlaps, the workspace, L2 norm and products before any
    launch."""
    gdr, L = _lib()
    a = _valid_args(gdr)                              # delta rule, scalar gate, HK 2, HV 4
    need = L.gdr_recurrent_bwd_workspace_bytes(ctypes.byref(a))
    slots = a.T_total // 8 + a.N + 1
    assert need >= slots * 4 * 128 * 128 * 4 + a.T_total * 4 * 4 * 2 * 128 * 4
    bufs = dict(dout=0x7000000, dq=0x8000000, dk=0x8100000, dv=0x8200000, dbeta=0x8300000,
                dg=0x8400000, ds=0x8500000, ws=0x10000000)
    call = lambda aa, **kw: L.gdr_recurrent_bwd(
        ctypes.byref(aa), *[kw.get(n, bufs[n]) for n in ("dout", "dq", "dk", "dv", "dbeta", "dg", "ds", "ws")],
        kw.get("wsb", need), None)
    assert call(a, ws=None) == 3                      # no workspace
    assert call(a, wsb=need - 1) == 3                 # short workspace
    assert call(a, ws=bufs["ws"] + 16) == 1           # misaligned workspace
    assert call(a, dbeta=None) == 1                   # delta rule needs dbeta
    assert call(a, dg=None) == 1                      # gated call needs dg
    assert call(a, dq=None) == 1
    assert call(a, dk=bufs["dq"] + 64) == 1           # gradients overlap
    assert call(a, dg=0x2000) == 1                    # dg overlaps g
    assert call(a, ds=0x4000000) == 1                 # dstate0 overlaps the pool
    assert call(a, dout=bufs["dout"] + 4) == 1        # misaligned dout
    b = _valid_args(gdr)
    b.flags = gdr.FLAG_QK_L2NORM
    assert call(b) == 2
    b = _valid_args(gdr)
    b.products = 2
    assert call(b) == 2
    b = _valid_args(gdr)                              # the linear rule ignores dbeta
    b.rule, b.gate, b.beta, b.g = 1, 0, None, None
    nb = L.gdr_recurrent_bwd_workspace_bytes(ctypes.byref(b))
    assert nb == need                                 # two partial-sum vectors per token either way
    b.gate, b.g = 2, 0x2000
    assert L.gdr_recurrent_bwd_workspace_bytes(ctypes.byref(b)) > nb   # a third (dg per column)
    b.N = 0
    assert L.gdr_recurrent_bwd_workspace_bytes(ctypes.byref(b)) == 0


def test_verify_ring_and_fold_on_host():
    """Record sizes by gate, and the host checks of the verify and the fold."""
    gdr, L = _lib()
    a = _valid_args(gdr)
    for gate, elems in ((0, 256), (1, 257), (2, 384)):
        a.gate = gate
        assert L.gdr_ring_record_elements(ctypes.byref(a)) == elems
        assert L.gdr_ring_record_stride(ctypes.byref(a)) == (elems + 3) // 4 * 4
    a.gate = 1
    assert L.gdr_verify_ring(ctypes.byref(a), None, None) == 1            # no ring
    assert L.gdr_verify_ring(ctypes.byref(a), 0x20000004, None) == 1      # misaligned
    assert L.gdr_verify_ring(ctypes.byref(a), 0x1000, None) == 1          # overlaps q
    a.products = 2
    assert L.gdr_verify_ring(ctypes.byref(a), 0x20000000, None) == 2
    a.products = 1
    assert L.gdr_state_fold(ctypes.byref(a), None, 0x30000000, None) == 1
    assert L.gdr_state_fold(ctypes.byref(a), 0x20000000, None, None) == 1
    a.DK = 96
    assert L.gdr_state_fold(ctypes.byref(a), 0x20000000, 0x30000000, None) == 2
