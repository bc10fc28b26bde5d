"""gated_delta_rule_gdr_amd: the gated delta rule forward pass on AMD MI355X.

A thin ctypes binding over libgdr.so (include/gdr.h). Argument marshalling
only: every step of the computation runs in the library's HIP kernels, torch
supplies device memory and the current HIP stream. There is no CPU fallback:
if the library is missing, importing the binding works but every call raises.

    o = chunk_fwd(q, k, v, g, beta, pool, slot_idx, cu_seqlens)
    o = recurrent_fwd(q, k, v, g, beta, pool, slot_idx, cu_seqlens, qk_l2norm=False)
    o = recurrent_step(q, k, v, g, beta, pool, slot_idx)

Layouts (torch tensors on the GPU):
    q, k   [T, HK, DK]  bf16 or fp32 (a strided token dimension is allowed, e.g.
           views into one fused qkv buffer; heads and dims must be contiguous)
    v      [T, HV, DV]  same dtype as q, k
    g      [T, HV] (scalar gate) | [T, HV, DK] (channel gate) | None, fp32, log alpha
    beta   [T, HV] fp32 (delta rule) | None (linear rule)
    pool   [num_slots, HV, DK, DV] fp32 or bf16, S^T per slot, updated in place
    slot_idx [N] int32, cu_seqlens [N+1] int32 (prefill)
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_workspace_bytes", "recurrent_step", "recurrent_fwd", "linear_chunk_bwd", "chunk_bwd", "recurrent_bwd",
           "verify_ring", "state_fold", "lib", "lib_path", "GdrError",
           "abi_version", "Args", "load"]

_HERE = os.path.dirname(os.path.abspath(__file__))
lib_path = os.path.join(_HERE, "libgdr.so")

GDR_OK = 0
_DT = {"f32": 0, "bf16": 1}
_RULE = {"delta": 0, "linear": 1}
_GATE = {"none": 0, "scalar": 1, "channel": 2}
FLAG_ZERO_INIT = 1
FLAG_DEBUG_CHECKS = 2
FLAG_QK_L2NORM = 4


# GDR_ABI_VERSION of include/gdr.h that Args mirrors.
ABI_VERSION = 7


class GdrError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"gdr status {status}: {msg}")
        self.status = status


class Args(ctypes.Structure):
    """Mirror of gdr_args (include/gdr.h)."""
    _fields_ = [
        ("q", ctypes.c_void_p), ("k", ctypes.c_void_p), ("v", ctypes.c_void_p),
        ("q_stride_t", ctypes.c_int64), ("k_stride_t", ctypes.c_int64),
        ("v_stride_t", ctypes.c_int64),
        ("in_dtype", ctypes.c_int),
        ("g", ctypes.c_void_p), ("beta", ctypes.c_void_p),
        ("o", ctypes.c_void_p), ("out_dtype", ctypes.c_int),
        ("state_pool", ctypes.c_void_p), ("state_dtype", ctypes.c_int),
        ("num_slots", ctypes.c_int64),
        ("slot_idx", ctypes.c_void_p), ("cu_seqlens", ctypes.c_void_p),
        ("N", ctypes.c_int32), ("HK", ctypes.c_int32), ("HV", ctypes.c_int32),
        ("DK", ctypes.c_int32), ("DV", ctypes.c_int32),
        ("T_total", ctypes.c_int64),
        ("scale", ctypes.c_float),
        ("chunk_size", ctypes.c_int32),
        ("rule", ctypes.c_int), ("gate", ctypes.c_int),
        ("flags", ctypes.c_uint32),
        ("products", ctypes.c_int32),
    ]


_lib = None


def load() -> ctypes.CDLL:
    """Load libgdr.so from this package directory (raises if it is absent)."""
    global _lib
    if _lib is not None:
        return _lib
    # torch first: the library then binds to the HIP runtime torch has already
    # loaded, the one that owns the streams and memory it is handed (loaded
    # first, it could bind another copy, on which torch's streams mean nothing)
    import torch  # noqa: F401
    if not os.path.exists(lib_path):
        raise ImportError(
            f"{lib_path} is missing: build it with `python -m gated_delta_rule_gdr_amd.build`")
    L = ctypes.CDLL(lib_path)
    L.gdr_abi_version.restype = ctypes.c_int
    if L.gdr_abi_version() != ABI_VERSION:
        raise ImportError(f"{lib_path} has ABI {L.gdr_abi_version()}, this binding expects "
                          f"{ABI_VERSION}: rebuild it")
    L.gdr_chunk_fwd_workspace_bytes.restype = ctypes.c_size_t
    L.gdr_chunk_fwd_workspace_bytes.argtypes = [ctypes.POINTER(Args)]
    L.gdr_chunk_fwd.restype = ctypes.c_int
    L.gdr_chunk_fwd.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p, ctypes.c_size_t,
                                ctypes.c_void_p]
    L.gdr_chunk_fwd_noalloc.restype = ctypes.c_int
    L.gdr_chunk_fwd_noalloc.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p]
    L.gdr_recurrent_step.restype = ctypes.c_int
    L.gdr_recurrent_step.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p]
    L.gdr_recurrent_fwd.restype = ctypes.c_int
    L.gdr_recurrent_fwd.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p]
    L.gdr_linear_chunk_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.gdr_linear_chunk_bwd_workspace_bytes.argtypes = [ctypes.POINTER(Args)]
    L.gdr_linear_chunk_bwd.restype = ctypes.c_int
    L.gdr_linear_chunk_bwd.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                       ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    L.gdr_gated_linear_chunk_bwd.restype = ctypes.c_int
    L.gdr_gated_linear_chunk_bwd.argtypes = [ctypes.POINTER(Args)] + [ctypes.c_void_p] * 6 + [ctypes.c_size_t,
                                                                                            ctypes.c_void_p]
    for name in ("gdr_recurrent_bwd", "gdr_chunk_bwd"):
        getattr(L, name + "_workspace_bytes").restype = ctypes.c_size_t
        getattr(L, name + "_workspace_bytes").argtypes = [ctypes.POINTER(Args)]
        getattr(L, name).restype = ctypes.c_int
        getattr(L, name).argtypes = [ctypes.POINTER(Args)] + [ctypes.c_void_p] * 8 + [ctypes.c_size_t,
                                                                                     ctypes.c_void_p]
    L.gdr_recurrent_bwd_workspace_bytes.restype = ctypes.c_size_t
    L.gdr_recurrent_bwd_workspace_bytes.argtypes = [ctypes.POINTER(Args)]
    L.gdr_recurrent_bwd.restype = ctypes.c_int
    L.gdr_recurrent_bwd.argtypes = [ctypes.POINTER(Args)] + [ctypes.c_void_p] * 8 + [ctypes.c_size_t,
                                                                                   ctypes.c_void_p]
    L.gdr_ring_record_elements.restype = ctypes.c_int
    L.gdr_ring_record_elements.argtypes = [ctypes.POINTER(Args)]
    L.gdr_ring_record_stride.restype = ctypes.c_int
    L.gdr_ring_record_stride.argtypes = [ctypes.POINTER(Args)]
    L.gdr_verify_ring.restype = ctypes.c_int
    L.gdr_verify_ring.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p, ctypes.c_void_p]
    L.gdr_state_fold.restype = ctypes.c_int
    L.gdr_state_fold.argtypes = [ctypes.POINTER(Args), ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    L.gdr_status_string.restype = ctypes.c_char_p
    L.gdr_status_string.argtypes = [ctypes.c_int]
    L.gdr_last_error.restype = ctypes.c_char_p
    _lib = L
    return L


def lib() -> ctypes.CDLL:
    return load()


def abi_version() -> int:
    return load().gdr_abi_version()


def _check(status: int):
    if status != GDR_OK:
        L = load()
        raise GdrError(status, f"{L.gdr_status_string(status).decode()}: "
                               f"{L.gdr_last_error().decode()}")


def _dt(t) -> int:
    import torch
    if t.dtype == torch.bfloat16:
        return _DT["bf16"]
    if t.dtype == torch.float32:
        return _DT["f32"]
    raise TypeError(f"unsupported dtype {t.dtype}")


def _tok_stride(t, name: str) -> int:
    """Token stride of a [T, H, D] tensor whose (H, D) block is contiguous."""
    if t.dim() != 3:
        raise ValueError(f"{name} must be [T, H, D], got {tuple(t.shape)}")
    H, D = t.shape[1], t.shape[2]
    if t.shape[0] > 0 and not (t.stride(2) == 1 and t.stride(1) == D):
        raise ValueError(f"{name}: heads and dims must be contiguous")
    return t.stride(0) if t.shape[0] > 1 else H * D


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _prepare(q, k, v, g, beta, pool, slot_idx, cu_seqlens, o, scale, rule, gate,
             zero_init, debug_checks, chunk_size, out_dtype, products=1):
    import torch
    T, HK, DK = q.shape
    HV, DV = v.shape[1], v.shape[2]
    P = max(int(products), 1)
    if k.shape[0] != T * P or v.shape[0] != T * P or (beta is not None and beta.shape[0] != T * P):
        raise ValueError(f"k, v and beta need T * products = {T * P} rows (q has {T} tokens)")
    if gate is None:
        gate = "none" if g is None else ("channel" if g.dim() == 3 else "scalar")
    if scale is None:
        scale = DK ** -0.5
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v), ("pool", pool), ("slot_idx", slot_idx)):
        if t.device != dev:
            raise ValueError(f"{name} is on {t.device}, q on {dev}")
    if slot_idx.dtype != torch.int32 or not slot_idx.is_contiguous():
        raise TypeError("slot_idx must be a contiguous int32 tensor")
    if cu_seqlens is not None and (cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous()):
        raise TypeError("cu_seqlens must be a contiguous int32 tensor")
    for name, t in (("g", g), ("beta", beta)):
        if t is not None and (t.dtype != torch.float32 or not t.is_contiguous() or t.device != dev):
            raise TypeError(f"{name} must be a contiguous fp32 tensor on {dev}")
    if not pool.is_contiguous():
        raise ValueError("pool must be contiguous")
    if o is None:
        o = torch.empty((T, HV, DV), dtype=out_dtype, device=dev)
    elif not o.is_contiguous() or tuple(o.shape) != (T, HV, DV):
        raise ValueError("o must be a contiguous [T, HV, DV] tensor")
    a = Args()
    a.q, a.k, a.v = _ptr(q), _ptr(k), _ptr(v)
    a.q_stride_t = _tok_stride(q, "q")
    a.k_stride_t = _tok_stride(k, "k")
    a.v_stride_t = _tok_stride(v, "v")
    a.in_dtype = _dt(q)
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise TypeError("q, k, v must share a dtype")
    a.g, a.beta = _ptr(g), _ptr(beta)
    a.o, a.out_dtype = _ptr(o), _dt(o)
    a.state_pool, a.state_dtype = _ptr(pool), _dt(pool)
    a.num_slots = pool.shape[0]
    a.slot_idx = _ptr(slot_idx)
    a.cu_seqlens = _ptr(cu_seqlens)
    a.N = slot_idx.shape[0]
    a.HK, a.HV, a.DK, a.DV = HK, HV, DK, DV
    a.T_total = T
    a.scale = float(scale)
    a.chunk_size = chunk_size
    a.rule = _RULE[rule]
    a.gate = _GATE[gate]
    a.flags = (FLAG_ZERO_INIT if zero_init else 0) | (FLAG_DEBUG_CHECKS if debug_checks else 0)
    a.products = P
    if tuple(pool.shape[1:]) != (HV, DK, DV):
        raise ValueError(f"pool must be [slots, {HV}, {DK}, {DV}], got {tuple(pool.shape)}")
    return a, o


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def chunk_fwd(q, k, v, g, beta, pool, slot_idx, cu_seqlens, *, scale=None, chunk_size=64,
              rule="delta", gate=None, out_dtype=None, zero_init=False, o=None,
              debug_checks=False, workspace=None, products=1):
    """Chunkwise prefill; returns o [T, HV, DV]; updates pool slots in place.

    ``chunk_size`` is the chunk length, 16, 32 or 64 tokens (the same
    recurrence up to rounding; 64 runs the tuned kernels). ``workspace`` is an
    optional uint8 device tensor for the calls that need one
    (gdr_chunk_fwd_workspace_bytes > 0: the channel gate with bf16 inputs at
    chunk_size 64); by default one of the preferred size is allocated from
    torch's allocator.
    """
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    a, o = _prepare(q, k, v, g, beta, pool, slot_idx, cu_seqlens, o, scale, rule, gate,
                    zero_init, debug_checks, chunk_size, out_dtype, products)
    L = load()
    if workspace is None:
        nbytes = L.gdr_chunk_fwd_workspace_bytes(ctypes.byref(a))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    if workspace is not None:
        if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
            raise TypeError(f"workspace must be a contiguous uint8 tensor on {q.device}")
        wptr, wbytes = workspace.data_ptr(), workspace.numel()
    else:
        wptr, wbytes = None, 0
    _check(L.gdr_chunk_fwd(ctypes.byref(a), wptr, wbytes, _stream(q)))
    return o


def chunk_fwd_noalloc(q, k, v, g, beta, pool, slot_idx, cu_seqlens, *, scale=None, chunk_size=64,
                      rule="delta", gate=None, out_dtype=None, zero_init=False, o=None,
                      debug_checks=False, products=1):
    """chunk_fwd through gdr_chunk_fwd_noalloc: the library's static device
    scratch instead of a workspace (pass ``o`` to allocate nothing at all)."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    a, o = _prepare(q, k, v, g, beta, pool, slot_idx, cu_seqlens, o, scale, rule, gate,
                    zero_init, debug_checks, chunk_size, out_dtype, products)
    _check(load().gdr_chunk_fwd_noalloc(ctypes.byref(a), _stream(q)))
    return o


def chunk_fwd_workspace_bytes(q, k, v, g, beta, pool, slot_idx, cu_seqlens, *, scale=None,
                              chunk_size=64, rule="delta", gate=None, out_dtype=None,
                              zero_init=False, products=1):
    """Preferred workspace size in bytes of the matching chunk_fwd call (0: none needed)."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    a, _ = _prepare(q, k, v, g, beta, pool, slot_idx, cu_seqlens, None, scale, rule, gate,
                    zero_init, False, chunk_size, out_dtype, products)
    return int(load().gdr_chunk_fwd_workspace_bytes(ctypes.byref(a)))


def recurrent_step(q, k, v, g, beta, pool, slot_idx, *, scale=None, rule="delta", gate=None,
                   out_dtype=None, zero_init=False, o=None, debug_checks=False, products=1):
    """One token per sequence (q: [N, HK, DK]; k, v, beta: N * products rows);
    returns o [N, HV, DV]."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    a, o = _prepare(q, k, v, g, beta, pool, slot_idx, None, o, scale, rule, gate,
                    zero_init, debug_checks, 64, out_dtype, products)
    L = load()
    _check(L.gdr_recurrent_step(ctypes.byref(a), _stream(q)))
    return o


def recurrent_fwd(q, k, v, g, beta, pool, slot_idx, cu_seqlens, *, scale=None, rule="delta",
                  gate=None, out_dtype=None, zero_init=False, o=None, debug_checks=False,
                  qk_l2norm=False, products=1):
    """Tokenwise recurrence over a ragged batch (the state on chip across each
    sequence); same results as chunk_fwd. qk_l2norm normalises q and k per
    token and key head inside the kernel. Returns o [T, HV, DV]."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    a, o = _prepare(q, k, v, g, beta, pool, slot_idx, cu_seqlens, o, scale, rule, gate,
                    zero_init, debug_checks, 64, out_dtype, products)
    if qk_l2norm:
        a.flags |= FLAG_QK_L2NORM
    L = load()
    _check(L.gdr_recurrent_fwd(ctypes.byref(a), _stream(q)))
    return o


def linear_chunk_bwd(q, k, v, do, pool, slot_idx, cu_seqlens, *, g=None, scale=None, zero_init=False,
                     out_dtype=None, workspace=None, debug_checks=False):
    """Gradients of causal linear attention (no delta), plain or with a
    scalar gate g (the log-decay, fp32 [T, HV]), with grouped key heads
    (HV a multiple of HK), for the forward call with these arguments and
    upstream gradient do [T, HV, DV] (contiguous, q's dtype). The pool
    supplies the initial state (read only) unless zero_init. Returns
    (dq, dk, dv), and with g also dg (fp32 [T, HV], the gradient of the
    log-decays). ``workspace`` is an optional uint8 device tensor of at least
    the size the library asks for (allocated from torch by default)."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    T, HK, DK = q.shape
    gated = g is not None
    if gated and g.dim() != 2:
        raise ValueError("the backward takes the scalar gate, g [T, HV]")
    dv = torch.empty(tuple(v.shape), dtype=out_dtype, device=q.device)
    a, _ = _prepare(q, k, v, g, None, pool, slot_idx, cu_seqlens, dv, scale, "linear",
                    "scalar" if gated else "none", zero_init, debug_checks, 64, out_dtype)
    if do.dtype != q.dtype or not do.is_contiguous() or tuple(do.shape) != tuple(v.shape) or do.device != q.device:
        raise ValueError("do must be a contiguous tensor shaped like v, in q's dtype, on q's device")
    dq = torch.empty((T, HK, DK), dtype=out_dtype, device=q.device)
    dk = torch.empty_like(dq)
    dg = torch.empty(tuple(g.shape), dtype=torch.float32, device=q.device) if gated else None
    L = load()
    if workspace is None:
        nbytes = L.gdr_linear_chunk_bwd_workspace_bytes(ctypes.byref(a))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise TypeError(f"workspace must be a contiguous uint8 tensor on {q.device}")
    if gated:
        _check(L.gdr_gated_linear_chunk_bwd(ctypes.byref(a), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                            dv.data_ptr(), dg.data_ptr(), workspace.data_ptr(),
                                            workspace.numel(), _stream(q)))
        return dq, dk, dv, dg
    _check(L.gdr_linear_chunk_bwd(ctypes.byref(a), do.data_ptr(), dq.data_ptr(), dk.data_ptr(),
                                  dv.data_ptr(), workspace.data_ptr(), workspace.numel(), _stream(q)))
    return dq, dk, dv


def recurrent_bwd(q, k, v, g, beta, do, pool, slot_idx, cu_seqlens, *, scale=None, rule="delta",
                  gate=None, zero_init=False, out_dtype=None, dstate0=True, workspace=None,
                  debug_checks=False):
    """Gradients of the tokenwise recurrence (any rule and gate) for the
    forward call with these arguments and upstream gradient do [T, HV, DV]
    (contiguous, q's dtype). Returns a dict with dq, dk [T, HK, DK] and dv
    [T, HV, DV] (out_dtype), dbeta [T, HV] (delta rule), dg shaped like g
    (gated calls) and dstate0 [N, HV, DK, DV] fp32 (the initial state's
    gradient, transposed like the pool) unless ``dstate0`` is False; absent
    entries are None. The pool is read, never written."""
    return _grads("gdr_recurrent_bwd", q, k, v, g, beta, do, pool, slot_idx, cu_seqlens, scale, rule, gate,
                  zero_init, out_dtype, dstate0, workspace, debug_checks)


def chunk_bwd(q, k, v, g, beta, do, pool, slot_idx, cu_seqlens, *, scale=None, gate=None, zero_init=False,
              out_dtype=None, dstate0=True, workspace=None, debug_checks=False):
    """The same gradients as recurrent_bwd for the delta rule with gate
    "none" or "scalar", computed chunkwise (gdr_chunk_bwd): a scan of the
    state's gradient over the chunk boundaries, then every chunk on its
    own. Same arguments and result."""
    return _grads("gdr_chunk_bwd", q, k, v, g, beta, do, pool, slot_idx, cu_seqlens, scale, "delta", gate,
                  zero_init, out_dtype, dstate0, workspace, debug_checks)


def _grads(entry, q, k, v, g, beta, do, pool, slot_idx, cu_seqlens, scale, rule, gate, zero_init, out_dtype,
           dstate0, workspace, debug_checks):
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    T, HK, DK = q.shape
    dv = torch.empty(tuple(v.shape), dtype=out_dtype, device=q.device)
    a, _ = _prepare(q, k, v, g, beta, pool, slot_idx, cu_seqlens, dv, scale, rule, gate,
                    zero_init, debug_checks, 64, out_dtype)
    if do.dtype != q.dtype or not do.is_contiguous() or tuple(do.shape) != tuple(v.shape) or do.device != q.device:
        raise ValueError("do must be a contiguous tensor shaped like v, in q's dtype, on q's device")
    dq = torch.empty((T, HK, DK), dtype=out_dtype, device=q.device)
    dk = torch.empty_like(dq)
    f32 = dict(dtype=torch.float32, device=q.device)
    dbeta = torch.empty((T, v.shape[1]), **f32) if rule == "delta" else None
    dg = torch.empty(tuple(g.shape), **f32) if g is not None and a.gate != 0 else None
    ds = torch.empty((slot_idx.shape[0], v.shape[1], DK, v.shape[2]), **f32) if dstate0 else None
    L = load()
    if workspace is None:
        nbytes = getattr(L, entry + "_workspace_bytes")(ctypes.byref(a))
        workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    if workspace.dtype != torch.uint8 or not workspace.is_contiguous() or workspace.device != q.device:
        raise TypeError(f"workspace must be a contiguous uint8 tensor on {q.device}")
    ptr = lambda x: None if x is None else x.data_ptr()
    _check(getattr(L, entry)(ctypes.byref(a), do.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                             ptr(dbeta), ptr(dg), ptr(ds), workspace.data_ptr(), workspace.numel(), _stream(q)))
    return dict(dq=dq, dk=dk, dv=dv, dbeta=dbeta, dg=dg, dstate0=ds)


def verify_ring(q, k, v, g, beta, pool, slot_idx, cu_seqlens, *, scale=None, rule="delta", gate=None,
                out_dtype=None, zero_init=False, o=None, debug_checks=False, qk_l2norm=False):
    """Verify of a speculative window: the tokenwise recurrence over each
    sequence's window with the pool left untouched. Returns (o, ring) with
    ring [T, HV, stride] fp32 records (e, k, log-gate) for state_fold."""
    import torch
    out_dtype = torch.float32 if out_dtype is None else out_dtype
    a, o = _prepare(q, k, v, g, beta, pool, slot_idx, cu_seqlens, o, scale, rule, gate,
                    zero_init, debug_checks, 64, out_dtype)
    if qk_l2norm:
        a.flags |= FLAG_QK_L2NORM
    L = load()
    stride = L.gdr_ring_record_stride(ctypes.byref(a))
    ring = torch.empty((q.shape[0], v.shape[1], stride), dtype=torch.float32, device=q.device)
    _check(L.gdr_verify_ring(ctypes.byref(a), ring.data_ptr(), _stream(q)))
    return o, ring


def state_fold(ring, accepted, pool, slot_idx, cu_seqlens, *, HK, gate, debug_checks=False):
    """Apply each sequence's first accepted[n] records of a verify to its pool
    slot in place (accepted: [N] int32 on the device)."""
    import torch
    T, HV, _ = ring.shape
    DK = pool.shape[2]
    if accepted.dtype != torch.int32 or not accepted.is_contiguous():
        raise TypeError("accepted must be a contiguous int32 tensor")
    a = Args()
    a.N, a.HK, a.HV, a.DK, a.DV = slot_idx.shape[0], HK, HV, DK, pool.shape[3]
    a.T_total = T
    a.gate = _GATE[gate]
    a.state_pool, a.state_dtype, a.num_slots = pool.data_ptr(), _dt(pool), pool.shape[0]
    a.slot_idx, a.cu_seqlens = slot_idx.data_ptr(), cu_seqlens.data_ptr()
    a.flags = FLAG_DEBUG_CHECKS if debug_checks else 0
    L = load()
    if ring.shape[2] != L.gdr_ring_record_stride(ctypes.byref(a)):
        raise ValueError("ring does not match these shapes and gate")
    _check(L.gdr_state_fold(ctypes.byref(a), ring.data_ptr(), accepted.data_ptr(), _stream(pool)))
