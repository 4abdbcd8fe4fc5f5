"""Gated delta-rule recurrence on MI355X (gfx950): Python binding of libdr.

``chunk_fwd`` is the prefill / training forward, ``chunk_fwd_varlen`` the same over a packed
batch of sequences of different lengths, and ``decode_step`` the single-token update; all call
the C ABI (include/dr.h) on torch's current HIP stream.  Tensors must live on the
GPU and be contiguous; the functions only check and marshal arguments, allocate outputs with
torch and pass raw device pointers.  No step of the recurrence runs in Python, and there is
no CPU fallback: without the built library every call raises.

The operation (per batch b and head h, state S of dk x dv in fp32):
    S' = Diag(a_t) S,   S = S' - (e_t * k_t)(k_t^T S') + k_t (w_t * v_t)^T,   o_t = S^T q_t
with a_t = exp(log_decay_t).  Gates are per head ([B, T, H]) or per channel ([B, T, H, d]);
``write=None`` means the write gate is the erase gate.  ``fg2=True`` reads ``erase`` as
FG2-GDN's per-channel learning rate beta [.., dk] (dk == dv, ``write=None``), absorbed as
k~ = sqrt(beta) k and v~ = sqrt(beta) v with unit erase and write gates:
    S = (I - k~ k~^T) Diag(a_t) S + k~ v~^T.
"""
from __future__ import annotations

import ctypes

import torch

from . import _abi

__all__ = ["chunk_fwd", "chunk_fwd_noalloc", "chunk_fwd_varlen", "chunk_bwd", "decode_step", "workspace_bytes",
           "varlen_workspace_bytes", "abi_version", "DrError"]

DrError = _abi.DrError


def abi_version() -> int:
    return _abi.lib().dr_abi_version()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _check_tensor(name, t, dtypes, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda" or (device is not None and t.device != device):
        raise ValueError(f"{name} must be on the GPU with the other inputs (got {t.device})")
    if t.dtype not in dtypes:
        raise TypeError(f"{name} has dtype {t.dtype}, expected one of {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _dtype_code(dt):
    if dt == torch.float32:
        return _abi.DR_F32
    if dt == torch.bfloat16:
        return _abi.DR_BF16
    raise TypeError(f"unsupported dtype {dt}")


def _gate_kind(name, g, lead, d):
    if tuple(g.shape) == lead:
        return _abi.DR_GATE_HEAD
    if tuple(g.shape) == lead + (d,):
        return _abi.DR_GATE_CHANNEL
    raise ValueError(f"{name} must have shape {lead} or {lead + (d,)}, got {tuple(g.shape)}")


def _desc(B, T, H, dk, dv, chunk, qkv_dtype, o_dtype, log_decay, erase, write, lead, fg2=False):
    d = _abi.DrDesc()
    d.B, d.T, d.H, d.dk, d.dv, d.chunk = B, T, H, dk, dv, chunk
    d.qkv_dtype = _dtype_code(qkv_dtype)
    d.o_dtype = _dtype_code(o_dtype)
    d.decay_kind = _gate_kind("log_decay", log_decay, lead, dk)
    d.erase_kind = _gate_kind("erase", erase, lead, dk)
    if fg2:
        if d.erase_kind != _abi.DR_GATE_CHANNEL or write is not None:
            raise ValueError("fg2: erase is the per-channel rate beta [.., dk] and write must be None")
        d.erase_kind = _abi.DR_GATE_RATE_SQRT
    if write is None:
        d.write_is_erase, d.write_kind = 1, d.erase_kind
    else:
        d.write_is_erase, d.write_kind = 0, _gate_kind("write", write, lead, dv)
    return d


def workspace_bytes(desc) -> int:
    return int(_abi.lib().dr_chunk_fwd_workspace_bytes(ctypes.byref(desc)))


def chunk_fwd(q, k, v, log_decay, erase, write=None, S0=None, *, chunk=64,
              o_dtype=torch.float32, out=None, S_T=None, return_state=True, fg2=False):
    """Chunked forward over T tokens.

    q, k: [B, T, H, dk]; v: [B, T, H, dv] (bf16 or fp32, same dtype); log_decay, erase:
    [B, T, H] or [B, T, H, dk] fp32; write: None, [B, T, H] or [B, T, H, dv] fp32;
    S0: None or [B, H, dk, dv] fp32.  ``chunk=1`` selects the token-by-token kernel.
    Returns (o [B, T, H, dv], S_T [B, H, dk, dv] or None).  ``out`` / ``S_T`` may supply
    preallocated outputs (S_T may be S0 itself for an in-place carry)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, (torch.float32, torch.bfloat16), dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B, T, H, dk] and v [B, T, H, dv]")
    B, T, H, dk = q.shape
    dv = v.shape[3]
    for name, t in (("log_decay", log_decay), ("erase", erase), ("write", write), ("S0", S0)):
        if t is not None:
            _check_tensor(name, t, (torch.float32,), dev)
    desc = _desc(B, T, H, dk, dv, chunk, q.dtype, o_dtype, log_decay, erase, write, (B, T, H), fg2)
    if out is None:
        out = torch.empty((B, T, H, dv), dtype=o_dtype, device=dev)
    else:
        _check_tensor("out", out, (o_dtype,), dev)
    if S_T is None and return_state:
        S_T = torch.empty((B, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _check_tensor("S_T", S_T, (torch.float32,), dev)
    ws_n = workspace_bytes(desc)
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    st = _abi.lib().dr_chunk_fwd(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(erase),
        _ptr(write), _ptr(S0), _ptr(out), _ptr(S_T), _ptr(ws), ws_n, _stream(),
    )
    _abi.check("dr_chunk_fwd", st)
    return out, S_T


def chunk_fwd_noalloc(q, k, v, log_decay, erase, write=None, S0=None, *, out, S_T=None, chunk=64, fg2=False):
    """``chunk_fwd`` through the allocation-free entry point: the caller passes the outputs
    (``out`` [B, T, H, dv], optional ``S_T``) and the library's fixed device scratch serves as
    the workspace, so the call allocates nothing (usable under graph capture).  Calls that may
    overlap on one device race on that scratch.  Raises DrError (DR_E_SCRATCH) when the problem
    needs more than ``noalloc_max_bytes()``.  Returns (out, S_T)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, (torch.float32, torch.bfloat16), dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B, T, H, dk] and v [B, T, H, dv]")
    B, T, H, dk = q.shape
    dv = v.shape[3]
    for name, t in (("log_decay", log_decay), ("erase", erase), ("write", write), ("S0", S0)):
        if t is not None:
            _check_tensor(name, t, (torch.float32,), dev)
    _check_tensor("out", out, (torch.float32, torch.bfloat16), dev)
    if tuple(out.shape) != (B, T, H, dv):
        raise ValueError(f"out must be [B, T, H, dv] = {(B, T, H, dv)}")
    if S_T is not None:
        _check_tensor("S_T", S_T, (torch.float32,), dev)
    desc = _desc(B, T, H, dk, dv, chunk, q.dtype, out.dtype, log_decay, erase, write, (B, T, H), fg2)
    st = _abi.lib().dr_chunk_fwd_noalloc(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(erase), _ptr(write), _ptr(S0),
        _ptr(out), _ptr(S_T), _stream(),
    )
    _abi.check("dr_chunk_fwd_noalloc", st)
    return out, S_T


def noalloc_max_bytes() -> int:
    return int(_abi.lib().dr_chunk_fwd_noalloc_max_bytes())


def varlen_workspace_bytes(desc, nseq) -> int:
    return int(_abi.lib().dr_chunk_fwd_varlen_workspace_bytes(ctypes.byref(desc), int(nseq)))


def chunk_fwd_varlen(q, k, v, log_decay, erase, write=None, S0=None, *, cu_seqlens, chunk=64,
                     o_dtype=torch.float32, out=None, S_T=None, return_state=True, workspace=None,
                     fg2=False):
    """Chunked forward over N packed sequences of different lengths, each from its own state.

    q, k: [1, T, H, dk]; v: [1, T, H, dv] with the sequences one after another on the token
    axis; gates [1, T, H] or [1, T, H, d]; cu_seqlens: int32 [N + 1] on the GPU (sequence n is
    tokens cu_seqlens[n] .. cu_seqlens[n + 1] - 1); S0: None or [N, H, dk, dv] fp32.
    Returns (o [1, T, H, dv], S_T [N, H, dk, dv] or None); S_T is the state layout of
    ``decode_step``.  ``workspace`` may supply a uint8 buffer of at least
    ``varlen_workspace_bytes`` bytes."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, (torch.float32, torch.bfloat16), dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if q.dim() != 4 or q.shape[0] != 1 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [1, T, H, dk] and v [1, T, H, dv]")
    _check_tensor("cu_seqlens", cu_seqlens, (torch.int32,), dev)
    if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
        raise ValueError("cu_seqlens must be a 1-d int32 tensor of N + 1 offsets")
    N = cu_seqlens.numel() - 1
    _, T, H, dk = q.shape
    dv = v.shape[3]
    for name, t in (("log_decay", log_decay), ("erase", erase), ("write", write), ("S0", S0)):
        if t is not None:
            _check_tensor(name, t, (torch.float32,), dev)
    if S0 is not None and tuple(S0.shape) != (N, H, dk, dv):
        raise ValueError(f"S0 must be [N, H, dk, dv] = {(N, H, dk, dv)}")
    desc = _desc(1, T, H, dk, dv, chunk, q.dtype, o_dtype, log_decay, erase, write, (1, T, H), fg2)
    if out is None:
        out = torch.empty((1, T, H, dv), dtype=o_dtype, device=dev)
    else:
        _check_tensor("out", out, (o_dtype,), dev)
    if S_T is None and return_state:
        S_T = torch.empty((N, H, dk, dv), dtype=torch.float32, device=dev)
    elif S_T is not None:
        _check_tensor("S_T", S_T, (torch.float32,), dev)
        if tuple(S_T.shape) != (N, H, dk, dv):
            raise ValueError(f"S_T must be [N, H, dk, dv] = {(N, H, dk, dv)}")
    ws_n = varlen_workspace_bytes(desc, N) if N > 0 and T > 0 else 0
    if workspace is None:
        workspace = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    elif workspace.numel() < ws_n:
        raise ValueError(f"workspace holds {workspace.numel()} bytes, {ws_n} needed")
    st = _abi.lib().dr_chunk_fwd_varlen(
        ctypes.byref(desc), _ptr(cu_seqlens), N, _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay),
        _ptr(erase), _ptr(write), _ptr(S0), _ptr(out), _ptr(S_T), _ptr(workspace),
        0 if workspace is None else workspace.numel(), _stream(),
    )
    _abi.check("dr_chunk_fwd_varlen", st)
    return out, S_T


def chunk_bwd(q, k, v, log_decay, erase, write=None, S0=None, *, dO, dS_T=None, need_dS0=True, fg2=False,
              cu_seqlens=None, chunk=64):
    """Gradients of sum(o * dO) + sum(S_T * dS_T) with respect to q, k, v, the gates and S0.

    Inputs as ``chunk_fwd`` (or, with ``cu_seqlens``, as ``chunk_fwd_varlen``: [1, T, ...] packed
    sequences with states [N, H, dk, dv]); dO [B, T, H, dv] and dS_T are fp32 (dS_T None: zero).
    Returns a dict of fp32 tensors dq, dk, dv, dlog_decay, derase, dwrite (None when ``write``
    is None: derase then holds the shared gate's whole gradient) and dS0 (None unless
    ``need_dS0``), each in its input's layout.  ``fg2=True``: ``erase`` is FG2's rate beta, and
    derase its gradient.  ``chunk=1`` takes the fp32 token adjoint wherever the chunk path would
    run (bf16 q/k/v, dk == dv == 128, a dense batch)."""
    dev = q.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, (torch.float32, torch.bfloat16), dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    if q.dim() != 4 or k.shape != q.shape or v.dim() != 4 or v.shape[:3] != q.shape[:3]:
        raise ValueError("q, k must be [B, T, H, dk] and v [B, T, H, dv]")
    B, T, H, dk = q.shape
    dv = v.shape[3]
    for name, t in (("log_decay", log_decay), ("erase", erase), ("write", write), ("S0", S0), ("dO", dO),
                    ("dS_T", dS_T)):
        if t is not None:
            _check_tensor(name, t, (torch.float32,), dev)
    if tuple(dO.shape) != (B, T, H, dv):
        raise ValueError(f"dO must be [B, T, H, dv] = {(B, T, H, dv)}")
    nstate = B
    if cu_seqlens is not None:
        _check_tensor("cu_seqlens", cu_seqlens, (torch.int32,), dev)
        if B != 1 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 1:
            raise ValueError("packed sequences: q is [1, T, H, dk] and cu_seqlens holds N + 1 offsets")
        nstate = cu_seqlens.numel() - 1
    desc = _desc(B, T, H, dk, dv, chunk, q.dtype, torch.float32, log_decay, erase, write, (B, T, H), fg2)
    f32 = dict(dtype=torch.float32, device=dev)
    out = dict(dq=torch.empty((B, T, H, dk), **f32), dk=torch.empty((B, T, H, dk), **f32),
               dv=torch.empty((B, T, H, dv), **f32), dlog_decay=torch.empty(log_decay.shape, **f32),
               derase=torch.empty(erase.shape, **f32),
               dwrite=None if write is None else torch.empty(write.shape, **f32),
               dS0=torch.empty((nstate, H, dk, dv), **f32) if need_dS0 else None)
    L = _abi.lib()
    if cu_seqlens is None:
        ws_n = int(L.dr_chunk_bwd_workspace_bytes(ctypes.byref(desc)))
    else:
        ws_n = int(L.dr_chunk_bwd_varlen_workspace_bytes(ctypes.byref(desc), nstate)) if nstate and T else 0
    ws = torch.empty(ws_n, dtype=torch.uint8, device=dev) if ws_n else None
    args = (_ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(erase), _ptr(write), _ptr(S0), _ptr(dO), _ptr(dS_T),
            _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dlog_decay"]), _ptr(out["derase"]),
            _ptr(out["dwrite"]), _ptr(out["dS0"]), _ptr(ws), ws_n, _stream())
    if cu_seqlens is None:
        _abi.check("dr_chunk_bwd", L.dr_chunk_bwd(ctypes.byref(desc), *args))
    else:
        _abi.check("dr_chunk_bwd_varlen",
                   L.dr_chunk_bwd_varlen(ctypes.byref(desc), _ptr(cu_seqlens), nstate, *args))
    return out


def decode_step(q, k, v, log_decay, erase, write=None, *, S, o=None, o_dtype=torch.float32, fg2=False):
    """One decode token for N sequences: q, k [N, H, dk]; v [N, H, dv]; gates [N, H] or
    [N, H, d]; S [N, H, dk, dv] fp32 updated in place.  Returns o [N, H, dv]."""
    dev = S.device
    for name, t in (("q", q), ("k", k), ("v", v)):
        _check_tensor(name, t, (torch.float32, torch.bfloat16), dev)
    if not (q.dtype == k.dtype == v.dtype):
        raise TypeError("q, k and v must share one dtype")
    _check_tensor("S", S, (torch.float32,), dev)
    if q.dim() != 3 or k.shape != q.shape or v.dim() != 3 or v.shape[:2] != q.shape[:2]:
        raise ValueError("q, k must be [N, H, dk] and v [N, H, dv]")
    N, H, dk = q.shape
    dv = v.shape[2]
    if tuple(S.shape) != (N, H, dk, dv):
        raise ValueError(f"S must be [N, H, dk, dv] = {(N, H, dk, dv)}")
    for name, t in (("log_decay", log_decay), ("erase", erase), ("write", write)):
        if t is not None:
            _check_tensor(name, t, (torch.float32,), dev)
    desc = _desc(N, 1, H, dk, dv, 0, q.dtype, o_dtype, log_decay, erase, write, (N, H), fg2)
    if o is None:
        o = torch.empty((N, H, dv), dtype=o_dtype, device=dev)
    else:
        _check_tensor("o", o, (o_dtype,), dev)
    st = _abi.lib().dr_decode_step(
        ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(log_decay), _ptr(erase),
        _ptr(write), _ptr(S), _ptr(o), _stream(),
    )
    _abi.check("dr_decode_step", st)
    return o
