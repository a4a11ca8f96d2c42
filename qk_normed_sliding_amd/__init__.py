"""Python binding of libsa_attn.so: QK-normed GQA sliding-window attention on MI355X.

Argument marshalling only: every step of the computation runs in the HIP
kernels behind the C ABI declared in include/sa_attn.h. PyTorch provides
device memory and the current stream. There is no CPU fallback: importing
this package fails if the library has not been built.

Entry points (same names as the C ABI):
  sa_qknorm(x, y=None, rstd=None, eps=1e-6)
  sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, head_dim)
  sa_attn_fwd(q, k, v, window=-1, softmax_scale=None, qk_norm=True, eps=1e-6, o=None, lse=None, workspace=None)
  sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, head_dim)
  sa_attn_bwd(q, k, v, o, lse, dout, window=-1, ..., dq=None, dk=None, dv=None, workspace=None)
  sa_attn_bwd_noalloc(q, k, v, o, lse, dout, ...)   (no workspace: the library's own scratch)
  sa_attn_fwd_rope(q, k, v, rope_cos, rope_sin, ...), sa_attn_bwd_rope(..., rope_cos, rope_sin, ...)
  sa_attn_fwd_ex / sa_attn_bwd_ex (rotary tables and value-embedding gate; also rope=..., ve=... on the plain calls)
  sa_attn_ve_workspace_bytes(B, T, Hkv, head_dim)
  sa_polar_express_workspace_bytes(batch, rows, cols), sa_polar_express(g, out=None, steps=5, eps=1e-7)
Helpers: attention(...) (autograd), sssl_windows(n_layer, T, pattern), rope_tables(T, D), ve_layers(n_layer).
"""

from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsa_attn.so")

SA_OK = 0
ABI_VERSION = 7
SA_KERNEL_FWD = 0
SA_KERNEL_BWD_DQ = 1
SA_KERNEL_BWD_DKDV = 2
SA_KERNEL_FWD_KNORM = 3
SA_KERNEL_BWD_KNORM = 4


class SAError(RuntimeError):
    """A libsa_attn entry point returned a non-zero sa_status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__(f"{fn} failed: {_lib.sa_status_string(status).decode()}")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python qk_normed_sliding_amd/build.py` "
            "(the HIP library is required; there is no fallback)")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, f32, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
    lib.sa_abi_version.restype = i32
    lib.sa_abi_version.argtypes = []
    lib.sa_status_string.restype = ctypes.c_char_p
    lib.sa_status_string.argtypes = [i32]
    lib.sa_qknorm.restype = i32
    lib.sa_qknorm.argtypes = [vp, vp, vp, i64, i32, f32, vp]
    lib.sa_attn_fwd_workspace_bytes.restype = sz
    lib.sa_attn_fwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.sa_attn_fwd.restype = i32
    lib.sa_attn_fwd.argtypes = [vp, vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, i32, f32, i32, f32, vp]
    lib.sa_attn_bwd_workspace_bytes.restype = sz
    lib.sa_attn_bwd_workspace_bytes.argtypes = [i32, i32, i32, i32, i32]
    lib.sa_attn_bwd.restype = i32
    lib.sa_attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                i32, i32, i32, i32, i32, i32, f32, i32, f32, vp]
    lib.sa_attn_bwd_noalloc_max_bytes.restype = sz
    lib.sa_attn_bwd_noalloc_max_bytes.argtypes = []
    lib.sa_attn_bwd_noalloc.restype = i32
    lib.sa_attn_bwd_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                        i32, i32, i32, i32, i32, i32, f32, i32, f32, vp]
    lib.sa_attn_fwd_rope.restype = i32
    lib.sa_attn_fwd_rope.argtypes = [vp, vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, i32, f32, i32, f32,
                                     vp, vp, i32, vp]
    lib.sa_attn_bwd_rope.restype = i32
    lib.sa_attn_bwd_rope.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz,
                                     i32, i32, i32, i32, i32, i32, f32, i32, f32, vp, vp, i32, vp]
    i64t = ctypes.c_int64
    lib.sa_attn_fwd_ex.restype = i32
    lib.sa_attn_fwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, sz, i32, i32, i32, i32, i32, i32, f32, i32, f32,
                                   vp, vp, i32, vp, i64t, vp, vp, vp, i32, vp]
    lib.sa_attn_ve_workspace_bytes.restype = sz
    lib.sa_attn_ve_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.sa_attn_bwd_ex.restype = i32
    lib.sa_attn_bwd_ex.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp, sz,
                                   i32, i32, i32, i32, i32, i32, f32, i32, f32, vp, vp, i32,
                                   vp, i64t, vp, vp, vp, i32, vp, vp, vp, vp, sz, vp]
    lib.sa_polar_express_workspace_bytes.restype = sz
    lib.sa_polar_express_workspace_bytes.argtypes = [i32, i32, i32]
    lib.sa_polar_express_executed_flops.restype = ctypes.c_double
    lib.sa_polar_express_executed_flops.argtypes = [i32, i32, i32, i32]
    lib.sa_polar_express.restype = i32
    lib.sa_polar_express.argtypes = [vp, vp, vp, sz, i32, i32, i32, i32, f32, vp]
    lib.sa_set_timing_events.restype = i32
    lib.sa_set_timing_events.argtypes = [i32, vp, vp]
    lib.sa_set_max_workgroups.restype = i32
    lib.sa_set_max_workgroups.argtypes = [i32]
    if lib.sa_abi_version() != ABI_VERSION:
        raise ImportError(f"libsa_attn ABI {lib.sa_abi_version()} != expected {ABI_VERSION}")
    return lib


_lib = _load()


def library():
    """The loaded ctypes handle of libsa_attn.so."""
    return _lib


# ------------------------------------------------------------------ marshalling

def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, status):
    if status != SA_OK:
        raise SAError(fn, status)


def _need(t, name, dtype, shape=None):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")


def _dims(q, k):
    if q.dim() != 4 or k.dim() != 4:
        raise ValueError("q is [B,T,Hq,D] and k, v are [B,T,Hkv,D]")
    B, T, Hq, D = q.shape
    Hkv = k.shape[2]
    return B, T, Hq, Hkv, D


def _scale(softmax_scale, D):
    return 1.0 / math.sqrt(D) if softmax_scale is None else float(softmax_scale)


# ------------------------------------------------------------------ entry points

def sa_qknorm(x, y=None, rstd=None, eps=1e-6, want_rstd=True, stream=None):
    """Weightless RMS norm of the rows of x ([..., D] bf16). Returns (y, rstd)."""
    _need(x, "x", torch.bfloat16)
    D = x.shape[-1]
    rows = x.numel() // D if D else 0
    if y is None:
        y = torch.empty_like(x)
    _need(y, "y", torch.bfloat16, x.shape)
    if rstd is None and want_rstd:
        rstd = torch.empty(x.shape[:-1], dtype=torch.float32, device=x.device)
    if rstd is not None:
        _need(rstd, "rstd", torch.float32, x.shape[:-1])
    _check("sa_qknorm", _lib.sa_qknorm(_ptr(x), _ptr(y), _ptr(rstd), rows, D, float(eps),
                                       _stream(x.device, stream)))
    return y, rstd


def sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, head_dim):
    return int(_lib.sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, head_dim))


def _rope_args(rope_cos, rope_sin, T, D, device):
    for t, n in ((rope_cos, "rope_cos"), (rope_sin, "rope_sin")):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.float32 or t.device != device or t.dim() != 2:
            raise SAError(f"{n}: fp32 [rows, >= D/2] tensor on {device} expected")
        if t.shape[0] < T or t.shape[1] < D // 2 or t.stride(1) != 1:
            raise SAError(f"{n}: at least T={T} rows of D/2={D // 2} unit-stride entries expected")
    if rope_cos.stride(0) != rope_sin.stride(0):
        raise SAError("rope_cos and rope_sin must share a row stride")
    return _ptr(rope_cos), _ptr(rope_sin), int(rope_cos.stride(0))


def _ve_args(ve, B, T, Hkv, D, device):
    """(x [B,T,C>=32] bf16, w [Hkv,32] bf16, ids [B,T] int32, table [V, Hkv*D] bf16) -> C-ABI arguments."""
    x, w, ids, table = ve
    _need(x, "ve x", torch.bfloat16)
    if x.dim() != 3 or tuple(x.shape[:2]) != (B, T) or x.shape[2] < 32:
        raise SAError(f"ve x: [B={B}, T={T}, >=32] expected")
    _need(w, "ve w", torch.bfloat16, (Hkv, 32))
    _need(ids, "ve ids", torch.int32, (B, T))
    _need(table, "ve table", torch.bfloat16)
    if table.dim() != 2 or table.shape[1] != Hkv * D:
        raise SAError(f"ve table: [vocab, Hkv*D={Hkv * D}] expected")
    return _ptr(x), int(x.shape[2]), _ptr(w), _ptr(ids), _ptr(table), int(table.shape[0])


def sa_attn_fwd_ex(q, k, v, window=-1, softmax_scale=None, qk_norm=True, eps=1e-6, o=None, lse=None,
                   workspace=None, stream=None, rope=None, ve=None):
    """Forward with optional rotary tables rope=(cos, sin) and value-embedding gate ve=(x, w, ids, table)."""
    B, T, Hq, Hkv, D = _dims(q, k)
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, T, Hkv, D))
    _need(v, "v", torch.bfloat16, (B, T, Hkv, D))
    rc, rs, rstride = _rope_args(rope[0], rope[1], T, D, q.device) if rope is not None else (None, None, 0)
    vx, vxs, vw, vids, vtab, vocab = _ve_args(ve, B, T, Hkv, D, q.device) if ve is not None else (
        None, 0, None, None, None, 0)
    o = torch.empty_like(q) if o is None else o
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device) if lse is None else lse
    _need(o, "o", torch.bfloat16, q.shape)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    if workspace is None:
        workspace = torch.empty(sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, D), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    _check("sa_attn_fwd_ex", _lib.sa_attn_fwd_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
        B, T, Hq, Hkv, D, int(window), _scale(softmax_scale, D), int(bool(qk_norm)), float(eps),
        rc, rs, rstride, vx, vxs, vw, vids, vtab, vocab, _stream(q.device, stream)))
    return o, lse


def sa_attn_ve_workspace_bytes(B, T, Hkv, head_dim):
    return int(_lib.sa_attn_ve_workspace_bytes(B, T, Hkv, head_dim))


def sa_attn_bwd_ex(q, k, v, o, lse, dout, window=-1, softmax_scale=None, qk_norm=True, eps=1e-6, dq=None, dk=None,
                   dv=None, workspace=None, stream=None, rope=None, ve=None, ve_workspace=None, fwd_workspace=None):
    """Backward with the optional extras. Returns (dq, dk, dv), plus (dve, dw, dx32) with ve.
    fwd_workspace: the workspace the forward of this layer wrote (same inputs, tables and
    embeddings); the backward then reads the normed k rows (and v', the gate) from it."""
    B, T, Hq, Hkv, D = _dims(q, k)
    for t, n, shp in ((q, "q", None), (k, "k", (B, T, Hkv, D)), (v, "v", (B, T, Hkv, D)),
                      (o, "o", q.shape), (dout, "dout", q.shape)):
        _need(t, n, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    rc, rs, rstride = _rope_args(rope[0], rope[1], T, D, q.device) if rope is not None else (None, None, 0)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    if workspace is None:
        workspace = torch.empty(sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, D), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    dve = dw = dx32 = None
    if ve is not None:
        vx, vxs, vw, vids, vtab, vocab = _ve_args(ve, B, T, Hkv, D, q.device)
        dve = torch.empty_like(v)
        dw = torch.empty((Hkv, 32), dtype=torch.float32, device=q.device)
        dx32 = torch.empty((B, T, 32), dtype=torch.float32, device=q.device)
        if ve_workspace is None:
            ve_workspace = torch.empty(sa_attn_ve_workspace_bytes(B, T, Hkv, D), dtype=torch.uint8, device=q.device)
        ve_ptrs = (vx, vxs, vw, vids, vtab, vocab, _ptr(dve), _ptr(dw), _ptr(dx32), _ptr(ve_workspace),
                   ve_workspace.numel())
    else:
        ve_ptrs = (None, 0, None, None, None, 0, None, None, None, None, 0)
    if fwd_workspace is not None:
        _need(fwd_workspace, "fwd_workspace", torch.uint8)
    _check("sa_attn_bwd_ex", _lib.sa_attn_bwd_ex(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), workspace.numel(), _ptr(fwd_workspace),
        0 if fwd_workspace is None else fwd_workspace.numel(), B, T, Hq, Hkv, D, int(window), _scale(softmax_scale, D),
        int(bool(qk_norm)), float(eps), rc, rs, rstride, *ve_ptrs, _stream(q.device, stream)))
    return (dq, dk, dv) if ve is None else (dq, dk, dv, dve, dw, dx32)


def sa_attn_fwd(q, k, v, window=-1, softmax_scale=None, qk_norm=True, eps=1e-6, o=None, lse=None,
                workspace=None, stream=None, rope=None, ve=None):
    """Forward of one layer. q [B,T,Hq,D], k/v [B,T,Hkv,D] bf16. Returns (o, lse).
    rope = (cos, sin) rotary tables and/or ve = (x, w, ids, table) value embeddings use the fused entry points."""
    if ve is not None:
        return sa_attn_fwd_ex(q, k, v, window, softmax_scale, qk_norm, eps, o, lse, workspace, stream, rope, ve)
    if rope is not None:
        return sa_attn_fwd_rope(q, k, v, rope[0], rope[1], window, softmax_scale, qk_norm, eps, o, lse,
                                workspace, stream)
    B, T, Hq, Hkv, D = _dims(q, k)
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, T, Hkv, D))
    _need(v, "v", torch.bfloat16, (B, T, Hkv, D))
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.bfloat16, q.shape)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    if workspace is None and qk_norm:
        workspace = torch.empty(sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, D), dtype=torch.uint8, device=q.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8)
    _check("sa_attn_fwd", _lib.sa_attn_fwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace),
        0 if workspace is None else workspace.numel(), B, T, Hq, Hkv, D, int(window),
        _scale(softmax_scale, D), int(bool(qk_norm)), float(eps), _stream(q.device, stream)))
    return o, lse


def sa_attn_fwd_rope(q, k, v, rope_cos, rope_sin, window=-1, softmax_scale=None, qk_norm=True, eps=1e-6, o=None,
                     lse=None, workspace=None, stream=None):
    """Forward with the rotary embedding of q and k fused (fp32 cos/sin tables [>= T, >= D/2])."""
    B, T, Hq, Hkv, D = _dims(q, k)
    _need(q, "q", torch.bfloat16)
    _need(k, "k", torch.bfloat16, (B, T, Hkv, D))
    _need(v, "v", torch.bfloat16, (B, T, Hkv, D))
    rc, rs, stride = _rope_args(rope_cos, rope_sin, T, D, q.device)
    if o is None:
        o = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    _need(o, "o", torch.bfloat16, q.shape)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    if workspace is None:
        workspace = torch.empty(sa_attn_fwd_workspace_bytes(B, T, Hq, Hkv, D), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    _check("sa_attn_fwd_rope", _lib.sa_attn_fwd_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(workspace), workspace.numel(),
        B, T, Hq, Hkv, D, int(window), _scale(softmax_scale, D), int(bool(qk_norm)), float(eps),
        rc, rs, stride, _stream(q.device, stream)))
    return o, lse


def sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, head_dim):
    return int(_lib.sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, head_dim))


def sa_attn_bwd(q, k, v, o, lse, dout, window=-1, softmax_scale=None, qk_norm=True, eps=1e-6,
                dq=None, dk=None, dv=None, workspace=None, stream=None, rope=None, ve=None, fwd_workspace=None):
    """Backward of one layer. Returns (dq, dk, dv) with respect to the raw q, k, v
    (with ve also (dve, dw, dx32)); rope/ve as for sa_attn_fwd; fwd_workspace as for
    sa_attn_bwd_ex."""
    if ve is not None or fwd_workspace is not None:
        return sa_attn_bwd_ex(q, k, v, o, lse, dout, window, softmax_scale, qk_norm, eps, dq, dk, dv, workspace,
                              stream, rope, ve, fwd_workspace=fwd_workspace)
    if rope is not None:
        return sa_attn_bwd_rope(q, k, v, o, lse, dout, rope[0], rope[1], window, softmax_scale, qk_norm, eps,
                                dq, dk, dv, workspace, stream)
    B, T, Hq, Hkv, D = _dims(q, k)
    for t, n, shp in ((q, "q", None), (k, "k", (B, T, Hkv, D)), (v, "v", (B, T, Hkv, D)),
                      (o, "o", q.shape), (dout, "dout", q.shape)):
        _need(t, n, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, q.shape)
    _need(dk, "dk", torch.bfloat16, k.shape)
    _need(dv, "dv", torch.bfloat16, v.shape)
    need = sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, D)
    if workspace is None:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    _check("sa_attn_bwd", _lib.sa_attn_bwd(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), workspace.numel(), B, T, Hq, Hkv, D, int(window), _scale(softmax_scale, D),
        int(bool(qk_norm)), float(eps), _stream(q.device, stream)))
    return dq, dk, dv


def sa_attn_bwd_noalloc_max_bytes():
    return int(_lib.sa_attn_bwd_noalloc_max_bytes())


def sa_attn_bwd_noalloc(q, k, v, o, lse, dout, window=-1, softmax_scale=None, qk_norm=True, eps=1e-6,
                        dq=None, dk=None, dv=None, stream=None):
    """sa_attn_bwd without a workspace argument: the library's own per-GPU scratch
    is used (for callers that cannot allocate; calls overlapping on one GPU race).
    Outputs are allocated here only when not given."""
    B, T, Hq, Hkv, D = _dims(q, k)
    for t, n, shp in ((q, "q", None), (k, "k", (B, T, Hkv, D)), (v, "v", (B, T, Hkv, D)),
                      (o, "o", q.shape), (dout, "dout", q.shape)):
        _need(t, n, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, q.shape)
    _need(dk, "dk", torch.bfloat16, k.shape)
    _need(dv, "dv", torch.bfloat16, v.shape)
    _check("sa_attn_bwd_noalloc", _lib.sa_attn_bwd_noalloc(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        B, T, Hq, Hkv, D, int(window), _scale(softmax_scale, D), int(bool(qk_norm)), float(eps),
        _stream(q.device, stream)))
    return dq, dk, dv


def sa_attn_bwd_rope(q, k, v, o, lse, dout, rope_cos, rope_sin, window=-1, softmax_scale=None, qk_norm=True,
                     eps=1e-6, dq=None, dk=None, dv=None, workspace=None, stream=None):
    """Backward with the rotary embedding fused; the same tables as the forward."""
    B, T, Hq, Hkv, D = _dims(q, k)
    for t, n, shp in ((q, "q", None), (k, "k", (B, T, Hkv, D)), (v, "v", (B, T, Hkv, D)),
                      (o, "o", q.shape), (dout, "dout", q.shape)):
        _need(t, n, torch.bfloat16, shp)
    _need(lse, "lse", torch.float32, (B, Hq, T))
    rc, rs, stride = _rope_args(rope_cos, rope_sin, T, D, q.device)
    dq = torch.empty_like(q) if dq is None else dq
    dk = torch.empty_like(k) if dk is None else dk
    dv = torch.empty_like(v) if dv is None else dv
    _need(dq, "dq", torch.bfloat16, q.shape)
    _need(dk, "dk", torch.bfloat16, k.shape)
    _need(dv, "dv", torch.bfloat16, v.shape)
    if workspace is None:
        workspace = torch.empty(sa_attn_bwd_workspace_bytes(B, T, Hq, Hkv, D), dtype=torch.uint8, device=q.device)
    _need(workspace, "workspace", torch.uint8)
    _check("sa_attn_bwd_rope", _lib.sa_attn_bwd_rope(
        _ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
        _ptr(workspace), workspace.numel(), B, T, Hq, Hkv, D, int(window), _scale(softmax_scale, D),
        int(bool(qk_norm)), float(eps), rc, rs, stride, _stream(q.device, stream)))
    return dq, dk, dv


def sa_polar_express_workspace_bytes(batch, rows, cols):
    return int(_lib.sa_polar_express_workspace_bytes(batch, rows, cols))


def sa_polar_express_executed_flops(batch, rows, cols, steps=5):
    """MFMA FLOP the library executes for sa_polar_express (symmetric products: upper tiles only)."""
    return float(_lib.sa_polar_express_executed_flops(batch, rows, cols, steps))


def sa_polar_express(g, out=None, steps=5, eps=1e-7, workspace=None, stream=None):
    """Muon's polar-express orthogonalisation of bf16 g [batch, rows, cols] (or [rows, cols])."""
    squeeze = g.dim() == 2
    g3 = g.unsqueeze(0) if squeeze else g
    if g3.dim() != 3:
        raise SAError("g: [batch, rows, cols] or [rows, cols] expected")
    _need(g3, "g", torch.bfloat16)
    batch, rows, cols = g3.shape
    if out is None:
        out = torch.empty_like(g3)
    out3 = out.unsqueeze(0) if out.dim() == 2 else out
    _need(out3, "out", torch.bfloat16, g3.shape)
    if workspace is None:
        workspace = torch.empty(max(1, sa_polar_express_workspace_bytes(batch, rows, cols)), dtype=torch.uint8,
                                device=g.device)
    _need(workspace, "workspace", torch.uint8)
    _check("sa_polar_express", _lib.sa_polar_express(
        _ptr(g3), _ptr(out3), _ptr(workspace), workspace.numel(), batch, rows, cols, int(steps), float(eps),
        _stream(g.device, stream)))
    return out3.squeeze(0) if squeeze else out3


def sa_set_timing_events(kernel, start_event, stop_event):
    """Benchmarking hook: attach raw hipEvent_t handles (ints, or None to clear)
    to the dispatch of kernel `kernel` (an SA_KERNEL_ id) in later calls from
    this thread."""
    _check("sa_set_timing_events", _lib.sa_set_timing_events(
        int(kernel), ctypes.c_void_p(start_event) if start_event else None,
        ctypes.c_void_p(stop_event) if stop_event else None))


def sa_set_max_workgroups(n):
    """Testing hook: launch at most n workgroups per persistent kernel from this
    thread (0 = one per compute unit)."""
    _check("sa_set_max_workgroups", _lib.sa_set_max_workgroups(int(n)))


# ------------------------------------------------------------------ helpers

class _Attention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, window, softmax_scale, qk_norm, eps, rope):
        q, k, v = q.contiguous(), k.contiguous(), v.contiguous()
        o, lse = sa_attn_fwd(q, k, v, window, softmax_scale, qk_norm, eps, rope=rope)
        ctx.save_for_backward(q, k, v, o, lse)
        ctx.args = (window, softmax_scale, qk_norm, eps)
        ctx.rope = rope
        return o

    @staticmethod
    def backward(ctx, do):
        q, k, v, o, lse = ctx.saved_tensors
        dq, dk, dv = sa_attn_bwd(q, k, v, o, lse, do.contiguous(), *ctx.args, rope=ctx.rope)
        return dq, dk, dv, None, None, None, None, None


def attention(q, k, v, window=-1, softmax_scale=None, qk_norm=True, eps=1e-6, rope=None):
    """Differentiable layer: o = attention(q, k, v); gradients via sa_attn_bwd.
    rope = (cos, sin) fp32 device tables (see rope_tables) turns q and k first."""
    return _Attention.apply(q, k, v, window, softmax_scale, qk_norm, eps, rope)


def ve_layers(n_layer: int):
    """Layers that carry value embeddings: alternating, the last always ([guide] 8.2.1)."""
    return [i for i in range(n_layer) if (n_layer - 1 - i) % 2 == 0]


def rope_tables(n_pos: int, head_dim: int, base: float = 10000.0, device=None):
    """Rotary tables (cos, sin), fp32 [n_pos, head_dim/2], of the angles
    t * base^(-2i/head_dim) ([guide] 8.2.1: the tables are precomputed once,
    for more positions than a sequence holds)."""
    t = torch.arange(n_pos, dtype=torch.float64, device=device).view(n_pos, 1)
    i = torch.arange(head_dim // 2, dtype=torch.float64, device=device).view(1, head_dim // 2)
    a = t * torch.pow(torch.tensor(base, dtype=torch.float64, device=device), -2.0 * i / head_dim)
    return torch.cos(a).float().contiguous(), torch.sin(a).float().contiguous()


def sssl_windows(n_layer: int, seq_len: int, pattern: str = "SSSL"):
    """Window of each layer for an S/L pattern: S = seq_len // 2, L = -1 (full causal).

    The pattern repeats over the layers and the last layer is always L
    ([post] SSSL passage; [guide] 3.4, WINDOW_PATTERN row).
    """
    pat = pattern.upper()
    if not pat or set(pat) - {"S", "L"}:
        raise ValueError(f"pattern must be a non-empty S/L string, got {pattern!r}")
    kinds = [pat[i % len(pat)] for i in range(n_layer)]
    if kinds:
        kinds[-1] = "L"
    return [seq_len // 2 if c == "S" else -1 for c in kinds]
