"""Python binding of libgdn.so (C ABI in include/gdn.h), with the same entry-point names.

Argument marshalling only: every step of the operator runs in the HIP kernels of the
library. torch supplies device memory and the current stream. There is no CPU path: a
missing library, or a tensor that is not on a GPU, raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
_DTYPE = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}
CHUNK = 64

# (name, restype, argtypes) of every function declared in include/gdn.h
_P, _I, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
_SIGNATURES = [
    ("gdn_version", _I, []),
    ("gdn_status_string", ctypes.c_char_p, [_I]),
    ("gdn_chunk_fwd_workspace_bytes", _SZ, [_I] * 9),
    ("gdn_chunk_fwd", _I, [_P] * 9 + [_I] * 9 + [_P, _SZ, _P]),
    ("gdn_chunk_fwd_noalloc", _I, [_P] * 9 + [_I] * 9 + [_P]),
    ("gdn_chunk_prepare", _I, [_P] * 5 + [_I] * 8 + [_P, _SZ, _P]),
    ("gdn_chunk_propagate", _I, [_P] * 7 + [_I] * 9 + [_P, _SZ, _P]),
    ("gdn_decode_step", _I, [_P] * 7 + [_I] * 6 + [_P]),
    ("gdn_chunk_bwd_workspace_bytes", _SZ, [_I] * 9),
    ("gdn_chunk_bwd", _I, [_P] * 15 + [_I] * 9 + [_P, _SZ, _P]),
    ("gdn_kda_chunk_fwd_workspace_bytes", _SZ, [_I] * 9),
    ("gdn_kda_chunk_fwd", _I, [_P] * 9 + [_I] * 9 + [_P, _SZ, _P]),
    ("gdn_kda_decode_step", _I, [_P] * 7 + [_I] * 6 + [_P]),
    ("gdn_decoupled_chunk_fwd", _I, [_P] * 10 + [_I] * 9 + [_P, _SZ, _P]),
    ("gdn_decoupled_decode_step", _I, [_P] * 8 + [_I] * 6 + [_P]),
]

_lib = None


class GDNError(RuntimeError):
    """A call into libgdn.so returned a negative gdn_status."""


def lib():
    """Load libgdn.so (built in-tree by gated_delta_rule_42_amd.build)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                               "`python -m gated_delta_rule_42_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, res, args in _SIGNATURES:
            fn = getattr(L, name)
            fn.restype, fn.argtypes = res, args
        _lib = L
    return _lib


def gdn_version() -> int:
    return lib().gdn_version()


def gdn_status_string(status: int) -> str:
    return lib().gdn_status_string(status).decode()


def _check(status: int, what: str):
    if status != 0:
        raise GDNError(f"{what}: {gdn_status_string(status)} (status {status})")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _need_gpu(*ts):
    for t in ts:
        if t is not None and (not t.is_cuda or not t.is_contiguous()):
            raise ValueError("gdn: every tensor must be a contiguous tensor on a GPU")


def _expect(t, name, shape, dtypes):
    """Raise ValueError unless tensor t (if given) has this shape and one of these dtypes: the C
    ABI sees raw pointers only, so a wrong shape or dtype would otherwise be read or written out
    of bounds on the device."""
    if t is None:
        return
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"gdn: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        names = " or ".join(str(d).replace("torch.", "") for d in dtypes)
        raise ValueError(f"gdn: {name} has dtype {str(t.dtype).replace('torch.', '')}, expected {names}")


_IN = (torch.float32, torch.bfloat16)
_F32 = (torch.float32,)


def _check_chunk_args(q, k, v, g, beta, h0, cu_seqlens, o=None, hT=None, g_channels=False):
    """Shapes and dtypes of the chunked forward (and backward) arguments; returns the sizes."""
    if q.dim() != 4:
        raise ValueError(f"gdn: q must be [B, T, H, d_k], got shape {tuple(q.shape)}")
    if q.dtype not in _IN:
        raise ValueError(f"gdn: q has dtype {q.dtype}, expected float32 or bfloat16")
    B, T, H, dk = q.shape
    if v.dim() != 4:
        raise ValueError(f"gdn: v must be [B, T, H, d_v], got shape {tuple(v.shape)}")
    dv = v.shape[-1]
    _expect(k, "k", q.shape, (q.dtype,))
    _expect(v, "v", (B, T, H, dv), (q.dtype,))
    _expect(g, "g", (B, T, H, dk) if g_channels else (B, T, H), _F32)
    _expect(beta, "beta", (B, T, H), _F32)
    if cu_seqlens is not None:
        if cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2 or cu_seqlens.dtype != torch.int32:
            raise ValueError("gdn: cu_seqlens must be a 1-D int32 tensor of N + 1 >= 2 offsets")
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    _expect(h0, "h0", (N, H, dv, dk), _F32)
    _expect(hT, "hT", (N, H, dv, dk), _F32)
    _expect(o, "o", (B, T, H, dv), _IN)
    return B, T, H, dk, dv, N


def _check_decode_args(q, k, v, g, beta, state, o, g_channels=False):
    if q.dim() != 3 or q.dtype not in _IN:
        raise ValueError(f"gdn: q must be [N, H, d_k] float32 or bfloat16, got {tuple(q.shape)} {q.dtype}")
    N, H, dk = q.shape
    if v.dim() != 3:
        raise ValueError(f"gdn: v must be [N, H, d_v], got shape {tuple(v.shape)}")
    dv = v.shape[-1]
    _expect(k, "k", q.shape, (q.dtype,))
    _expect(v, "v", (N, H, dv), (q.dtype,))
    _expect(g, "g", (N, H, dk) if g_channels else (N, H), _F32)
    _expect(beta, "beta", (N, H), _F32)
    _expect(state, "state", (N, H, dv, dk), _F32)
    _expect(o, "o", (N, H, dv), _IN)
    return N, H, dk, dv


def gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, varlen, chunk=CHUNK, dtype=torch.bfloat16) -> int:
    return lib().gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, int(bool(varlen)), chunk,
                                               _DTYPE[dtype])


def _workspace(B, T, H, dk, dv, N, cu_seqlens, dtype, device, workspace):
    need = gdn_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, cu_seqlens is not None, CHUNK, dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=device)
    return workspace, need


def gdn_chunk_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk=CHUNK, *, o=None, hT=None,
                  o_dtype=None, output_final_state=True, workspace=None, stream=None):
    """Chunkwise forward pass. q, k [B,T,H,dk], v [B,T,H,dv] (fp32 or bf16); g, beta
    [B,T,H] fp32; h0 [N,H,dv,dk] fp32 or None; cu_seqlens int32 [N+1] or None.
    o is written in o_dtype (default: the dtype of q; fp32 is allowed for bf16 inputs).
    Returns (o [B,T,H,dv], hT [N,H,dv,dk] fp32 or None)."""
    B, T, H, dk, dv, N = _check_chunk_args(q, k, v, g, beta, h0, cu_seqlens, o, hT)
    _need_gpu(q, k, v, g, beta, h0, cu_seqlens, o, hT, workspace)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=o_dtype or q.dtype, device=q.device)
    if hT is None and output_final_state:
        hT = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    workspace, need = _workspace(B, T, H, dk, dv, N, cu_seqlens, q.dtype, q.device, workspace)
    st = lib().gdn_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                             _ptr(hT), _ptr(cu_seqlens), chunk, B, T, H, dk, dv, N,
                             _DTYPE.get(q.dtype, -1), _DTYPE.get(o.dtype, -1), _ptr(workspace),
                             workspace.numel() if workspace is not None else 0,
                             _stream(q.device, stream))
    _check(st, "gdn_chunk_fwd")
    return o, hT


def gdn_chunk_fwd_noalloc(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk=CHUNK, *, o=None, hT=None,
                          o_dtype=None, output_final_state=True, stream=None):
    """gdn_chunk_fwd on the library's own device scratch array (no workspace argument, no
    allocation inside the call; outputs are allocated here unless given)."""
    B, T, H, dk, dv, N = _check_chunk_args(q, k, v, g, beta, h0, cu_seqlens, o, hT)
    _need_gpu(q, k, v, g, beta, h0, cu_seqlens, o, hT)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=o_dtype or q.dtype, device=q.device)
    if hT is None and output_final_state:
        hT = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    st = lib().gdn_chunk_fwd_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                                     _ptr(hT), _ptr(cu_seqlens), chunk, B, T, H, dk, dv, N,
                                     _DTYPE.get(q.dtype, -1), _DTYPE.get(o.dtype, -1),
                                     _stream(q.device, stream))
    _check(st, "gdn_chunk_fwd_noalloc")
    return o, hT


def gdn_chunk_prepare(q, k, g, beta, workspace, cu_seqlens=None, chunk=CHUNK, *, dv=None, stream=None):
    """Stage 1 (per-chunk gate scan, gated Gram, UT transform, chunk operators) into
    `workspace` (uint8 tensor of gdn_chunk_fwd_workspace_bytes bytes)."""
    if q.dim() != 4 or q.dtype not in _IN:
        raise ValueError(f"gdn: q must be [B, T, H, d_k] float32 or bfloat16, got {tuple(q.shape)} {q.dtype}")
    B, T, H, dk = q.shape
    dv = dk if dv is None else dv
    _check_chunk_args(q, k, q.new_empty((B, T, H, dv), device="meta"), g, beta, None, cu_seqlens)
    _need_gpu(q, k, g, beta, cu_seqlens, workspace)
    N = B if cu_seqlens is None else cu_seqlens.numel() - 1
    st = lib().gdn_chunk_prepare(_ptr(q), _ptr(k), _ptr(g), _ptr(beta), _ptr(cu_seqlens), chunk, B, T,
                                 H, dk, dv, N, _DTYPE.get(q.dtype, -1), _ptr(workspace),
                                 workspace.numel() if workspace is not None else 0,
                                 _stream(q.device, stream))
    _check(st, "gdn_chunk_prepare")


def gdn_chunk_propagate(q, k, v, workspace, h0=None, cu_seqlens=None, chunk=CHUNK, *, o=None,
                        hT=None, o_dtype=None, output_final_state=True, stream=None):
    """Stage 2 (state carried across chunks, chunk outputs) from a prepared workspace."""
    B, T, H, dk, dv, N = _check_chunk_args(q, k, v, None, None, h0, cu_seqlens, o, hT)
    _need_gpu(q, k, v, h0, cu_seqlens, o, hT, workspace)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=o_dtype or q.dtype, device=q.device)
    if hT is None and output_final_state:
        hT = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    st = lib().gdn_chunk_propagate(_ptr(q), _ptr(k), _ptr(v), _ptr(h0), _ptr(o), _ptr(hT),
                                   _ptr(cu_seqlens), chunk, B, T, H, dk, dv, N,
                                   _DTYPE.get(q.dtype, -1), _DTYPE.get(o.dtype, -1), _ptr(workspace),
                                   workspace.numel() if workspace is not None else 0,
                                   _stream(q.device, stream))
    _check(st, "gdn_chunk_propagate")
    return o, hT


def gdn_decode_step(q, k, v, g, beta, state, o=None, *, o_dtype=torch.float32, stream=None):
    """One decode step: q, k [N,H,dk], v [N,H,dv] (fp32 or bf16), g, beta [N,H] fp32,
    state [N,H,dv,dk] fp32 updated in place. Returns o [N,H,dv] in o_dtype (fp32 by
    default; bf16 gives the fp32 result rounded to nearest even)."""
    N, H, dk, dv = _check_decode_args(q, k, v, g, beta, state, o)
    _need_gpu(q, k, v, g, beta, state, o)
    if o is None:
        o = torch.empty((N, H, dv), dtype=o_dtype, device=q.device)
    st = lib().gdn_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                               N, H, dk, dv, _DTYPE.get(q.dtype, -1), _DTYPE.get(o.dtype, -1),
                               _stream(q.device, stream))
    _check(st, "gdn_decode_step")
    return o


def gdn_chunk_bwd_workspace_bytes(B, T, H, dk, dv, N, varlen, chunk=CHUNK, dtype=torch.bfloat16) -> int:
    return lib().gdn_chunk_bwd_workspace_bytes(B, T, H, dk, dv, N, int(bool(varlen)), chunk,
                                               _DTYPE[dtype])


def gdn_chunk_bwd(q, k, v, g, beta, do, h0=None, dhT=None, cu_seqlens=None, chunk=CHUNK, *,
                  grad_dtype=None, need_dh0=True, workspace=None, stream=None):
    """Backward pass of gdn_chunk_fwd for output gradients do [B,T,H,dv] (dtype of q) and
    final-state gradients dhT [N,H,dv,dk] fp32 (or None). Returns dq, dk, dv (grad_dtype,
    default the dtype of q; fp32 is allowed for bf16 inputs), dg, dbeta [B,T,H] fp32 and
    dh0 [N,H,dv,dk] fp32 (None unless need_dh0)."""
    B, T, H, dk, dv, N = _check_chunk_args(q, k, v, g, beta, h0, cu_seqlens, hT=dhT)
    _expect(do, "do", (B, T, H, dv), (q.dtype,))
    _need_gpu(q, k, v, g, beta, do, h0, dhT, cu_seqlens, workspace)
    dev = q.device
    gd = grad_dtype or q.dtype
    dq = torch.empty(q.shape, dtype=gd, device=dev)
    dk_ = torch.empty(k.shape, dtype=gd, device=dev)
    dv_ = torch.empty(v.shape, dtype=gd, device=dev)
    dg = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    db = torch.empty((B, T, H), dtype=torch.float32, device=dev)
    dh0 = torch.empty((N, H, dv, dk), dtype=torch.float32, device=dev) if need_dh0 else None
    need = gdn_chunk_bwd_workspace_bytes(B, T, H, dk, dv, N, cu_seqlens is not None, chunk, q.dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=dev)
    st = lib().gdn_chunk_bwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(do), _ptr(dhT),
                             _ptr(dq), _ptr(dk_), _ptr(dv_), _ptr(dg), _ptr(db), _ptr(dh0),
                             _ptr(cu_seqlens), chunk, B, T, H, dk, dv, N, _DTYPE.get(q.dtype, -1),
                             _DTYPE.get(gd, -1), _ptr(workspace),
                             workspace.numel() if workspace is not None else 0,
                             _stream(dev, stream))
    _check(st, "gdn_chunk_bwd")
    return dq, dk_, dv_, dg, db, dh0


def gdn_kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, varlen, chunk=CHUNK, dtype=torch.bfloat16) -> int:
    return lib().gdn_kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, int(bool(varlen)), chunk,
                                                   _DTYPE[dtype])


def gdn_kda_chunk_fwd(q, k, v, g, beta, h0=None, cu_seqlens=None, chunk=CHUNK, *, o=None, hT=None,
                      o_dtype=None, output_final_state=True, workspace=None, stream=None):
    """Chunkwise forward pass with a channel-wise decay: as gdn_chunk_fwd, with g
    [B,T,H,dk] fp32 (log of one decay per key channel)."""
    B, T, H, dk, dv, N = _check_chunk_args(q, k, v, g, beta, h0, cu_seqlens, o, hT, g_channels=True)
    _need_gpu(q, k, v, g, beta, h0, cu_seqlens, o, hT, workspace)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=o_dtype or q.dtype, device=q.device)
    if hT is None and output_final_state:
        hT = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    need = gdn_kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, cu_seqlens is not None, chunk, q.dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().gdn_kda_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(h0), _ptr(o),
                                 _ptr(hT), _ptr(cu_seqlens), chunk, B, T, H, dk, dv, N,
                                 _DTYPE.get(q.dtype, -1), _DTYPE.get(o.dtype, -1), _ptr(workspace),
                                 workspace.numel() if workspace is not None else 0,
                                 _stream(q.device, stream))
    _check(st, "gdn_kda_chunk_fwd")
    return o, hT


def gdn_kda_decode_step(q, k, v, g, beta, state, o=None, *, o_dtype=torch.float32, stream=None):
    """One decode step with a channel-wise decay: g [N,H,dk] fp32; otherwise as
    gdn_decode_step (state updated in place)."""
    N, H, dk, dv = _check_decode_args(q, k, v, g, beta, state, o, g_channels=True)
    _need_gpu(q, k, v, g, beta, state, o)
    if o is None:
        o = torch.empty((N, H, dv), dtype=o_dtype, device=q.device)
    st = lib().gdn_kda_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(o),
                                   N, H, dk, dv, _DTYPE.get(q.dtype, -1), _DTYPE.get(o.dtype, -1),
                                   _stream(q.device, stream))
    _check(st, "gdn_kda_decode_step")
    return o


def gdn_decoupled_chunk_fwd(q, k, v, g, erase, write, h0=None, cu_seqlens=None, chunk=CHUNK, *, o=None,
                            hT=None, o_dtype=None, output_final_state=True, workspace=None, stream=None):
    """Chunkwise forward pass with a channel-wise decay g [B,T,H,dk] and decoupled erase
    [B,T,H,dk] and write [B,T,H,dv] gates (fp32) in place of beta."""
    B, T, H, dk, dv, N = _check_chunk_args(q, k, v, g, None, h0, cu_seqlens, o, hT, g_channels=True)
    _expect(erase, "erase", (B, T, H, dk), _F32)
    _expect(write, "write", (B, T, H, dv), _F32)
    _need_gpu(q, k, v, g, erase, write, h0, cu_seqlens, o, hT, workspace)
    if o is None:
        o = torch.empty((B, T, H, dv), dtype=o_dtype or q.dtype, device=q.device)
    if hT is None and output_final_state:
        hT = torch.empty((N, H, dv, dk), dtype=torch.float32, device=q.device)
    need = gdn_kda_chunk_fwd_workspace_bytes(B, T, H, dk, dv, N, cu_seqlens is not None, chunk, q.dtype)
    if workspace is None and need:
        workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
    st = lib().gdn_decoupled_chunk_fwd(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(erase), _ptr(write), _ptr(h0),
                                       _ptr(o), _ptr(hT), _ptr(cu_seqlens), chunk, B, T, H, dk, dv, N,
                                       _DTYPE.get(q.dtype, -1), _DTYPE.get(o.dtype, -1), _ptr(workspace),
                                       workspace.numel() if workspace is not None else 0,
                                       _stream(q.device, stream))
    _check(st, "gdn_decoupled_chunk_fwd")
    return o, hT


def gdn_decoupled_decode_step(q, k, v, g, erase, write, state, o=None, *, o_dtype=torch.float32, stream=None):
    """One decode step with a channel-wise decay g [N,H,dk] and decoupled erase [N,H,dk] and
    write [N,H,dv] gates; the state is updated in place."""
    N, H, dk, dv = _check_decode_args(q, k, v, g, None, state, o, g_channels=True)
    _expect(erase, "erase", (N, H, dk), _F32)
    _expect(write, "write", (N, H, dv), _F32)
    _need_gpu(q, k, v, g, erase, write, state, o)
    if o is None:
        o = torch.empty((N, H, dv), dtype=o_dtype, device=q.device)
    st = lib().gdn_decoupled_decode_step(_ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(erase), _ptr(write),
                                         _ptr(state), _ptr(o), N, H, dk, dv, _DTYPE.get(q.dtype, -1),
                                         _DTYPE.get(o.dtype, -1), _stream(q.device, stream))
    _check(st, "gdn_decoupled_decode_step")
    return o
