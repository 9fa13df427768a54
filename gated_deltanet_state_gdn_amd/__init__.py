"""Gated DeltaNet state rebuild (Tail-Replay) for MI355X: Python binding of libgdn.so.

The functions below have the names of the C ABI entry points (include/gdn.h) and
only marshal arguments: torch tensors become device pointers, torch's current HIP
stream becomes the call's stream, and missing output buffers are allocated with
torch.  Every step of the computation runs in the library's gfx950 kernels; there
is no other code path.  The library must be built (``python -m
gated_deltanet_state_gdn_amd.build``); importing the functions works without it,
calling them raises.
"""
from __future__ import annotations

import ctypes
from typing import Optional

import torch

from . import _lib
from ._lib import (GDN_BF16, GDN_F32, GdnDesc, GdnError, GDN_ERR_DEVICE_INPUT, GDN_OK,
                   LIB_PATH, load)

__all__ = ["gdn_replay", "gdn_prefill", "gdn_state_relerr", "gdn_device_status",
           "gdn_replay_segmented", "gdn_segmented_workspace_bytes",
           "gdn_adaptive_replay_len", "gdn_adaptive_replay_len_static",
           "gdn_workspace_bytes", "gdn_replay_len", "gdn_status_str", "gdn_abi_version",
           "GdnError", "make_desc", "workspace", "LIB_PATH", "load"]

_DT = {torch.float32: GDN_F32, torch.bfloat16: GDN_BF16}


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(int(stream.cuda_stream))


def gdn_abi_version() -> int:
    return int(load().gdn_abi_version())


def gdn_status_str(code: int) -> str:
    return load().gdn_status_str(int(code)).decode()


def gdn_replay_len(L: int, rho: float) -> int:
    return int(load().gdn_replay_len(int(L), float(rho)))


def make_desc(q, v, n_seqs, total_out_tokens, scale=1.0, o_dtype=None) -> GdnDesc:
    d = GdnDesc()
    d.n_seqs = int(n_seqs)
    d.h_qk, d.d_k = int(q.shape[1]), int(q.shape[2])
    d.h_v, d.d_v = int(v.shape[1]), int(v.shape[2])
    d.qkv_dtype = _DT.get(q.dtype, -1)
    d.o_dtype = _DT.get(o_dtype if o_dtype is not None else q.dtype, -1)
    d.scale = float(scale)
    d.total_tokens = int(q.shape[0])
    d.total_out_tokens = int(total_out_tokens)
    return d


def gdn_workspace_bytes(desc: GdnDesc) -> int:
    return int(load().gdn_workspace_bytes(ctypes.byref(desc)))


def workspace(desc: GdnDesc, device) -> torch.Tensor:
    """A zero-filled workspace (its status word accumulates bits until read)."""
    return torch.zeros(gdn_workspace_bytes(desc), dtype=torch.uint8, device=device)


def _check(code: int, where: str):
    if code != GDN_OK:
        raise GdnError(code, where)


def gdn_replay(q, k, v, g, beta, cu_seqlens, r, *, total_out_tokens: int, S_out=None,
               o_out=True, cu_out=None, ws=None, scale: float = 1.0, o_dtype=None, stream=None):
    """Tail replay (see include/gdn.h). ``o_out``: a tensor, True (allocate) or None (skip).

    Returns (S_out, o_out or None, cu_out or None).
    """
    lib = load()
    n = int(cu_seqlens.shape[0]) - 1
    desc = make_desc(q, v, n, total_out_tokens, scale, o_dtype)
    dev = q.device
    if S_out is None:
        S_out = torch.empty((n, desc.h_v, desc.d_k, desc.d_v), dtype=torch.float32, device=dev)
    if o_out is True:
        odt = o_dtype if o_dtype is not None else q.dtype
        o_out = torch.empty((int(total_out_tokens), desc.h_v, desc.d_v), dtype=odt, device=dev)
    elif o_out is False:
        o_out = None
    if ws is None:
        ws = workspace(desc, dev)
    code = lib.gdn_replay(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                          _ptr(cu_seqlens), _ptr(r), _ptr(S_out), _ptr(o_out), _ptr(cu_out),
                          _ptr(ws), ws.numel(), _stream(stream))
    _check(code, "gdn_replay")
    return S_out, o_out, cu_out


def gdn_segmented_workspace_bytes(desc: GdnDesc, n_segments: int = 0) -> int:
    return int(load().gdn_segmented_workspace_bytes(ctypes.byref(desc), int(n_segments)))


def gdn_replay_segmented(q, k, v, g, beta, cu_seqlens, r, *, total_out_tokens: int,
                         n_segments: int = 0, S_out=None, o_out=True, cu_out=None, ws=None,
                         scale: float = 1.0, o_dtype=None, stream=None):
    """Segment-parallel tail replay (see include/gdn.h); arguments as gdn_replay plus
    ``n_segments`` (0 = the library's choice).  ``ws``, when given, must hold
    gdn_segmented_workspace_bytes(desc, n_segments) bytes, zero-filled before first use.

    Returns (S_out, o_out or None, cu_out or None).
    """
    lib = load()
    n = int(cu_seqlens.shape[0]) - 1
    desc = make_desc(q, v, n, total_out_tokens, scale, o_dtype)
    dev = q.device
    if S_out is None:
        S_out = torch.empty((n, desc.h_v, desc.d_k, desc.d_v), dtype=torch.float32, device=dev)
    if o_out is True:
        odt = o_dtype if o_dtype is not None else q.dtype
        o_out = torch.empty((int(total_out_tokens), desc.h_v, desc.d_v), dtype=odt, device=dev)
    elif o_out is False:
        o_out = None
    if ws is None:
        nb = gdn_segmented_workspace_bytes(desc, n_segments)
        ws = torch.zeros(max(nb, 256), dtype=torch.uint8, device=dev)
    code = lib.gdn_replay_segmented(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                                    _ptr(cu_seqlens), _ptr(r), _ptr(S_out), _ptr(o_out), _ptr(cu_out),
                                    int(n_segments), _ptr(ws), ws.numel(), _stream(stream))
    _check(code, "gdn_replay_segmented")
    return S_out, o_out, cu_out


def gdn_prefill(q, k, v, g, beta, cu_seqlens, *, S0=None, S_out=None, o_out=True, ws=None,
                scale: float = 1.0, o_dtype=None, stream=None):
    """Full prefill from S0 (None = zero). Returns (S_out, o_out or None)."""
    lib = load()
    n = int(cu_seqlens.shape[0]) - 1
    desc = make_desc(q, v, n, q.shape[0], scale, o_dtype)
    dev = q.device
    if S_out is None:
        S_out = torch.empty((n, desc.h_v, desc.d_k, desc.d_v), dtype=torch.float32, device=dev)
    if o_out is True:
        odt = o_dtype if o_dtype is not None else q.dtype
        o_out = torch.empty((int(q.shape[0]), desc.h_v, desc.d_v), dtype=odt, device=dev)
    elif o_out is False:
        o_out = None
    if ws is None:
        ws = workspace(desc, dev)
    code = lib.gdn_prefill(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                           _ptr(cu_seqlens), _ptr(S0), _ptr(S_out), _ptr(o_out), _ptr(ws),
                           ws.numel(), _stream(stream))
    _check(code, "gdn_prefill")
    return S_out, o_out


def gdn_state_relerr(S_a, S_ref, *, relerr_out=None, nonfinite_out=None, stream=None):
    """Per-state relative Frobenius error on the GPU. Returns (relerr fp32, nonfinite int32)."""
    lib = load()
    d_k, d_v = int(S_a.shape[-2]), int(S_a.shape[-1])
    n_states = S_a.numel() // (d_k * d_v)
    if relerr_out is None:
        relerr_out = torch.empty(S_a.shape[:-2], dtype=torch.float32, device=S_a.device)
    if nonfinite_out is None:
        nonfinite_out = torch.empty(S_a.shape[:-2], dtype=torch.int32, device=S_a.device)
    code = lib.gdn_state_relerr(_ptr(S_a), _ptr(S_ref), n_states, d_k, d_v, _ptr(relerr_out),
                                _ptr(nonfinite_out), _stream(stream))
    _check(code, "gdn_state_relerr")
    return relerr_out, nonfinite_out


def gdn_device_status(ws, stream=None) -> int:
    """Synchronise and return the status word of the last call that used ``ws``."""
    out = ctypes.c_int32(-1)
    code = load().gdn_device_status(_ptr(ws), _stream(stream), ctypes.byref(out))
    _check(code, "gdn_device_status")
    return int(out.value)


def gdn_adaptive_replay_len(g, cu_seqlens, *, eps: float, r_min: int = 0, r_max: int = 2**31 - 1,
                            r_out=None, ws=None, stream=None):
    """Per-sequence replay length from the gates (see include/gdn.h). ``g``: [T, h_v] fp32.

    Returns r_out (int32 [n_seqs], on the device), usable as gdn_replay's ``r``.
    """
    lib = load()
    n = int(cu_seqlens.shape[0]) - 1
    d = GdnDesc()
    d.n_seqs, d.h_v, d.total_tokens = n, int(g.shape[1]), int(g.shape[0])
    if r_out is None:
        r_out = torch.empty(max(n, 0), dtype=torch.int32, device=g.device)
    if ws is None:
        ws = workspace(d, g.device)
    code = lib.gdn_adaptive_replay_len(ctypes.byref(d), _ptr(g), _ptr(cu_seqlens), float(eps),
                                       int(r_min), int(r_max), _ptr(r_out), _ptr(ws), ws.numel(),
                                       _stream(stream))
    _check(code, "gdn_adaptive_replay_len")
    return r_out


def gdn_adaptive_replay_len_static(g, cu_seqlens, *, eps: float, r_min: int = 0,
                                   r_max: int = 2**31 - 1, r_out=None, stream=None):
    """gdn_adaptive_replay_len without a workspace (the library's static device scratch;
    see include/gdn.h).  ``r_out`` must be given by callers that cannot allocate."""
    lib = load()
    n = int(cu_seqlens.shape[0]) - 1
    d = GdnDesc()
    d.n_seqs, d.h_v, d.total_tokens = n, int(g.shape[1]), int(g.shape[0])
    if r_out is None:
        r_out = torch.empty(max(n, 0), dtype=torch.int32, device=g.device)
    code = lib.gdn_adaptive_replay_len_static(ctypes.byref(d), _ptr(g), _ptr(cu_seqlens), float(eps),
                                              int(r_min), int(r_max), _ptr(r_out), _stream(stream))
    _check(code, "gdn_adaptive_replay_len_static")
    return r_out
