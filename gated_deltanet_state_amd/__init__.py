"""Gated DeltaNet state replay for MI355X (gfx950).

Thin Python binding over the C ABI in ``include/gdn.h`` (``libgdn.so``,
built in-tree by ``gated_deltanet_state_amd.build``).  The binding only
marshals arguments: every step of the computation runs in the library's HIP
kernels.  PyTorch supplies device memory and the current stream.

If ``libgdn.so`` is missing or cannot be loaded, every call raises: there is
no fallback implementation.

Functions (same names as the C entry points, without the ``gdn_`` prefix):
  replay(q, k, v, alpha, beta, cu_seqlens, S0=None, want_o=True, o_dtype=float32,
         segments=None)      (gdn_replay, or gdn_replay_segmented when segments is given)
  chunk_operator(k, alpha, beta, cu_chunks, v=None)
  compose(T_C, S_local, S_in=None)
  replay_noalloc(...)  (gdn_replay_noalloc: no workspace, the library's built-in scratch)
  decode, front_end, scalar_chunk_operator, scalar_compose

Every call launches on ``stream`` (default: the current stream).  The
workspace a call needs is allocated on that stream, so the caching allocator
hands its memory to other work only after the call's kernels.
"""
from __future__ import annotations

import ctypes
import os

__all__ = ["front_end", "replay", "replay_noalloc", "decode", "chunk_operator", "compose", "scalar_chunk_operator", "scalar_compose", "GdnError", "library", "LIB_PATH"]

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libgdn.so")

GDN_F32, GDN_BF16 = 0, 1
_lib = None


class GdnError(RuntimeError):
    def __init__(self, status: int, name: str, detail: str):
        super().__init__("%s (%d): %s" % (name, status, detail))
        self.status = status
        self.name = name
        self.detail = detail


def library():
    """Load libgdn.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError("libgdn.so is not built (run python -m gated_deltanet_state_amd.build)")
    _lib = declare(ctypes.CDLL(LIB_PATH))
    return _lib


def declare(lib):
    """Set the C signatures of the entry points on a loaded library (the
    product library, or its host-sanitized build in the tests)."""
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    cint = ctypes.c_int
    lib.gdn_replay.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, cint,
                               vp, cint, vp, vp, sz, vp]
    lib.gdn_replay_workspace_bytes.argtypes = [i32, i64, i32, i32, i32]
    lib.gdn_replay_segmented.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, cint,
                                         vp, cint, vp, i32, vp, sz, vp]
    lib.gdn_replay_segmented_workspace_bytes.argtypes = [i32, i64, i32, i32, i32, i32]
    lib.gdn_replay_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, cint,
                                       vp, cint, vp, vp]
    lib.gdn_replay_raw.argtypes = [vp, vp, vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, cint,
                                   vp, cint, vp, vp, sz, vp]
    lib.gdn_replay_raw_workspace_bytes.argtypes = [i32, i64, i32, i32, i32]
    lib.gdn_chunk_operator.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, cint,
                                       vp, vp, vp, sz, vp]
    lib.gdn_chunk_operator_workspace_bytes.argtypes = [i32, i64, i32, i32, i32]
    lib.gdn_compose.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp, sz, vp]
    lib.gdn_compose_workspace_bytes.argtypes = [i32, i32, i32, i32]
    lib.gdn_decode.argtypes = [vp, vp, vp, vp, vp, vp, i32, i32, i32, i32, cint, vp, cint, vp, vp]
    lib.gdn_front_end.argtypes = [vp, vp, vp, vp, i64, i32, i32, cint, vp, vp, vp, vp, vp]
    lib.gdn_scalar_chunk_operator.argtypes = [vp, vp, vp, vp, vp, i32, i64, i32, i32, i32, cint, vp, vp, vp]
    lib.gdn_scalar_compose.argtypes = [vp, vp, vp, i32, i32, i32, i32, vp, vp]
    for f in (lib.gdn_replay, lib.gdn_replay_segmented, lib.gdn_replay_noalloc, lib.gdn_replay_raw,
              lib.gdn_chunk_operator, lib.gdn_compose, lib.gdn_decode, lib.gdn_front_end,
              lib.gdn_scalar_chunk_operator, lib.gdn_scalar_compose):
        f.restype = cint
    for f in (lib.gdn_replay_workspace_bytes, lib.gdn_replay_segmented_workspace_bytes,
              lib.gdn_replay_raw_workspace_bytes, lib.gdn_chunk_operator_workspace_bytes,
              lib.gdn_compose_workspace_bytes):
        f.restype = sz
    lib.gdn_status_string.argtypes = [cint]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    lib.gdn_abi_version.argtypes = []
    lib.gdn_abi_version.restype = cint
    return lib


def _check(status: int):
    if status != 0:
        lib = library()
        raise GdnError(status, lib.gdn_status_string(status).decode(),
                       lib.gdn_last_error().decode())


def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_ptr(stream):
    torch = _torch()
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _launch_stream(stream, device):
    torch = _torch()
    return torch.cuda.current_stream(device) if stream is None else stream


def _dtype_code(dt):
    torch = _torch()
    if dt == torch.float32:
        return GDN_F32
    if dt == torch.bfloat16:
        return GDN_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % dt)


def _dev(t, name):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("%s must be a device tensor" % name)
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    return t


def _workspace(nbytes, device, stream):
    """Scratch for one call, allocated on the stream the call launches on:
    the caching allocator then reuses the block only for work ordered after
    the call's kernels on that stream (or after a synchronisation)."""
    torch = _torch()
    if nbytes == 0:
        return None, 0
    with torch.cuda.stream(_launch_stream(stream, device)):
        return torch.empty(nbytes, dtype=torch.uint8, device=device), nbytes


def replay(q, k, v, alpha, beta, cu_seqlens, S0=None, want_o=True, o_dtype=None,
           out=None, S_out=None, stream=None, segments=None):
    """Replay packed sequences through the gated delta rule.

    q, k [T, H, dk]; v [T, H, dv]; alpha, beta [T, H] (all float32 or all
    bfloat16); cu_seqlens int32 [N+1] on the device; S0 [N, H, dv, dk]
    float32 or None (zero state).  Returns (o [T, H, dv] or None,
    S_final [N, H, dv, dk] float32).  ``out`` / ``S_out`` may supply the
    output tensors (S_out may be S0: the update is then in place).
    ``segments`` (0 .. 64) calls gdn_replay_segmented with that many time
    segments per sequence; None calls gdn_replay.
    """
    return _replay(q, k, v, alpha, beta, cu_seqlens, S0, want_o, o_dtype, out, S_out, stream, segments, False)


def replay_raw(q_raw, k_raw, v, g, b, cu_seqlens, S0=None, want_o=True, o_dtype=None,
               out=None, S_out=None, stream=None):
    """gdn_replay_raw: the front end (normalised q and k, alpha = exp(g),
    beta = sigmoid(b)) inside the replay, from raw bfloat16 projections.
    Arguments and results as replay, with q_raw, k_raw, g and b in place of
    q, k, alpha and beta."""
    return _replay(q_raw, k_raw, v, g, b, cu_seqlens, S0, want_o, o_dtype, out, S_out, stream, None, True)


def _replay(q, k, v, alpha, beta, cu_seqlens, S0, want_o, o_dtype, out, S_out, stream, segments, raw):
    torch = _torch()
    lib = library()
    for name, t in (("k", k), ("v", v), ("alpha", alpha), ("beta", beta),
                    ("cu_seqlens", cu_seqlens), ("S0", S0)):
        _dev(t, name)
    if want_o:
        _dev(q, "q")
    T, H, dk = k.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    in_code = _dtype_code(k.dtype)
    for name, t in (("q", q if want_o else None), ("v", v), ("alpha", alpha), ("beta", beta)):
        if t is not None and t.dtype != k.dtype:
            raise TypeError("%s must have the dtype of k" % name)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    if S0 is not None and S0.dtype != torch.float32:
        raise TypeError("S0 must be float32")
    o = None
    if want_o:
        o_dt = torch.float32 if o_dtype is None else o_dtype
        o = out if out is not None else torch.empty((T, H, dv), dtype=o_dt, device=k.device)
        _dev(o, "out")
        o_code = _dtype_code(o.dtype)
    else:
        o_code = GDN_F32
    S = S_out if S_out is not None else torch.empty((N, H, dv, dk), dtype=torch.float32,
                                                    device=k.device)
    _dev(S, "S_out")
    args = (_ptr(q) if want_o else None, _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
            _ptr(S0), _ptr(cu_seqlens), N, T, H, dk, dv, in_code, _ptr(o), o_code, _ptr(S))
    if raw:
        ws, ws_bytes = _workspace(lib.gdn_replay_raw_workspace_bytes(N, T, H, dk, dv), k.device, stream)
        _check(lib.gdn_replay_raw(*args, _ptr(ws), ws_bytes, _stream_ptr(stream)))
    elif segments is None:
        ws, ws_bytes = _workspace(lib.gdn_replay_workspace_bytes(N, T, H, dk, dv), k.device, stream)
        _check(lib.gdn_replay(*args, _ptr(ws), ws_bytes, _stream_ptr(stream)))
    else:
        ws, ws_bytes = _workspace(lib.gdn_replay_segmented_workspace_bytes(N, T, H, dk, dv, int(segments)),
                                  k.device, stream)
        _check(lib.gdn_replay_segmented(*args, int(segments), _ptr(ws), ws_bytes, _stream_ptr(stream)))
    return o, S


def replay_noalloc(q, k, v, alpha, beta, cu_seqlens, S0=None, want_o=True, o_dtype=None,
                   out=None, S_out=None, stream=None):
    """replay() through gdn_replay_noalloc: no workspace is allocated; the
    library's built-in per-GPU scratch serves instead (calls that overlap on
    one GPU race on it).  Pass ``out`` / ``S_out`` to allocate nothing at all
    (e.g. under graph capture); otherwise the outputs are allocated here.
    """
    torch = _torch()
    lib = library()
    for name, t in (("k", k), ("v", v), ("alpha", alpha), ("beta", beta),
                    ("cu_seqlens", cu_seqlens), ("S0", S0)):
        _dev(t, name)
    if want_o:
        _dev(q, "q")
    T, H, dk = k.shape
    dv = v.shape[2]
    N = cu_seqlens.shape[0] - 1
    in_code = _dtype_code(k.dtype)
    for name, t in (("q", q if want_o else None), ("v", v), ("alpha", alpha), ("beta", beta)):
        if t is not None and t.dtype != k.dtype:
            raise TypeError("%s must have the dtype of k" % name)
    if cu_seqlens.dtype != torch.int32:
        raise TypeError("cu_seqlens must be int32")
    o, o_code = None, GDN_F32
    if want_o:
        o = out if out is not None else torch.empty((T, H, dv), dtype=o_dtype or torch.float32, device=k.device)
        _dev(o, "out")
        o_code = _dtype_code(o.dtype)
    S = S_out if S_out is not None else torch.empty((N, H, dv, dk), dtype=torch.float32, device=k.device)
    _dev(S, "S_out")
    _check(lib.gdn_replay_noalloc(_ptr(q) if want_o else None, _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                  _ptr(S0), _ptr(cu_seqlens), N, T, H, dk, dv, in_code, _ptr(o), o_code,
                                  _ptr(S), _stream_ptr(stream)))
    return o, S


def front_end(q_raw, k_raw, g, b, out=None, stream=None):
    """Normalised q and k and activated gates, the inputs of the recurrence.

    q_raw, k_raw [T, H, dk]; g (log-gate), b (beta logit) [T, H]; all
    float32 or all bfloat16; q_raw may be None.  Returns (q or None, k,
    alpha, beta) in the input dtype: q / |q|, k / |k|, exp(g), sigmoid(b).
    ``out`` = (q, k, alpha, beta) tensors to write into (they may be the
    inputs themselves; q None when q_raw is None).
    """
    lib = library()
    for name, t in (("k_raw", k_raw), ("g", g), ("b", b)):
        _dev(t, name)
    if q_raw is not None:
        _dev(q_raw, "q_raw")
    T, H, dk = k_raw.shape
    code = _dtype_code(k_raw.dtype)
    for name, t in (("q_raw", q_raw), ("g", g), ("b", b)):
        if t is not None and t.dtype != k_raw.dtype:
            raise TypeError("%s must have the dtype of k_raw" % name)
    if out is None:
        out = (None if q_raw is None else q_raw.new_empty(q_raw.shape), k_raw.new_empty(k_raw.shape),
               g.new_empty(g.shape), b.new_empty(b.shape))
    q, k, alpha, beta = out
    for name, t in (("k", k), ("alpha", alpha), ("beta", beta)) + ((("q", q),) if q is not None else ()):
        _dev(t, name)
    if T == 0:    # empty tensors may have no storage; nothing to compute
        return q, k, alpha, beta
    _check(lib.gdn_front_end(_ptr(q_raw), _ptr(k_raw), _ptr(g), _ptr(b), T, H, dk, code, _ptr(q), _ptr(k),
                             _ptr(alpha), _ptr(beta), _stream_ptr(stream)))
    return q, k, alpha, beta


def scalar_chunk_operator(k, alpha, beta, cu_chunks, v=None, stream=None):
    """Scalar-decay chunk operators: gamma [C, H] (the product of the
    chunk's alphas) and S_local [C, H, dv, dk] (None when v is None), float32."""
    torch = _torch()
    lib = library()
    for name, t in (("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("cu_chunks", cu_chunks)):
        _dev(t, name)
    T, H, dk = k.shape
    dv = v.shape[2] if v is not None else dk
    C = cu_chunks.shape[0] - 1
    if cu_chunks.dtype != torch.int32:
        raise TypeError("cu_chunks must be int32")
    gamma = torch.empty((C, H), dtype=torch.float32, device=k.device)
    SL = torch.empty((C, H, dv, dk), dtype=torch.float32, device=k.device) if v is not None else None
    _check(lib.gdn_scalar_chunk_operator(_ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(cu_chunks), C, T, H, dk,
                                         dv, _dtype_code(k.dtype), _ptr(gamma), _ptr(SL), _stream_ptr(stream)))
    return gamma, SL


def scalar_compose(gamma, S_local, S_in=None, out=None, stream=None):
    """S <- gamma[c] S + S_local[c] over the chunks in order, from S_in or zero."""
    torch = _torch()
    lib = library()
    for name, t in (("gamma", gamma), ("S_local", S_local), ("S_in", S_in)):
        _dev(t, name)
    C, H, dv, dk = S_local.shape
    S = out if out is not None else torch.empty((H, dv, dk), dtype=torch.float32, device=S_local.device)
    _dev(S, "out")
    _check(lib.gdn_scalar_compose(_ptr(S_in), _ptr(gamma), _ptr(S_local), C, H, dk, dv, _ptr(S),
                                  _stream_ptr(stream)))
    return S


def decode(q, k, v, alpha, beta, S_in=None, want_o=True, o_dtype=None, out=None, S_out=None,
           stream=None):
    """One token per sequence from the states S_in (the step after a replay).

    q, k [N, H, dk]; v [N, H, dv]; alpha, beta [N, H] (all float32 or all
    bfloat16); S_in [N, H, dv, dk] float32 or None (zero state).  Returns
    (o [N, H, dv] or None, S [N, H, dv, dk] float32).  ``S_out`` may be S_in
    (the states are then updated in place).
    """
    torch = _torch()
    lib = library()
    for name, t in (("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("S_in", S_in)):
        _dev(t, name)
    if want_o:
        _dev(q, "q")
    N, H, dk = k.shape
    dv = v.shape[2]
    in_code = _dtype_code(k.dtype)
    for name, t in (("q", q if want_o else None), ("v", v), ("alpha", alpha), ("beta", beta)):
        if t is not None and t.dtype != k.dtype:
            raise TypeError("%s must have the dtype of k" % name)
    if S_in is not None and S_in.dtype != torch.float32:
        raise TypeError("S_in must be float32")
    o = None
    o_code = GDN_F32
    if want_o:
        o_dt = torch.float32 if o_dtype is None else o_dtype
        o = out if out is not None else torch.empty((N, H, dv), dtype=o_dt, device=k.device)
        _dev(o, "out")
        o_code = _dtype_code(o.dtype)
    S = S_out if S_out is not None else torch.empty((N, H, dv, dk), dtype=torch.float32, device=k.device)
    _dev(S, "S_out")
    _check(lib.gdn_decode(_ptr(q) if want_o else None, _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                          _ptr(S_in), N, H, dk, dv, in_code, _ptr(o), o_code, _ptr(S),
                          _stream_ptr(stream)))
    return o, S


def chunk_operator(k, alpha, beta, cu_chunks, v=None, stream=None):
    """Per-chunk transition product T_C [C, H, dk, dk] and local state
    S_local [C, H, dv, dk] (None when v is None), both float32."""
    torch = _torch()
    lib = library()
    for name, t in (("k", k), ("v", v), ("alpha", alpha), ("beta", beta), ("cu_chunks", cu_chunks)):
        _dev(t, name)
    T, H, dk = k.shape
    dv = v.shape[2] if v is not None else dk
    C = cu_chunks.shape[0] - 1
    in_code = _dtype_code(k.dtype)
    if cu_chunks.dtype != torch.int32:
        raise TypeError("cu_chunks must be int32")
    TC = torch.empty((C, H, dk, dk), dtype=torch.float32, device=k.device)
    SL = torch.empty((C, H, dv, dk), dtype=torch.float32, device=k.device) if v is not None else None
    ws_bytes = lib.gdn_chunk_operator_workspace_bytes(C, T, H, dk, dv)
    ws, ws_bytes = _workspace(ws_bytes, k.device, stream)
    _check(lib.gdn_chunk_operator(_ptr(k), _ptr(v), _ptr(alpha), _ptr(beta), _ptr(cu_chunks), C, T,
                                  H, dk, dv, in_code, _ptr(TC), _ptr(SL), _ptr(ws), ws_bytes,
                                  _stream_ptr(stream)))
    return TC, SL


def compose(T_C, S_local, S_in=None, out=None, stream=None):
    """S <- S_in (or 0); S <- S T_C[c] + S_local[c] for c in context order.
    Returns S_out [H, dv, dk] float32."""
    torch = _torch()
    lib = library()
    for name, t in (("T_C", T_C), ("S_local", S_local), ("S_in", S_in)):
        _dev(t, name)
    C, H, dk, _ = T_C.shape
    dv = S_local.shape[2]
    S = out if out is not None else torch.empty((H, dv, dk), dtype=torch.float32, device=T_C.device)
    _dev(S, "out")
    ws_bytes = lib.gdn_compose_workspace_bytes(C, H, dk, dv)
    ws, ws_bytes = _workspace(ws_bytes, T_C.device, stream)
    _check(lib.gdn_compose(_ptr(S_in), _ptr(T_C), _ptr(S_local), C, H, dk, dv, _ptr(S),
                           _ptr(ws), ws_bytes, _stream_ptr(stream)))
    return S
