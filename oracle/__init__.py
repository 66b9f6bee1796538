"""fp64 CPU oracle for Gated DeltaNet replay, chunk operators and composition.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
CPU-baseline leg of the benchmark, never by the product path.  It shares no
code with the HIP library and imports nothing from it.

The recurrence's arithmetic lives in ``gdn_oracle.c`` (plain sequential
loops in double precision); this module builds it with gcc and marshals numpy
arrays.  The front end (normalisation and gate activations) and the scalar-decay
operator and composition are written here in numpy float64.

Sources: "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching
for Hybrid LLMs", section 2 Eq. (1) and section 3 Eq. (2); "LinearKV: One
Cached State Suffices for Position-Independent Caching in Hybrid LLMs", the
affine chunk operator and its back-to-back composition in context order.

Parity pins (tests/test_oracle_pins.py) tie every function here to facts the
pages and the mathematics fix, the two error measures (rel_fro,
rel_fro_blocks) included; none of them is "parity unpinned".
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None


def build(force: bool = False) -> str:
    """Compile gdn_oracle.c into liboracle.so with gcc (OpenMP over heads)."""
    if force or not os.path.exists(_LIB_PATH) or (
            os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC)):
        tmp = _LIB_PATH + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-std=c99", "-fopenmp", "-fPIC", "-shared",
               "-Wall", "-o", tmp, _SRC]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is None:
        build()
        lib = ctypes.CDLL(_LIB_PATH)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int32)
        lib.gdn_oracle_replay.argtypes = [dp, dp, dp, dp, dp, dp, ip,
                                          ctypes.c_int, ctypes.c_int64,
                                          ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                          dp, dp, ctypes.c_int]
        lib.gdn_oracle_chunk_operator.argtypes = [dp, dp, dp, dp, ip, ctypes.c_int,
                                                  ctypes.c_int64, ctypes.c_int,
                                                  ctypes.c_int, ctypes.c_int,
                                                  dp, dp, ctypes.c_int]
        lib.gdn_oracle_compose.argtypes = [dp, dp, dp, ctypes.c_int, ctypes.c_int,
                                           ctypes.c_int, ctypes.c_int, dp, ctypes.c_int]
        lib.gdn_oracle_threads.argtypes = []
        for f in (lib.gdn_oracle_replay, lib.gdn_oracle_chunk_operator,
                  lib.gdn_oracle_compose, lib.gdn_oracle_threads):
            f.restype = ctypes.c_int
        _lib = lib
    return _lib


def threads() -> int:
    """Default OpenMP thread count the oracle uses."""
    return int(_load().gdn_oracle_threads())


def _f64(a):
    if a is None:
        return None
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int32))


def replay(q, k, v, alpha, beta, cu_seqlens, S0=None, want_o=True, n_threads=0):
    """Sequential per-token replay (Tail-Replay Eq. (1); Eq. (2) when S0 is None).

    Shapes: q, k [T, H, dk]; v [T, H, dv]; alpha, beta [T, H];
    cu_seqlens int [N+1]; S0 [N, H, dv, dk] or None (zero state).
    Returns (o [T, H, dv] or None, S_final [N, H, dv, dk]) in float64.
    """
    k, v, alpha, beta = _f64(k), _f64(v), _f64(alpha), _f64(beta)
    q = _f64(q) if (want_o and q is not None) else None
    if want_o and q is None:
        raise ValueError("o requested without q")
    cu = np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))
    T, H, dk = k.shape
    dv = v.shape[2]
    N = cu.shape[0] - 1
    S0 = _f64(S0)
    o = np.empty((T, H, dv), np.float64) if want_o else None
    S = np.empty((N, H, dv, dk), np.float64)
    rc = _load().gdn_oracle_replay(_ptr(q), _ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                   _ptr(S0), _iptr(cu), N, T, H, dk, dv,
                                   _ptr(o), _ptr(S), int(n_threads))
    if rc != 0:
        raise ValueError("oracle replay rejected its arguments")
    return o, S


def chunk_operator(k, alpha, beta, cu_chunks, v=None, n_threads=0):
    """Per-chunk transition product and local state (LinearKV chunk operator).

    Returns (T_C [C, H, dk, dk], S_local [C, H, dv, dk] or None) in float64.
    """
    k, alpha, beta = _f64(k), _f64(alpha), _f64(beta)
    v = _f64(v)
    cu = np.ascontiguousarray(np.asarray(cu_chunks, dtype=np.int32))
    T, H, dk = k.shape
    C = cu.shape[0] - 1
    dv = v.shape[2] if v is not None else dk
    TC = np.empty((C, H, dk, dk), np.float64)
    SL = np.empty((C, H, dv, dk), np.float64) if v is not None else None
    rc = _load().gdn_oracle_chunk_operator(_ptr(k), _ptr(v), _ptr(alpha), _ptr(beta),
                                           _iptr(cu), C, T, H, dk, dv,
                                           _ptr(TC), _ptr(SL), int(n_threads))
    if rc != 0:
        raise ValueError("oracle chunk_operator rejected its arguments")
    return TC, SL


def compose(T_C, S_local, S_in=None, n_threads=0):
    """Back-to-back composition S <- S T_C[c] + S_local[c] in context order.

    T_C [C, H, dk, dk], S_local [C, H, dv, dk], S_in [H, dv, dk] or None.
    Returns S_out [H, dv, dk] in float64.
    """
    T_C, S_local, S_in = _f64(T_C), _f64(S_local), _f64(S_in)
    C, H, dk, _ = T_C.shape
    dv = S_local.shape[2]
    out = np.empty((H, dv, dk), np.float64)
    rc = _load().gdn_oracle_compose(_ptr(S_in), _ptr(T_C), _ptr(S_local), C, H, dk, dv,
                                    _ptr(out), int(n_threads))
    if rc != 0:
        raise ValueError("oracle compose rejected its arguments")
    return out


def front_end(q_raw, k_raw, g, b):
    """The inputs of the recurrence from raw projections, in float64.

    Tail-Replay, section 3 (the replayed hidden states produce the keys,
    transitions and write strengths) and section 2 Eq. (1) (alpha in (0, 1]):
    q and k divided by their Euclidean norm over the last axis (a zero row
    stays zero), alpha = exp(g) from the log-gate, beta = the logistic
    sigmoid of its logit.  q_raw may be None.  Returns (q, k, alpha, beta).
    """
    def unit(x):
        x = _f64(x)
        n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        return np.divide(x, n, out=np.zeros_like(x), where=n > 0)
    q = None if q_raw is None else unit(q_raw)
    return q, unit(k_raw), np.exp(_f64(g)), 1.0 / (1.0 + np.exp(-_f64(b)))


def scalar_chunk_operator(k, alpha, beta, cu_chunks, v=None):
    """Chunk operators of the scalar-decay recurrence, in float64.

    LinearKV, the affine-operator paragraph (with a scalar per-token
    transition the chunk's transition is a single scalar decay) and the
    write term of Tail-Replay section 2 Eq. (1): per head,
    S_t = alpha_t S_{t-1} + beta_t v_t k_t^T, run token by token from zero
    over each chunk.  Returns (gamma [C, H], S_local [C, H, dv, dk] or None).
    """
    k, a, b = _f64(k), _f64(alpha), _f64(beta)
    v = _f64(v)
    cu = np.asarray(cu_chunks, np.int64)
    C, H, dk = cu.shape[0] - 1, k.shape[1], k.shape[2]
    gamma = np.ones((C, H))
    SL = None if v is None else np.zeros((C, H, v.shape[2], dk))
    for c in range(C):
        for t in range(cu[c], cu[c + 1]):
            gamma[c] *= a[t]
            if SL is not None:
                SL[c] = a[t][:, None, None] * SL[c] + b[t][:, None, None] * v[t][:, :, None] * k[t][:, None, :]
    return gamma, SL


def scalar_compose(gamma, S_local, S_in=None):
    """Scalar-decay operators back to back in context order (LinearKV, the
    composition paragraph): S <- gamma[c] S + S_local[c], from S_in or zero."""
    g, SL = _f64(gamma), _f64(S_local)
    S = np.zeros(SL.shape[1:]) if S_in is None else _f64(S_in).copy()
    for c in range(SL.shape[0]):
        S = g[c][:, None, None] * S + SL[c]
    return S


def rel_fro(x, ref) -> float:
    """Relative Frobenius error ||x - ref||_F / ||ref||_F over the whole tensor.

    The error measure of the LinearKV state probe (relative state error
    against the full-prefix state).  When ||ref|| is 0 the absolute norm of
    x is returned instead.
    """
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    den = float(np.linalg.norm(ref.ravel()))
    num = float(np.linalg.norm((x - ref).ravel()))
    return num / den if den > 0 else num


def rel_fro_blocks(x, ref, nred: int, floor: float = 0.0) -> np.ndarray:
    """Relative Frobenius error of every block of a tensor.

    A block is one index of the leading axes, the last ``nred`` axes being
    reduced: for a state [N, H, dv, dk] with nred = 2 a block is one
    (sequence, head) matrix; for outputs [T, H, dv] with nred = 1 a block is
    one token row of one head.  Block b's error is
        ||x_b - ref_b||_F / max(||ref_b||_F, floor * r),
    r being the root mean square of ||ref_b||_F over all blocks, so that a
    block whose reference is tiny against the rest is measured against a
    fraction ``floor`` of the typical block (0 = plain relative error).
    Where that denominator is 0 the block's absolute error is returned.
    The per-block form of the LinearKV state probe's relative error.
    """
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    if x.shape != ref.shape or not 0 <= nred <= ref.ndim:
        raise ValueError("rel_fro_blocks: shapes %s / %s, nred %d" % (x.shape, ref.shape, nred))
    lead = ref.shape[:ref.ndim - nred]
    d = (x - ref).reshape(lead + (-1,))
    r = ref.reshape(lead + (-1,))
    num = np.asarray(np.sqrt(np.sum(d * d, axis=-1)))
    den = np.asarray(np.sqrt(np.sum(r * r, axis=-1)))
    if floor > 0 and den.size:
        den = np.maximum(den, floor * np.sqrt(np.mean(den * den)))
    return np.divide(num, den, out=np.array(num), where=den > 0)
