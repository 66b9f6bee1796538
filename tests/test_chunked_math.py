"""The chunkwise-parallel form used by the HIP kernels, written in fp64 numpy,
against the sequential oracle (CPU only).

This checks the algebra the kernels are built on before any GPU code runs:
within a chunk of L tokens with cumulative log-gates g_r = sum_{s<=r} log alpha_s,
  A   = strictly-lower  beta_r exp(g_r - g_s) (k_r . k_s)
  Tau = (I + A)^{-1}                       (unit lower triangular)
  W   = Tau diag(beta exp(g)) K,   U = Tau diag(beta) V
  D   = U - W S^T                  (the per-token delta-rule corrections)
  O   = diag(exp(g)) Q S^T + (M o Q K^T) D,  M_rs = exp(g_r - g_s) for s <= r
  S  <- exp(g_L) S + (diag(exp(g_L - g)) D)^T K
and the chunk operator T_C = exp(g_L) I - W^T diag(exp(g_L - g)) K,
S_local = U^T diag(exp(g_L - g)) K.  These follow from unrolling the
Tail-Replay Eq. (1) recurrence over the chunk.
"""
import numpy as np
import pytest

import oracle


def chunked_replay(q, k, v, a, b, S0, C):
    T, dk = k.shape
    dv = v.shape[1]
    S = S0.copy()
    O = np.zeros((T, dv))
    for c0 in range(0, T, C):
        sl = slice(c0, min(T, c0 + C))
        K, Q, V = k[sl], q[sl], v[sl]
        g = np.cumsum(np.log(a[sl]))
        L = K.shape[0]
        diff = g[:, None] - g[None, :]
        low = np.tril(np.ones((L, L)), -1)
        A = b[sl][:, None] * np.exp(np.where(low > 0, diff, 0.0)) * (K @ K.T) * low
        Tau = np.linalg.inv(np.eye(L) + A)
        W = Tau @ (np.diag(b[sl] * np.exp(g)) @ K)
        U = Tau @ (np.diag(b[sl]) @ V)
        D = U - W @ S.T
        M = np.exp(np.where(np.tril(np.ones((L, L))) > 0, diff, -np.inf))
        O[sl] = np.exp(g)[:, None] * (Q @ S.T) + (M * (Q @ K.T)) @ D
        dec = np.exp(g[-1] - g)
        S = np.exp(g[-1]) * S + (dec[:, None] * D).T @ K
    return O, S


def chunk_operator_form(k, a, b, v):
    g = np.cumsum(np.log(a))
    L = k.shape[0]
    diff = g[:, None] - g[None, :]
    low = np.tril(np.ones((L, L)), -1)
    A = b[:, None] * np.exp(np.where(low > 0, diff, 0.0)) * (k @ k.T) * low
    Tau = np.linalg.inv(np.eye(L) + A)
    W = Tau @ (np.diag(b * np.exp(g)) @ k)
    U = Tau @ (np.diag(b) @ v)
    dec = np.exp(g[-1] - g)
    TC = np.exp(g[-1]) * np.eye(k.shape[1]) - W.T @ (dec[:, None] * k)
    SL = U.T @ (dec[:, None] * k)
    return TC, SL


@pytest.mark.parametrize("T", [1, 2, 63, 64, 65, 130])
@pytest.mark.parametrize("C", [1, 4, 16, 64])
def test_chunked_equals_sequential(T, C):
    rng = np.random.Generator(np.random.PCG64(100 + T * 7 + C))
    dk, dv = 12, 10
    q = rng.standard_normal((T, 1, dk))
    k = rng.standard_normal((T, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, 1, dv))
    a = np.exp(-0.1 * np.logaddexp(0, rng.standard_normal((T, 1))))
    b = 1 / (1 + np.exp(-rng.standard_normal((T, 1))))
    S0 = rng.standard_normal((1, 1, dv, dk))
    o_ref, S_ref = oracle.replay(q, k, v, a, b, [0, T], S0=S0)
    O, S = chunked_replay(q[:, 0], k[:, 0], v[:, 0], a[:, 0], b[:, 0], S0[0, 0], C)
    assert oracle.rel_fro(S, S_ref[0, 0]) < 1e-13
    assert oracle.rel_fro(O, o_ref[:, 0]) < 1e-13


@pytest.mark.parametrize("L", [1, 5, 64])
def test_chunk_operator_form(L):
    rng = np.random.Generator(np.random.PCG64(200 + L))
    dk, dv = 9, 7
    k = rng.standard_normal((L, 1, dk))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((L, 1, dv))
    a = rng.uniform(0.8, 1.0, (L, 1))
    b = rng.uniform(0.0, 1.0, (L, 1))
    TC_ref, SL_ref = oracle.chunk_operator(k, a, b, [0, L], v=v)
    TC, SL = chunk_operator_form(k[:, 0], a[:, 0], b[:, 0], v[:, 0])
    assert oracle.rel_fro(TC, TC_ref[0, 0]) < 1e-13
    assert oracle.rel_fro(SL, SL_ref[0, 0]) < 1e-13
