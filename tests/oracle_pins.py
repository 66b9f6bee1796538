"""Pins that tie the fp64 oracle to facts fixed by the pages and by algebra.

Each ``pin_*`` function takes an oracle module (the real one, or a mutated
copy in the mutation tests) and raises AssertionError when the oracle
disagrees with the fact it checks.  None of them re-types the oracle's own
rank-1 formula: they use the literal matrix form of the update (forming the
per-token transition explicitly), exact rational arithmetic, closed forms
for special cases, and identities between different oracle entry points.

Facts used (pages cited by title and passage):
  * Tail-Replay, section 2, Eq. (1): the per-token transition
    T = alpha (I - beta k k^T) and the write beta v k^T; alpha in (0, 1].
  * Tail-Replay, section 3, Eq. (2): replay starts from a zero state.
  * LinearKV, affine chunk operator paragraph: a chunk maps S_in to
    S_in T_C + S_local, T_C being the product of the chunk's transitions and
    S_local the state reached from an empty start; applying the operators
    back to back in context order adds no approximation.
"""
from __future__ import annotations

from fractions import Fraction

import numpy as np


def _rng(seed):
    return np.random.Generator(np.random.PCG64(seed))


def _random_inputs(rng, T, H, dk, dv, unit_k=False, alpha=None, beta=None):
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    if unit_k:
        k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    a = rng.uniform(0.5, 1.0, (T, H)) if alpha is None else np.full((T, H), float(alpha))
    b = rng.uniform(0.0, 1.5, (T, H)) if beta is None else np.full((T, H), float(beta))
    return q, k, v, a, b


def _literal_replay(q, k, v, a, b, S0):
    """Eq. (1) with the transition formed as a dk x dk matrix (state dv x dk)."""
    T, H, dk = k.shape
    dv = v.shape[2]
    S = np.array(S0, np.float64, copy=True)
    o = np.zeros((T, H, dv))
    for t in range(T):
        for h in range(H):
            kk = k[t, h][:, None]
            Tm = a[t, h] * (np.eye(dk) - b[t, h] * (kk @ kk.T))
            S[h] = S[h] @ Tm + b[t, h] * (v[t, h][:, None] @ kk.T)
            o[t, h] = S[h] @ q[t, h]
    return o, S


def pin_literal_matrix_form(orc):
    """Oracle replay equals the literal matrix form of Eq. (1) (dk=5, dv=3)."""
    rng = _rng(11)
    T, H, dk, dv = 9, 2, 5, 3
    q, k, v, a, b = _random_inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    o_ref, S_ref = _literal_replay(q, k, v, a, b, S0[0])
    o, S = orc.replay(q, k, v, a, b, [0, T], S0=S0)
    assert np.max(np.abs(S[0] - S_ref)) < 1e-12
    assert np.max(np.abs(o - o_ref)) < 1e-12


def pin_exact_rational(orc):
    """Exact rational arithmetic of Eq. (1) on dyadic inputs (dk=3, dv=2, T=4).

    All inputs are small dyadic rationals, exactly representable in fp64, so
    the exact result is known; the oracle must agree to rounding (1e-14).
    """
    rng = _rng(5)
    T, dk, dv = 4, 3, 2
    def dy(shape, lo, hi, den):
        return rng.integers(lo, hi, size=shape) / den
    q = dy((T, 1, dk), -8, 9, 8)
    k = dy((T, 1, dk), -4, 5, 4)
    v = dy((T, 1, dv), -8, 9, 8)
    a = dy((T, 1), 8, 17, 16)       # alpha in [1/2, 1]
    b = dy((T, 1), 0, 9, 8)         # beta in [0, 1]
    S0 = dy((1, 1, dv, dk), -4, 5, 4)
    Fr = lambda x: Fraction(float(x))
    S = [[Fr(S0[0, 0, i, j]) for j in range(dk)] for i in range(dv)]
    o_exact = []
    for t in range(T):
        kt = [Fr(x) for x in k[t, 0]]
        at, bt = Fr(a[t, 0]), Fr(b[t, 0])
        Tm = [[at * ((1 if i == j else 0) - bt * kt[i] * kt[j]) for j in range(dk)]
              for i in range(dk)]
        S = [[sum(S[i][m] * Tm[m][j] for m in range(dk)) + bt * Fr(v[t, 0, i]) * kt[j]
              for j in range(dk)] for i in range(dv)]
        o_exact.append([sum(S[i][j] * Fr(q[t, 0, j]) for j in range(dk)) for i in range(dv)])
    o, Sf = orc.replay(q, k, v, a, b, [0, T], S0=S0)
    S_ex = np.array([[float(x) for x in r] for r in S])
    o_ex = np.array([[float(x) for x in r] for r in o_exact])
    assert np.max(np.abs(Sf[0, 0] - S_ex)) <= 1e-14 * max(1.0, np.max(np.abs(S_ex)))
    assert np.max(np.abs(o[:, 0] - o_ex)) <= 1e-14 * max(1.0, np.max(np.abs(o_ex)))


def pin_identity_gate(orc):
    """alpha = 1, beta = 0 leaves S unchanged (bitwise) and o_t = S0 q_t."""
    rng = _rng(1)
    T, H, dk, dv = 17, 3, 8, 6
    q, k, v, a, b = _random_inputs(rng, T, H, dk, dv, alpha=1.0, beta=0.0)
    S0 = rng.standard_normal((1, H, dv, dk))
    o, S = orc.replay(q, k, v, a, b, [0, T], S0=S0)
    assert np.array_equal(S, S0)
    ref = np.einsum("hij,thj->thi", S0[0], q)
    assert np.max(np.abs(o - ref)) < 1e-13


def pin_delta_write(orc):
    """Unit keys: S_t k_t = alpha_t (1 - beta_t) S_{t-1} k_t + beta_t v_t.

    With alpha = beta = 1 this is S_t k_t = v_t: the delta rule writes v_t
    under key k_t exactly.  Reading with q = k makes o_t = S_t k_t.
    """
    rng = _rng(2)
    T, H, dk, dv = 12, 2, 16, 7
    q, k, v, a, b = _random_inputs(rng, T, H, dk, dv, unit_k=True)
    S0 = rng.standard_normal((1, H, dv, dk))
    # general form, token by token through the S0 path
    S_prev = S0
    for t in range(T):
        sl = slice(t, t + 1)
        o, S = orc.replay(k[sl], k[sl], v[sl], a[sl], b[sl], [0, 1], S0=S_prev)
        pred = (a[t][:, None] * (1 - b[t])[:, None]
                * np.einsum("hij,hj->hi", S_prev[0], k[t]) + b[t][:, None] * v[t])
        assert np.max(np.abs(o[0] - pred)) < 1e-12
        S_prev = S
    # alpha = beta = 1
    q, k, v, a, b = _random_inputs(rng, T, H, dk, dv, unit_k=True, alpha=1.0, beta=1.0)
    o, _ = orc.replay(k, k, v, a, b, [0, T], S0=S0)
    assert np.max(np.abs(o - v)) < 1e-12


def pin_orthonormal_memory(orc):
    """Orthonormal keys, alpha = beta = 1, zero start: the delta rule is an
    exact associative memory, S_T = sum_t v_t k_t^T and
    o_t = sum_{s<=t} v_s (k_s . q_t)."""
    rng = _rng(3)
    T, H, dk, dv = 10, 2, 12, 5
    k = np.empty((T, H, dk))
    for h in range(H):
        Qm, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        k[:, h] = Qm[:, :T].T
    q = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    a = np.ones((T, H))
    b = np.ones((T, H))
    o, S = orc.replay(q, k, v, a, b, [0, T])
    S_ref = np.einsum("thi,thj->hij", v, k)
    assert np.max(np.abs(S[0] - S_ref)) < 1e-12
    kq = np.einsum("shj,thj->hts", k, q)               # [h, t, s]
    mask = np.tril(np.ones((T, T)))
    o_ref = np.einsum("hts,shi->thi", kq * mask[None], v)
    assert np.max(np.abs(o - o_ref)) < 1e-12


def pin_beta_zero_decay(orc):
    """beta = 0: the state only decays, S_t = (prod alpha) S0."""
    rng = _rng(4)
    T, H, dk, dv = 20, 2, 6, 4
    q, k, v, a, b = _random_inputs(rng, T, H, dk, dv, beta=0.0)
    S0 = rng.standard_normal((1, H, dv, dk))
    _, S = orc.replay(q, k, v, a, b, [0, T], S0=S0, want_o=False)
    ref = np.prod(a, axis=0)[:, None, None] * S0[0]
    assert np.max(np.abs(S[0] - ref)) < 1e-13


def pin_split_resume(orc):
    """Replaying A then B from A's state equals replaying A||B (bitwise)."""
    rng = _rng(6)
    T, H, dk, dv = 40, 2, 8, 8
    q, k, v, a, b = _random_inputs(rng, T, H, dk, dv)
    S0 = rng.standard_normal((1, H, dv, dk))
    o_all, S_all = orc.replay(q, k, v, a, b, [0, T], S0=S0)
    c = 13
    o1, S1 = orc.replay(q[:c], k[:c], v[:c], a[:c], b[:c], [0, c], S0=S0)
    o2, S2 = orc.replay(q[c:], k[c:], v[c:], a[c:], b[c:], [0, T - c], S0=S1)
    assert np.array_equal(S2, S_all)
    assert np.array_equal(np.concatenate([o1, o2]), o_all)


def pin_varlen_and_heads(orc):
    """A packed batch equals one call per sequence; zero-length sequences
    return their start state; permuting heads permutes the outputs."""
    rng = _rng(7)
    lens = [5, 0, 11, 1, 0, 7]
    H, dk, dv = 3, 6, 4
    T = sum(lens)
    q, k, v, a, b = _random_inputs(rng, T, H, dk, dv)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    S0 = rng.standard_normal((len(lens), H, dv, dk))
    o, S = orc.replay(q, k, v, a, b, cu, S0=S0)
    for n, L in enumerate(lens):
        sl = slice(cu[n], cu[n + 1])
        on, Sn = orc.replay(q[sl], k[sl], v[sl], a[sl], b[sl], [0, L], S0=S0[n:n + 1])
        assert np.array_equal(Sn[0], S[n])
        assert np.array_equal(on, o[sl])
        if L == 0:
            assert np.array_equal(S[n], S0[n])
    _, Sz = orc.replay(q, k, v, a, b, cu, S0=None, want_o=False)
    for n, L in enumerate(lens):
        if L == 0:
            assert not np.any(Sz[n])
    perm = np.array([2, 0, 1])
    op, Sp = orc.replay(q[:, perm], k[:, perm], v[:, perm], a[:, perm], b[:, perm], cu,
                        S0=S0[:, perm])
    assert np.array_equal(Sp, S[:, perm])
    assert np.array_equal(op, o[:, perm])


def pin_single_token_operator(orc):
    """The operator of a one-token chunk is that token's transition
    alpha (I - beta k k^T), and its local state is beta v k^T."""
    rng = _rng(8)
    H, dk, dv = 2, 7, 3
    _, k, v, a, b = _random_inputs(rng, 1, H, dk, dv)
    TC, SL = orc.chunk_operator(k, a, b, [0, 1], v=v)
    for h in range(H):
        kk = k[0, h][:, None]
        ref = a[0, h] * (np.eye(dk) - b[0, h] * kk @ kk.T)
        assert np.max(np.abs(TC[0, h] - ref)) < 1e-15
        assert np.max(np.abs(SL[0, h] - b[0, h] * v[0, h][:, None] @ kk.T)) < 1e-15


def pin_operator_determinant_and_kernel(orc):
    """log|det T_C| = sum_t (dk log alpha_t + log|1 - beta_t ||k_t||^2|)
    (matrix determinant lemma per factor), and T_C x = (prod alpha) x for
    x orthogonal to every key of the chunk (L < dk)."""
    rng = _rng(9)
    L, H, dk = 5, 2, 9
    _, k, _, a, b = _random_inputs(rng, L, H, dk, 1)
    TC, _ = orc.chunk_operator(k, a, b, [0, L])
    for h in range(H):
        sign, logdet = np.linalg.slogdet(TC[0, h])
        ref = np.sum(dk * np.log(a[:, h]) + np.log(np.abs(1 - b[:, h] * np.sum(k[:, h] ** 2, -1))))
        assert abs(logdet - ref) < 1e-9
        # null space of the keys
        Kh = k[:, h]                                    # [L, dk]
        _, _, Vt = np.linalg.svd(Kh)
        X = Vt[L:]                                      # rows orthogonal to all keys
        g = np.prod(a[:, h])
        # S_out = S_in T_C, so a row vector x^T with x orthogonal to the keys maps to g x^T
        assert np.max(np.abs(X @ TC[0, h] - g * X)) < 1e-13
        # and the operator is not trivial along a key
        assert np.max(np.abs(Kh @ TC[0, h] - g * Kh)) > 1e-6


def pin_compose_equals_sequential(orc):
    """S_seq = S_in T_C + S_local chunk after chunk, in context order, for
    uneven chunks and a nonzero incoming state (LinearKV composition)."""
    rng = _rng(10)
    H, dk, dv = 2, 6, 5
    bounds = np.array([0, 4, 4, 13, 14, 30], np.int32)
    T = int(bounds[-1])
    q, k, v, a, b = _random_inputs(rng, T, H, dk, dv)
    S_in = rng.standard_normal((1, H, dv, dk))
    _, S_seq = orc.replay(q, k, v, a, b, [0, T], S0=S_in, want_o=False)
    TC, SL = orc.chunk_operator(k, a, b, bounds, v=v)
    S_c = orc.compose(TC, SL, S_in=S_in[0])
    assert np.max(np.abs(S_c - S_seq[0])) < 1e-12
    # no chunks: the incoming state is returned
    S_e = orc.compose(TC[:0], SL[:0], S_in=S_in[0])
    assert np.array_equal(S_e, S_in[0])
    # empty chunk: identity operator, zero local state
    assert np.array_equal(TC[1], np.broadcast_to(np.eye(dk), (H, dk, dk)))
    assert not np.any(SL[1])


def pin_tail_error_identity(orc):
    """Replaying only the tail from zero misses exactly the carried state:
    S_full(m) - S_tail(m) = S_full(m - k) T_tail."""
    rng = _rng(12)
    m, kk, H, dk, dv = 50, 17, 2, 6, 6
    q, k, v, a, b = _random_inputs(rng, m, H, dk, dv, unit_k=True)
    _, S_full = orc.replay(q, k, v, a, b, [0, m], want_o=False)
    _, S_head = orc.replay(q[:m - kk], k[:m - kk], v[:m - kk], a[:m - kk], b[:m - kk],
                           [0, m - kk], want_o=False)
    _, S_tail = orc.replay(q[m - kk:], k[m - kk:], v[m - kk:], a[m - kk:], b[m - kk:],
                           [0, kk], want_o=False)
    TC, _ = orc.chunk_operator(k[m - kk:], a[m - kk:], b[m - kk:], [0, kk])
    lhs = S_full[0] - S_tail[0]
    rhs = np.einsum("hij,hjk->hik", S_head[0], TC[0])
    assert np.max(np.abs(lhs - rhs)) < 1e-12 * max(1.0, np.max(np.abs(S_full)))
    assert np.max(np.abs(rhs)) > 1e-6


def pin_front_end_values(orc):
    # Tail-Replay, section 3 (the replayed hidden states produce k, the
    # transitions and beta) with section 2 Eq. (1): worked by hand.
    # (3, 4) has norm 5; a zero row stays zero; exp(log 1/2) = 1/2;
    # sigmoid(log 3) = 3/4 and sigmoid(-log 3) = 1/4.
    k = np.array([[[3.0, 4.0, 0.0, 0.0]], [[0.0, 0.0, 0.0, 0.0]], [[-1.0, 1.0, -1.0, 1.0]]])
    q = np.array([[[0.0, 0.0, 0.0, 2.0]], [[1e-3, 0.0, 0.0, 0.0]], [[1.0, 2.0, 2.0, 0.0]]])
    g = np.array([[0.0], [np.log(0.5)], [-np.inf]])
    b = np.array([[0.0], [np.log(3.0)], [-np.log(3.0)]])
    qo, ko, a, be = orc.front_end(q, k, g, b)
    assert np.array_equal(ko, [[[0.6, 0.8, 0.0, 0.0]], [[0.0, 0.0, 0.0, 0.0]], [[-0.5, 0.5, -0.5, 0.5]]])
    assert np.allclose(qo, [[[0, 0, 0, 1.0]], [[1.0, 0, 0, 0]], [[1 / 3, 2 / 3, 2 / 3, 0]]], rtol=0, atol=1e-15)
    assert np.allclose(a, [[1.0], [0.5], [0.0]], rtol=0, atol=1e-15)
    assert np.allclose(be, [[0.5], [0.75], [0.25]], rtol=0, atol=1e-15)
    assert orc.front_end(None, k, g, b)[0] is None


def pin_front_end_invariants(orc):
    # unit rows, invariance under positive scaling, oddness, alpha in (0, 1]
    # for g <= 0, beta(b) + beta(-b) = 1
    rng = _rng(31)
    x = rng.standard_normal((50, 3, 128)) * rng.uniform(0.01, 100, (50, 3, 1))
    g = -np.abs(rng.standard_normal((50, 3))) * 5
    b = rng.standard_normal((50, 3)) * 4
    q, k, a, be = orc.front_end(x, x, g, b)
    assert np.max(np.abs(np.linalg.norm(k, axis=-1) - 1)) < 1e-14
    assert np.array_equal(q, k)
    _, k2, _, _ = orc.front_end(None, 7.5 * x, g, b)
    assert np.max(np.abs(k2 - k)) < 1e-15
    _, k3, _, _ = orc.front_end(None, -x, g, b)
    assert np.array_equal(k3, -k)
    assert np.max(np.abs(k * np.linalg.norm(x, axis=-1, keepdims=True) - x)) < 1e-12 * np.max(np.abs(x))
    assert np.all((a > 0) & (a <= 1))
    assert np.max(np.abs(be + orc.front_end(None, x, g, -b)[3] - 1)) < 1e-15


def pin_scalar_by_hand(orc):
    # one head, dk = dv = 1, alpha = (1/2, 1/2, 1/4), beta = 1, v = (1, 2, 4),
    # k = (1, 1, 1/2): S = 1; then 1/2 + 2 = 5/2; then 5/8 + 2 = 21/8;
    # gamma = 1/16.  A second chunk that is empty gives gamma 1 and S 0.
    k = np.array([[[1.0]], [[1.0]], [[0.5]]])
    v = np.array([[[1.0]], [[2.0]], [[4.0]]])
    a = np.array([[0.5], [0.5], [0.25]])
    b = np.ones((3, 1))
    g, SL = orc.scalar_chunk_operator(k, a, b, [0, 3, 3], v=v)
    assert np.array_equal(g, [[1 / 16], [1.0]])
    assert np.array_equal(SL[:, 0, 0, 0], [21 / 8, 0.0])
    assert orc.scalar_chunk_operator(k, a, b, [0, 3])[1] is None
    # composed from S_in = 8: 8/16 + 21/8 = 25/8, then the empty chunk
    assert np.array_equal(orc.scalar_compose(g, SL, S_in=np.array([[[8.0]]])), [[[25 / 8]]])


def pin_scalar_closed_forms(orc):
    # alpha = 1: S_local = V^T diag(beta) K.  General alpha: the sum of
    # beta_t (prod_{s>t} alpha_s) v_t k_t^T with the products formed one by one.
    rng = _rng(41)
    T, H, dk, dv = 37, 2, 5, 3
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    a = rng.uniform(0.5, 1.0, (T, H))
    b = rng.uniform(0.0, 1.0, (T, H))
    _, SL1 = orc.scalar_chunk_operator(k, np.ones((T, H)), b, [0, T], v=v)
    for h in range(H):
        ref = v[:, h].T @ np.diag(b[:, h]) @ k[:, h]
        assert np.max(np.abs(SL1[0, h] - ref)) < 1e-12
    g, SL = orc.scalar_chunk_operator(k, a, b, [0, T], v=v)
    for h in range(H):
        ref = sum(b[t, h] * np.prod(a[t + 1:, h]) * np.outer(v[t, h], k[t, h]) for t in range(T))
        assert np.max(np.abs(SL[0, h] - ref)) < 1e-12
        assert abs(g[0, h] - np.prod(a[:, h])) < 1e-15


def pin_scalar_compose_is_concatenation(orc):
    # composing the operators of consecutive chunks gives the operator of the
    # whole span: gamma multiplies, S_local = gamma_2 S_1 + S_2
    rng = _rng(42)
    T, H, dk, dv = 90, 3, 4, 6
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    a = rng.uniform(0.8, 1.0, (T, H))
    b = rng.uniform(0.0, 1.0, (T, H))
    g, SL = orc.scalar_chunk_operator(k, a, b, [0, 20, 20, 61, 90], v=v)
    g1, SL1 = orc.scalar_chunk_operator(k, a, b, [0, 90], v=v)
    assert np.max(np.abs(orc.scalar_compose(g, SL) - SL1[0])) < 1e-12
    assert np.max(np.abs(np.prod(g, axis=0) - g1[0])) < 1e-14
    S0 = rng.standard_normal((H, dv, dk))
    assert np.max(np.abs(orc.scalar_compose(g, SL, S_in=S0) - (g1[0][:, None, None] * S0 + SL1[0]))) < 1e-12


def pin_error_measures(orc):
    """The relative Frobenius error and its per-block form on hand-worked
    values (the LinearKV state probe's measure, ||x - ref|| / ||ref||)."""
    import math
    # ||(3, 4) - (0, 5)|| / ||(0, 5)|| = ||(3, -1)|| / 5 = sqrt(10) / 5
    assert abs(orc.rel_fro([3.0, 4.0], [0.0, 5.0]) - math.sqrt(10) / 5) < 1e-15
    # equal norms but different vectors: not zero
    assert abs(orc.rel_fro([5.0, 0.0], [0.0, 5.0]) - math.sqrt(2)) < 1e-15
    assert orc.rel_fro([1.0, 2.0], [1.0, 2.0]) == 0.0
    # zero reference: the absolute norm of x
    assert abs(orc.rel_fro([0.0, 3.0, 4.0], [0.0, 0.0, 0.0]) - 5.0) < 1e-15
    # scale invariance in the pair
    assert abs(orc.rel_fro([6.0, 8.0], [0.0, 10.0]) - math.sqrt(10) / 5) < 1e-15
    # blocks: rows of a 2 x 2 array
    x = np.array([[3.0, 4.0], [1.0, 1.0]])
    ref = np.array([[0.0, 5.0], [1.0, 0.0]])
    e = orc.rel_fro_blocks(x, ref, 1)
    assert e.shape == (2,)
    assert abs(e[0] - math.sqrt(10) / 5) < 1e-15 and abs(e[1] - 1.0) < 1e-15
    # reducing every axis gives the whole-tensor error (one block)
    whole = orc.rel_fro_blocks(x, ref, 2)
    assert whole.shape == () and abs(float(whole) - orc.rel_fro(x, ref)) < 1e-15
    assert abs(float(whole) - math.sqrt(11) / math.sqrt(26)) < 1e-15
    # floor: a tiny reference row is measured against floor * rms(row norms)
    x2 = np.array([[0.0, 5.0], [0.0, 0.2]])
    ref2 = np.array([[0.0, 5.0], [0.0, 0.1]])
    rms = math.sqrt((25.0 + 0.01) / 2)
    e2 = orc.rel_fro_blocks(x2, ref2, 1, floor=0.1)
    assert e2[0] == 0.0 and abs(e2[1] - 0.1 / (0.1 * rms)) < 1e-12
    assert abs(orc.rel_fro_blocks(x2, ref2, 1)[1] - 1.0) < 1e-12
    # blocks over leading axes [2, 3] with a reduced trailing pair [2, 2]
    rng = _rng(99)
    big = rng.standard_normal((2, 3, 2, 2))
    noisy = big + 1e-3 * rng.standard_normal(big.shape)
    eb = orc.rel_fro_blocks(noisy, big, 2)
    assert eb.shape == (2, 3)
    for i in range(2):
        for j in range(3):
            num = math.sqrt(sum((noisy[i, j] - big[i, j]).ravel() ** 2))
            den = math.sqrt(sum(big[i, j].ravel() ** 2))
            assert abs(eb[i, j] - num / den) < 1e-12
    # zero reference block (empty sequence): absolute error
    z = orc.rel_fro_blocks(np.array([[0.0, 0.0], [3.0, 4.0]]), np.zeros((2, 2)), 1)
    assert z[0] == 0.0 and abs(z[1] - 5.0) < 1e-15


ALL_PINS = [
    pin_error_measures,
    pin_scalar_by_hand,
    pin_scalar_closed_forms,
    pin_scalar_compose_is_concatenation,
    pin_front_end_values,
    pin_front_end_invariants,
    pin_literal_matrix_form,
    pin_exact_rational,
    pin_identity_gate,
    pin_delta_write,
    pin_orthonormal_memory,
    pin_beta_zero_decay,
    pin_split_resume,
    pin_varlen_and_heads,
    pin_single_token_operator,
    pin_operator_determinant_and_kernel,
    pin_compose_equals_sequential,
    pin_tail_error_identity,
]
