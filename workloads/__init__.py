"""Seeded synthetic inputs for Gated DeltaNet replay (numpy only).

This module holds no part of the method's arithmetic: it only draws random
inputs with the shapes and value distributions of the workloads and rounds
them to the input dtype.  Both the HIP path (through the tests and the
benchmark) and the fp64 oracle receive exactly the arrays made here.

Recipe (one numpy PCG64 generator per call, seeded by the caller):
  1. varlen only: tail lengths = rng.integers(lo, hi, size=n, endpoint=True);
  2. q, k, v ~ N(0, 1) in float64 with shape [T_tot, H, d];
  3. beta-logit then alpha-logit ~ N(0, 1) with shape [T_tot, H];
  4. q and k are L2-normalised per (token, head); beta = sigmoid(x_beta);
     alpha = exp(-c * softplus(x_alpha)) with c = 0.1 by default (0.001 is
     the slow-decay stress law, 5 the strong-decay law whose in-chunk
     cumulative gates reach exp(-100) and below);
  4b. optional, drawn after everything above so that the other recipes keep
     their values: a per-(token, head) key scale s ~ U[lo, hi] (keys of
     non-unit norm: k <- s k), then a fraction of the gates set to exactly 0
     (a uniform draw per (token, head));
  5. values are rounded to float32 (round to nearest even) and, for bf16
     inputs, further to bfloat16 (round to nearest even).  The oracle is fed
     the rounded values, upcast exactly.

The tail length of a replay follows the Tail-Replay rule (section 3,
"Independent Tail-Replay"): the latest k = ceil(r * m) tokens of an m-token
matched prefix, with r a fraction such as 5% or 10%.
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from fractions import Fraction
from typing import Optional

import numpy as np


def tail_length(m: int, r) -> int:
    """ceil(r * m) computed exactly (r given as a float, str or Fraction)."""
    fr = Fraction(str(r)) if not isinstance(r, Fraction) else r
    return int(math.ceil(fr * int(m)))


def f32_round(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, np.float64).astype(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round to float32 then to bfloat16 (both round-to-nearest-even).

    Returns the uint16 bit patterns.  NaN is not expected in these inputs.
    """
    x = np.asarray(x)
    out = np.empty(x.shape, np.uint16)
    src, dst = x.reshape(-1), out.reshape(-1)
    step = 1 << 22   # elementwise, in cache-sized pieces
    for s in range(0, src.size, step):
        u = f32_round(src[s:s + step]).view(np.uint32)
        # finite inputs only: the rounding increment cannot carry out of 32 bits
        r = u >> np.uint32(16)
        r &= np.uint32(1)
        r += np.uint32(0x7FFF)
        u += r
        u >>= np.uint32(16)
        dst[s:s + step] = u
    return out


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    u = np.asarray(bits, np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


@dataclass
class Inputs:
    """One batch of replay inputs.

    ``q``, ``k``, ``v``, ``alpha``, ``beta`` are numpy arrays in the input
    dtype's storage: float32, or uint16 bf16 bit patterns when dtype == 'bf16'.
    ``f64`` gives the same values upcast exactly to float64.
    """
    dtype: str
    H: int
    dk: int
    dv: int
    cu_seqlens: np.ndarray
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    alpha: np.ndarray
    beta: np.ndarray
    _f64: Optional[dict] = None

    @property
    def f64(self) -> dict:
        """The same values upcast exactly to float64 (computed on first use)."""
        if self._f64 is None:
            conv = bf16_to_f64 if self.dtype == "bf16" else (lambda a: a.astype(np.float64))
            self._f64 = {n: conv(getattr(self, n)) for n in ("q", "k", "v", "alpha", "beta")}
        return self._f64

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])

    @property
    def n_seqs(self) -> int:
        return int(self.cu_seqlens.shape[0] - 1)

    @property
    def lengths(self) -> np.ndarray:
        return np.diff(self.cu_seqlens)


def _softplus(x):
    return np.logaddexp(0.0, x)


def _unit_rows(x):
    """x / ||x|| along the last axis, in pieces along the first (same values)."""
    out = np.empty_like(x)
    step = max(1, (1 << 22) // max(1, x[0].size)) if x.shape[0] else 1
    for s in range(0, x.shape[0], step):
        xs = x[s:s + step]
        np.divide(xs, np.linalg.norm(xs, axis=-1, keepdims=True), out=out[s:s + step])
    return out


def generate(lengths, H: int, dk: int, dv: int, dtype: str = "bf16",
             seed: int = 0, gate_scale: float = 0.1, rng=None,
             alpha_one: bool = False, beta_value: Optional[float] = None,
             key_scale: Optional[tuple] = None, alpha_zero_frac: float = 0.0) -> Inputs:
    """Draw one packed batch with the recipe in the module docstring.

    ``lengths``: per-sequence token counts (any may be 0).
    ``gate_scale``: c in alpha = exp(-c * softplus(x)); 0.1 is the workload law,
    0.001 the slow-decay stress law, 5 the strong-decay law.  ``alpha_one``
    forces alpha = 1 and ``beta_value`` forces a constant beta (stress /
    invariant cases).  ``key_scale`` = (lo, hi) scales each normalised key by
    U[lo, hi]; ``alpha_zero_frac`` sets that fraction of the gates to 0.
    """
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    rng = np.random.Generator(np.random.PCG64(seed)) if rng is None else rng
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(lengths.shape[0] + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    v = rng.standard_normal((T, H, dv))
    xb = rng.standard_normal((T, H))
    xa = rng.standard_normal((T, H))
    q, k = _unit_rows(q), _unit_rows(k)
    beta = 1.0 / (1.0 + np.exp(-xb)) if beta_value is None else np.full((T, H), beta_value)
    alpha = np.ones((T, H)) if alpha_one else np.exp(-gate_scale * _softplus(xa))
    if key_scale is not None:
        k = k * rng.uniform(key_scale[0], key_scale[1], (T, H, 1))
    if alpha_zero_frac > 0:
        alpha = np.where(rng.uniform(0.0, 1.0, (T, H)) < alpha_zero_frac, 0.0, alpha)
    arrs = dict(q=q, k=k, v=v, alpha=alpha, beta=beta)
    rnd = bf16_bits if dtype == "bf16" else f32_round
    store = {name: rnd(a) for name, a in arrs.items()}
    return Inputs(dtype=dtype, H=H, dk=dk, dv=dv, cu_seqlens=cu, **store)


@dataclass
class RawInputs:
    """Projections before the front end: ``q_raw``, ``k_raw`` [T, H, dk] and
    ``v`` [T, H, dv] ~ N(0, 1) with a per-(token, head) scale U[0.25, 4] on q
    and k; the log-gate ``g`` = -c * softplus(x_alpha) and the beta logit
    ``b`` = x_beta [T, H] (the recipe's steps 1-3 and 5, without step 4's
    normalisation and activations).  Storage as in Inputs."""
    dtype: str
    H: int
    dk: int
    dv: int
    cu_seqlens: np.ndarray
    q_raw: np.ndarray
    k_raw: np.ndarray
    v: np.ndarray
    g: np.ndarray
    b: np.ndarray

    def f64(self, name: str) -> np.ndarray:
        a = getattr(self, name)
        return bf16_to_f64(a) if self.dtype == "bf16" else a.astype(np.float64)

    @property
    def n_tokens(self) -> int:
        return int(self.cu_seqlens[-1])


def generate_raw(lengths, H: int, dk: int, dv: int, dtype: str = "bf16", seed: int = 0,
                 gate_scale: float = 0.1) -> RawInputs:
    """Draw one packed batch of raw projections (see RawInputs)."""
    if dtype not in ("f32", "bf16"):
        raise ValueError("dtype must be 'f32' or 'bf16'")
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = np.asarray(lengths, np.int64)
    cu = np.zeros(lengths.shape[0] + 1, np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q = rng.standard_normal((T, H, dk)) * rng.uniform(0.25, 4.0, (T, H, 1))
    k = rng.standard_normal((T, H, dk)) * rng.uniform(0.25, 4.0, (T, H, 1))
    v = rng.standard_normal((T, H, dv))
    xb = rng.standard_normal((T, H))
    xa = rng.standard_normal((T, H))
    arrs = dict(q_raw=q, k_raw=k, v=v, g=-gate_scale * _softplus(xa), b=xb)
    rnd = bf16_bits if dtype == "bf16" else f32_round
    return RawInputs(dtype=dtype, H=H, dk=dk, dv=dv, cu_seqlens=cu, **{n: rnd(a) for n, a in arrs.items()})


# ---------------------------------------------------------------------------
# The five workloads.  Shapes follow the pages: a 32768-token prefix with a
# 10% tail (ceil(0.1 * 32768) = 3277), tails of 5-10% of 8K-32K prefixes
# (bounds ceil(0.05 * 8192) = 410 and 3277), a full 32K prefill, and 64
# fixed contiguous 512-token chunks (the LinearKV chunking).
# ---------------------------------------------------------------------------

WORKLOADS = {
    0: dict(name="single-head-T256-d64-f32", H=1, d=64, dtype="f32", lengths=[256]),
    1: dict(name="tail-replay-T3277-H32-d128-bf16", H=32, d=128, dtype="bf16",
            lengths=[tail_length(32768, "0.1")], state_only=True),
    2: dict(name="varlen-16x[410,3277]-H32-d128-bf16", H=32, d=128, dtype="bf16",
            n_varlen=16, lo=tail_length(8192, "0.05"), hi=tail_length(32768, "0.1")),
    3: dict(name="full-prefill-T32768-H32-d128-bf16", H=32, d=128, dtype="bf16",
            lengths=[32768]),
    4: dict(name="chunk-ops-64x512-H32-d128-bf16", H=32, d=128, dtype="bf16",
            lengths=[64 * 512], chunk=512),
}


def workload_lengths(cfg_id: int, rng) -> list:
    w = WORKLOADS[cfg_id]
    if "n_varlen" in w:
        return [int(x) for x in rng.integers(w["lo"], w["hi"], size=w["n_varlen"],
                                             endpoint=True)]
    return list(w["lengths"])


def make_workload(cfg_id: int, seed: Optional[int] = None, H: Optional[int] = None) -> Inputs:
    """Inputs of workload ``cfg_id`` (seed defaults to the workload index).

    ``H`` may reduce the head count (heads are independent and identically
    distributed, so fewer heads is a sample of the same workload).
    """
    w = WORKLOADS[cfg_id]
    seed = cfg_id if seed is None else seed
    rng = np.random.Generator(np.random.PCG64(seed))
    lengths = workload_lengths(cfg_id, rng)
    return generate(lengths, H=w["H"] if H is None else H, dk=w["d"], dv=w["d"],
                    dtype=w["dtype"], rng=rng)


# Tail-error curve: the latest k tokens of the 32768-token prefill inputs
# replayed from zero, k = 8 .. 256 tokens and ceil(r * 32768) for r = 1.25%,
# 2.5%, 5% and 10%, under the workload gate law and, as a supplement, the
# slow law (gate_scale 0.001).
TAIL_CURVE_M = 32768
TAIL_CURVE_KS = [8, 16, 32, 64, 128, 256] + [tail_length(32768, r) for r in ("0.0125", "0.025", "0.05", "0.1")]
TAIL_CURVE_LAWS = {"workload": 0.1, "slow": 0.001}


def tail_curve_inputs(law: str) -> Inputs:
    """The prefix of the tail-error curve: workload 3's draw (seed 3, H = 32,
    d = 128, bf16) with the named gate law."""
    return generate([TAIL_CURVE_M], H=32, dk=128, dv=128, dtype="bf16", seed=3,
                    gate_scale=TAIL_CURVE_LAWS[law])


def chunk_bounds(n_tokens: int, chunk: int) -> np.ndarray:
    """cu_chunks for fixed contiguous chunks of ``chunk`` tokens (last may be short)."""
    starts = list(range(0, n_tokens, chunk)) + [n_tokens]
    return np.asarray(starts, np.int32)
