"""Host-side logic of the synthetic workloads (CPU only)."""
import json
import os

import numpy as np

import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_replay_budget_golden():
    with open(os.path.join(GOLDEN, "replay_budget.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        assert workloads.tail_length(c["m"], c["r"]) == c["k"], c


def test_bf16_rounding_is_rne():
    x = np.array([1.0, 1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, 1.0 + 2 ** -9, -2.5, 0.0])
    got = workloads.bf16_to_f64(workloads.bf16_bits(x))
    # ties go to even: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    assert list(got) == [1.0, 1.0, 1.0 + 2 ** -6, 1.0, -2.5, 0.0]


def test_workload_shapes_and_distributions():
    w2 = workloads.make_workload(2, H=2)
    lens = w2.lengths
    assert lens.shape == (16,) and lens.min() >= 410 and lens.max() <= 3277
    assert w2.q.dtype == np.uint16 and w2.q.shape == (w2.n_tokens, 2, 128)
    kn = np.linalg.norm(w2.f64["k"], axis=-1)
    assert np.all(np.abs(kn - 1) < 2e-2)
    a = w2.f64["alpha"]
    assert np.all((a > 0) & (a <= 1))
    b = w2.f64["beta"]
    assert np.all((b > 0) & (b < 1))
    w0 = workloads.make_workload(0)
    assert w0.q.dtype == np.float32 and w0.n_tokens == 256 and w0.dk == 64
    # same seed, same data
    w0b = workloads.make_workload(0)
    assert np.array_equal(w0.k, w0b.k)
    w1 = workloads.make_workload(1, H=1)
    assert w1.n_tokens == 3277


def test_raw_inputs_recipe():
    # raw projections: seeded, rounded to the dtype, log-gate <= 0, q and k
    # not normalised (per-row scales in [0.25, 4])
    a = workloads.generate_raw([5, 0, 70], H=3, dk=64, dv=128, dtype="bf16", seed=9)
    b = workloads.generate_raw([5, 0, 70], H=3, dk=64, dv=128, dtype="bf16", seed=9)
    assert a.q_raw.shape == (75, 3, 64) and a.v.shape == (75, 3, 128) and a.g.shape == (75, 3)
    assert a.q_raw.dtype == np.uint16 and np.array_equal(a.k_raw, b.k_raw) and a.n_tokens == 75
    assert np.all(a.f64("g") <= 0)
    n = np.linalg.norm(a.f64("k_raw"), axis=-1)
    assert n.min() > 0.25 * 4 and n.max() < 4 * 16 and np.std(n) > 1
    f = workloads.generate_raw([8], H=1, dk=64, dv=64, dtype="f32", seed=9)
    assert f.q_raw.dtype == np.float32
