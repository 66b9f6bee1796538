"""Tail-replay state error as a function of the replayed fraction.

Pages: "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching
for Hybrid LLMs", section 3 (Independent Tail-Replay: the state at the end of
an m-token prefix is rebuilt from the latest k tokens, starting from zero);
"LinearKV: One Cached State Suffices for Position-Independent Caching in
Hybrid LLMs", the relative error of a constructed state against the
full-prefix state (Figure 3 discussion).

tests/golden/tail_curve.json holds the fp64 oracle's curve on the
32768-token, 32-head prefill inputs, written by tests/golden/make_tail_curve.py.
The CPU tests pin the script's arithmetic on a small case to the exact
identity S_full - S_tail = S_head T_tail (the tail as one affine chunk
operator) and check the stored curve against its bound; the GPU tests
rebuild the curve with gdn_replay and compare it with the stored one.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "tail_curve.json")


def _make():
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_tail_curve", os.path.join(HERE, "golden", "make_tail_curve.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def _stored():
    with open(GOLDEN) as fh:
        return json.load(fh)


def test_curve_arithmetic_matches_the_operator_identity():
    mk = _make()
    ks = [1, 8, 64, 65, 200]
    for scale in (0.1, 0.001):
        inp = workloads.generate([640], H=3, dk=16, dv=8, dtype="bf16", seed=71, gate_scale=scale)
        got = mk.curve(inp, ks)
        f = inp.f64
        m = 640
        _, S_full = oracle.replay(None, f["k"], f["v"], f["alpha"], f["beta"], [0, m], want_o=False)
        for i, kk in enumerate(ks):
            # S_full - S_tail = S_head T_tail, T_tail the tail's chunk operator
            _, S_head = oracle.replay(None, f["k"][:m - kk], f["v"][:m - kk], f["alpha"][:m - kk],
                                      f["beta"][:m - kk], [0, m - kk], want_o=False)
            T_tail, _ = oracle.chunk_operator(f["k"][m - kk:], f["alpha"][m - kk:], f["beta"][m - kk:], [0, kk])
            diff = np.einsum("hij,hjk->hik", S_head[0], T_tail[0])
            err = np.linalg.norm(diff) / np.linalg.norm(S_full)
            assert abs(got["err"][i] - err) <= 1e-10 * max(err, 1e-300) + 1e-15
            assert got["err"][i] <= got["bound"][i] * (1 + 1e-12) + 1e-300
            for h in range(3):
                eh = np.linalg.norm(diff[h]) / np.linalg.norm(S_full[0, h])
                assert abs(got["err_per_head"][i][h] - eh) <= 1e-10 * max(eh, 1e-300) + 1e-15


def test_stored_curve_is_bounded_and_saturates():
    st = _stored()
    assert st["m"] == workloads.TAIL_CURVE_M and st["k"] == workloads.TAIL_CURVE_KS
    assert st["k"][-1] == workloads.tail_length(32768, "0.1")
    for law, r in st["laws"].items():
        err, bound = np.array(r["err"]), np.array(r["bound"])
        assert np.all(err <= bound * (1 + 1e-9) + 1e-15), law
        assert np.all(np.diff(err) <= 1e-15), law          # longer tails never do worse here
        assert err[0] > 0.5, law                           # 8 tokens rebuild little of the state
    wl = st["laws"]["workload"]["err"]
    assert wl[-1] < 1e-15 and wl[-2] < 1e-15               # 5% and 10%: exact up to rounding
    assert st["laws"]["slow"]["err"][-1] > 1e-6            # slow gates still remember the head


@pytest.mark.gpu
@pytest.mark.parametrize("law", ["workload", "slow"])
def test_gpu_tail_curve_matches_oracle(law):
    import torch
    import bench
    import gated_deltanet_state_amd as gdn
    from tests.gpu_helpers import BLOCK_TOL
    ref = _stored()["laws"][law]["err"]
    got = bench.tail_curve_gpu(law, gdn, torch, np)
    print(law, " ".join("%.2e/%.2e" % (g, r) for g, r in zip(got, ref)), flush=True)
    for g, r in zip(got, ref):
        # A curve point compares two GPU states, each within its element bar
        # (1e-4 relative per (sequence, head); measured ~5e-6) of the oracle's
        # state, so it moves by at most about the sum of the two errors,
        # scaled by (1 + r) since ||S_tail|| <= (1 + r) ||S_full||.  Points
        # well above that rounding level are also held to 1e-3 of their value.
        assert abs(g - r) <= 2 * BLOCK_TOL["bf16"] * (1 + r), (g, r)
        if r > 1e-2:
            assert abs(g - r) <= 1e-3 * r, (g, r)
