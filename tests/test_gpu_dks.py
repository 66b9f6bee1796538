"""GPU parity of the state-only replay whose waves split the key dimension
(bf16 inputs, at most 256 row tiles in all; selected by
``GDN_REPLAY_KEYSPLIT=1``).

Every case is checked against the fp64 oracle (page "Tail-Replay: Escaping
the Curse of Linear Attention in Prefix Caching for Hybrid LLMs", section 2
Eq. (1)) at the bf16 tolerance, and the state must not depend on the path:
the time split (``GDN_REPLAY_SEGMENTS``) gives the same state within that
tolerance.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_helpers import TOL_BF16, dev, oracle_replay, rel, to_np

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def state_only(inp, S0=None, S_out_alias=False):
    gdn, torch = _gdn()
    d = dev(inp)
    S0_t = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    kw = dict(S_out=S0_t) if S_out_alias else {}
    _, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=S0_t, want_o=False, **kw)
    torch.cuda.synchronize()
    return to_np(S)


def start_state(n, H, dv, dk, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((n, H, dv, dk)) * 0.1).astype(np.float32).astype(np.float64)


def check(inp, S0=None, tol=TOL_BF16, heads=None):
    S = state_only(inp, S0=S0)
    _, S_ref = oracle_replay(inp, S0=S0, want_o=False, heads=heads)
    if heads is not None:
        S = S[:, heads]
    e = rel(S, S_ref)
    print("key-split err_S %.3e (tol %.1e)" % (e, tol), flush=True)
    assert e <= tol
    return S


@pytest.fixture(autouse=True)
def _key_split(monkeypatch):
    monkeypatch.delenv("GDN_REPLAY_SEGMENTS", raising=False)
    monkeypatch.setenv("GDN_REPLAY_KEYSPLIT", "1")


def test_ragged_with_and_without_start_state():
    # partial chunks, exact multiples, an empty sequence; 7 x 3 x 8 = 168 row tiles
    lengths = [1, 63, 64, 65, 0, 200, 330]
    inp = workloads.generate(lengths, H=3, dk=128, dv=128, dtype="bf16", seed=61)
    check(inp)
    check(inp, S0=start_state(len(lengths), 3, 128, 128, 62))


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_shapes(dk, dv):
    inp = workloads.generate([500, 77], H=2, dk=dk, dv=dv, dtype="bf16", seed=63)
    check(inp, S0=start_state(2, 2, dv, dk, 64))


@pytest.mark.parametrize("law", ["workload", "slow", "alpha1"])
def test_long_tail_gate_laws_match_time_split(law, monkeypatch):
    kw = {"workload": {}, "slow": dict(gate_scale=0.001), "alpha1": dict(alpha_one=True)}[law]
    inp = workloads.generate([3277], H=4, dk=128, dv=128, dtype="bf16", seed=65, **kw)
    S = check(inp)
    monkeypatch.delenv("GDN_REPLAY_KEYSPLIT")
    monkeypatch.setenv("GDN_REPLAY_SEGMENTS", "4")
    S4 = state_only(inp)
    assert rel(S4, S) <= TOL_BF16


def test_tail_replay_shape():
    # one 3277-token tail on 32 heads (256 row tiles): checked on sampled heads
    inp = workloads.generate([3277], H=32, dk=128, dv=128, dtype="bf16", seed=66)
    check(inp, heads=[0, 17, 31])


def test_final_state_may_alias_start_state():
    gdn, torch = _gdn()
    inp = workloads.generate([700, 129], H=2, dk=128, dv=128, dtype="bf16", seed=67)
    S0 = start_state(2, 2, 128, 128, 68)
    d = dev(inp)
    buf = torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=buf, want_o=False, S_out=buf)
    torch.cuda.synchronize()
    _, S_ref = oracle_replay(inp, S0=S0, want_o=False)
    assert rel(to_np(buf), S_ref) <= TOL_BF16


def test_repeat_calls_are_bitwise_identical():
    gdn, torch = _gdn()
    inp = workloads.generate([1000], H=8, dk=128, dv=128, dtype="bf16", seed=69)
    d = dev(inp)
    outs = []
    for _ in range(3):
        _, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], want_o=False)
        torch.cuda.synchronize()
        outs.append(S.cpu().numpy())
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
