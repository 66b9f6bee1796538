"""GPU parity of time-split replay (bf16 inputs, final state only).

A sequence cut into P segments of whole 64-token chunks runs as P
independent recurrences: segment 0 from S0, later segments as affine
operators (T_seg, S_seg) of the page "LinearKV: One Cached State Suffices
for Position-Independent Caching in Hybrid LLMs" (affine chunk operator and
composition paragraphs), composed back to back.  The composed state is the
state of the plain sequential replay (page "Tail-Replay: Escaping the Curse
of Linear Attention in Prefix Caching for Hybrid LLMs", section 2 Eq. (1)),
so every case is checked against the fp64 oracle at the bf16 tolerance.
``GDN_REPLAY_SEGMENTS`` forces P.
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


def state_only(inp, S0=None):
    gdn, torch = _gdn()
    d = dev(inp)
    S0_t = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    _, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=S0_t, want_o=False)
    torch.cuda.synchronize()
    return to_np(S)


def start_state(n, H, dv, dk, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((n, H, dv, dk)) * 0.1).astype(np.float32).astype(np.float64)


def check(inp, S0=None, tol=TOL_BF16):
    S = state_only(inp, S0=S0)
    _, S_ref = oracle_replay(inp, S0=S0, want_o=False)
    e = rel(S, S_ref)
    print("P-split err_S %.3e (tol %.1e)" % (e, tol), flush=True)
    assert e <= tol
    return S


@pytest.mark.parametrize("P", [2, 3, 5])
def test_split_ragged_with_and_without_start_state(P, monkeypatch):
    # partial chunks, exact multiples, empty sequences and segments past the end
    monkeypatch.setenv("GDN_REPLAY_SEGMENTS", str(P))
    lengths = [1, 63, 64, 65, 0, 200, 330]
    inp = workloads.generate(lengths, H=3, dk=128, dv=128, dtype="bf16", seed=41)
    check(inp)
    check(inp, S0=start_state(len(lengths), 3, 128, 128, 42))


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_split_shapes(dk, dv, monkeypatch):
    monkeypatch.setenv("GDN_REPLAY_SEGMENTS", "4")
    inp = workloads.generate([500, 77], H=2, dk=dk, dv=dv, dtype="bf16", seed=43)
    check(inp, S0=start_state(2, 2, dv, dk, 44))


@pytest.mark.parametrize("law", ["workload", "slow", "alpha1"])
def test_split_long_tail_gate_laws(law, monkeypatch):
    # one 3277-token tail (10% of 32K) on 4 heads; with alpha = 1 the segment
    # transitions stay far from zero, so the composition carries real weight
    kw = {"workload": {}, "slow": dict(gate_scale=0.001), "alpha1": dict(alpha_one=True)}[law]
    inp = workloads.generate([3277], H=4, dk=128, dv=128, dtype="bf16", seed=45, **kw)
    monkeypatch.setenv("GDN_REPLAY_SEGMENTS", "1")
    S1 = check(inp)
    for P in (2, 4):
        monkeypatch.setenv("GDN_REPLAY_SEGMENTS", str(P))
        SP = check(inp)
        assert rel(SP, S1) <= TOL_BF16


def test_default_choice_splits_a_single_long_tail(monkeypatch):
    # without the override a single 3277-token sequence on 32 heads is split
    monkeypatch.delenv("GDN_REPLAY_SEGMENTS", raising=False)
    gdn, torch = _gdn()
    lib = gdn.library()
    tau = (3277 // 64 + 2) * 32 * 13312
    assert lib.gdn_replay_workspace_bytes(1, 3277, 32, 128, 128) > tau
    inp = workloads.generate([3277], H=32, dk=128, dv=128, dtype="bf16", seed=46)
    S = state_only(inp)
    heads = [0, 13, 31]
    _, S_ref = oracle_replay(inp, want_o=False, heads=heads)
    e = rel(S[:, heads], S_ref)
    print("default split err_S %.3e" % e, flush=True)
    assert e <= TOL_BF16


# ---- time split with outputs: segment operators, their composition (which
# also gives every segment's start state), then each segment again with
# outputs from that start state ----

def with_outputs(inp, S0=None):
    gdn, torch = _gdn()
    d = dev(inp)
    S0_t = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    o, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=S0_t, want_o=True)
    torch.cuda.synchronize()
    return to_np(o), to_np(S)


def check_o(inp, S0=None, tol=TOL_BF16):
    o, S = with_outputs(inp, S0=S0)
    o_ref, S_ref = oracle_replay(inp, S0=S0, want_o=True)
    eo, eS = rel(o, o_ref), rel(S, S_ref)
    print("P-split with outputs err_o %.3e err_S %.3e (tol %.1e)" % (eo, eS, tol), flush=True)
    assert eo <= tol and eS <= tol
    return o, S


@pytest.mark.parametrize("P", [2, 3, 5])
def test_split_with_outputs_ragged(P, monkeypatch):
    monkeypatch.setenv("GDN_REPLAY_SEGMENTS", str(P))
    lengths = [1, 63, 64, 65, 0, 200, 330]
    inp = workloads.generate(lengths, H=3, dk=128, dv=128, dtype="bf16", seed=51)
    check_o(inp)
    check_o(inp, S0=start_state(len(lengths), 3, 128, 128, 52))


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_split_with_outputs_shapes(dk, dv, monkeypatch):
    monkeypatch.setenv("GDN_REPLAY_SEGMENTS", "4")
    inp = workloads.generate([500, 77], H=2, dk=dk, dv=dv, dtype="bf16", seed=53)
    check_o(inp, S0=start_state(2, 2, dv, dk, 54))


def test_split_with_outputs_alpha_one_matches_unsplit(monkeypatch):
    # alpha = 1: every segment's start state carries real weight
    inp = workloads.generate([1500], H=4, dk=128, dv=128, dtype="bf16", seed=55, alpha_one=True)
    monkeypatch.setenv("GDN_REPLAY_SEGMENTS", "1")
    o1, S1 = check_o(inp)
    monkeypatch.setenv("GDN_REPLAY_SEGMENTS", "6")
    o6, S6 = check_o(inp)
    assert rel(o6, o1) <= TOL_BF16 and rel(S6, S1) <= TOL_BF16


def test_split_with_outputs_start_state_aliases_final(monkeypatch):
    # S_final may alias S0: the start state of segment 0 is read before the
    # composed final state is written
    monkeypatch.setenv("GDN_REPLAY_SEGMENTS", "3")
    gdn, torch = _gdn()
    inp = workloads.generate([400], H=2, dk=128, dv=128, dtype="bf16", seed=57)
    S0 = start_state(1, 2, 128, 128, 58)
    d = dev(inp)
    buf = torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    o, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=buf, want_o=True, S_out=buf)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_replay(inp, S0=S0, want_o=True)
    assert rel(to_np(o), o_ref) <= TOL_BF16 and rel(to_np(buf), S_ref) <= TOL_BF16
