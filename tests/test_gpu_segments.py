"""GPU parity of time-split replay (bf16 inputs).

A sequence cut into P segments of whole 64-token chunks runs as P
independent recurrences: segment 0 from S0, later segments as affine
operators (T_seg, S_seg) of the page "LinearKV: One Cached State Suffices
for Position-Independent Caching in Hybrid LLMs" (affine chunk operator and
composition paragraphs), composed back to back.  The composed state is the
state of the plain sequential replay (page "Tail-Replay: Escaping the Curse
of Linear Attention in Prefix Caching for Hybrid LLMs", section 2 Eq. (1)),
so every case is checked against the fp64 oracle with the bars of
tests/gpu_helpers.py.  gdn_replay_segmented (the binding's ``segments=``)
forces P.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_helpers import (TOL_BF16, check_out, check_replay, check_state, dev, oracle_replay, rel,
                               run_replay, to_np)

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def start_state(n, H, dv, dk, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((n, H, dv, dk)) * 0.1).astype(np.float32).astype(np.float64)


def check(inp, S0=None, P=None):
    _, S = check_replay("P=%s state only" % P, inp, S0=S0, want_o=False, segments=P)
    return S


@pytest.mark.parametrize("P", [2, 3, 5])
def test_split_ragged_with_and_without_start_state(P):
    # partial chunks, exact multiples, empty sequences and segments past the end
    lengths = [1, 63, 64, 65, 0, 200, 330]
    inp = workloads.generate(lengths, H=3, dk=128, dv=128, dtype="bf16", seed=41)
    check(inp, P=P)
    check(inp, S0=start_state(len(lengths), 3, 128, 128, 42), P=P)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_split_shapes(dk, dv):
    inp = workloads.generate([500, 77], H=2, dk=dk, dv=dv, dtype="bf16", seed=43)
    check(inp, S0=start_state(2, 2, dv, dk, 44), P=4)


@pytest.mark.parametrize("law", ["workload", "slow", "alpha1", "strong"])
def test_split_long_tail_gate_laws(law):
    # one 3277-token tail (10% of 32K) on 4 heads; with alpha = 1 the segment
    # transitions stay far from zero, so the composition carries real weight
    kw = {"workload": {}, "slow": dict(gate_scale=0.001), "alpha1": dict(alpha_one=True),
          "strong": dict(gate_scale=5.0)}[law]
    inp = workloads.generate([3277], H=4, dk=128, dv=128, dtype="bf16", seed=45, **kw)
    S1 = check(inp, P=1)
    for P in (2, 4):
        SP = check(inp, P=P)
        assert rel(SP, S1) <= TOL_BF16


def test_default_choice_splits_a_single_long_tail():
    # without a forced count a single 3277-token sequence on 32 heads is split
    gdn, torch = _gdn()
    lib = gdn.library()
    tau = (3277 // 64 + 2) * 32 * 12288
    assert lib.gdn_replay_workspace_bytes(1, 3277, 32, 128, 128) > tau
    inp = workloads.generate([3277], H=32, dk=128, dv=128, dtype="bf16", seed=46)
    _, S = run_replay(inp, want_o=False)
    heads = [0, 5, 13, 21, 31]
    _, S_ref = oracle_replay(inp, want_o=False, heads=heads)
    check_state("default split heads %s" % heads, S[:, heads], S_ref, "bf16")


# ---- time split with outputs: segment operators, their composition (which
# also gives every segment's start state), then each segment again with
# outputs from that start state ----

def check_o(inp, S0=None, P=None):
    return check_replay("P=%s with outputs" % P, inp, S0=S0, segments=P)


@pytest.mark.parametrize("P", [2, 3, 5])
def test_split_with_outputs_ragged(P):
    lengths = [1, 63, 64, 65, 0, 200, 330]
    inp = workloads.generate(lengths, H=3, dk=128, dv=128, dtype="bf16", seed=51)
    check_o(inp, P=P)
    check_o(inp, S0=start_state(len(lengths), 3, 128, 128, 52), P=P)


@pytest.mark.parametrize("dk,dv", [(64, 64), (64, 128), (128, 64)])
def test_split_with_outputs_shapes(dk, dv):
    inp = workloads.generate([500, 77], H=2, dk=dk, dv=dv, dtype="bf16", seed=53)
    check_o(inp, S0=start_state(2, 2, dv, dk, 54), P=4)


@pytest.mark.parametrize("law", ["workload", "strong"])
def test_split_with_outputs_lead_layout_many_segments(law):
    # the layout of a long split with outputs: a lead segment that runs
    # with its outputs beside the transition segments (which also build the
    # last segment's records), then every later segment with outputs; nine
    # segments as the cost model picks for one sequence over 32 heads, here
    # on sequences of different lengths (one of them shorter than the
    # segment count in chunks, one empty) with a start state
    kw = dict(gate_scale=5.0) if law == "strong" else {}
    lengths = [2000, 1500, 0, 300, 640]
    inp = workloads.generate(lengths, H=2, dk=128, dv=128, dtype="bf16", seed=60, **kw)
    check_o(inp, S0=start_state(len(lengths), 2, 128, 128, 61), P=9)


def test_split_with_outputs_alpha_one_matches_unsplit():
    # alpha = 1: every segment's start state carries real weight
    inp = workloads.generate([1500], H=4, dk=128, dv=128, dtype="bf16", seed=55, alpha_one=True)
    o1, S1 = check_o(inp, P=1)
    o6, S6 = check_o(inp, P=6)
    assert rel(o6, o1) <= TOL_BF16 and rel(S6, S1) <= TOL_BF16


def test_split_with_outputs_start_state_aliases_final():
    # S_final may alias S0: the start state of segment 0 is read before the
    # composed final state is written
    gdn, torch = _gdn()
    inp = workloads.generate([400], H=2, dk=128, dv=128, dtype="bf16", seed=57)
    S0 = start_state(1, 2, 128, 128, 58)
    d = dev(inp)
    buf = torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    o, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=buf, want_o=True, S_out=buf,
                      segments=3)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_replay(inp, S0=S0, want_o=True)
    check_out("aliased o", to_np(o), o_ref, "bf16")
    check_state("aliased S", to_np(buf), S_ref, "bf16")


def test_segment_count_is_checked():
    gdn, torch = _gdn()
    inp = workloads.generate([100], H=1, dk=64, dv=64, dtype="bf16", seed=59)
    d = dev(inp)
    for bad in (-1, 65):
        with pytest.raises(gdn.GdnError) as e:
            gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], segments=bad)
        assert e.value.name == "GDN_ERR_BAD_SHAPE"
    # the cost model (0) and the largest count (64, mostly empty segments)
    check_replay("P=0", inp, segments=0)
    check_replay("P=64", inp, segments=64)
