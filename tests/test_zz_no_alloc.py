"""gdn_replay_noalloc (the replay with the library's built-in scratch, for
callers that cannot allocate) against gdn_replay on the same inputs: the
same kernels, so the results must be equal bit for bit, and both within the
bars of tests/gpu_helpers.py against the fp64 oracle.  Two calls in a row,
the second smaller (the scratch keeps the first call's contents), then a
third on a time-split shape again; a replay that needs more scratch than
the array holds is rejected before anything runs."""
import numpy as np
import pytest

import workloads
from tests.gpu_helpers import check_out, check_state, dev, oracle_replay, to_np

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def both(inp, want_o, S0=None):
    gdn, torch = _gdn()
    d = dev(inp)
    S0_t = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    o1, S1 = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=S0_t, want_o=want_o)
    o2, S2 = gdn.replay_noalloc(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=S0_t, want_o=want_o)
    torch.cuda.synchronize()
    assert torch.equal(S1, S2)
    if want_o:
        assert torch.equal(o1, o2)
    return (to_np(o2) if want_o else None), to_np(S2)


def test_noalloc_matches_replay_two_calls_then_split_again():
    # 1: the 3277-token tail over 32 heads, state only (a time split: records,
    #    segment operators and states in the scratch, ~56 MB of 64 MiB)
    big = workloads.generate([3277], H=32, dk=128, dv=128, dtype="bf16", seed=141)
    _, S = both(big, want_o=False)
    heads = [0, 7, 19, 31]
    _, S_ref = oracle_replay(big, want_o=False, heads=heads)
    check_state("noalloc tail S heads %s" % heads, S[:, heads], S_ref, "bf16")
    # 2: smaller, packed with outputs and a start state (records and the
    #    longest-first order in the scratch, over the first call's contents)
    small = workloads.generate([300, 0, 77, 129], H=4, dk=128, dv=64, dtype="bf16", seed=142)
    S0 = (np.random.Generator(np.random.PCG64(143)).standard_normal((4, 4, 64, 128)) * 0.2).astype(np.float32)
    o, S = both(small, want_o=True, S0=S0)
    o_ref, S_ref = oracle_replay(small, S0=S0.astype(np.float64))
    check_out("noalloc small o", o, o_ref, "bf16")
    check_state("noalloc small S", S, S_ref, "bf16")
    # 3: fp32 inputs, then a split with outputs (segment start states too)
    f32 = workloads.generate([200, 65], H=2, dk=64, dv=64, dtype="f32", seed=144)
    o, S = both(f32, want_o=True)
    o_ref, S_ref = oracle_replay(f32)
    check_out("noalloc f32 o", o, o_ref, "f32")
    check_state("noalloc f32 S", S, S_ref, "f32")
    split = workloads.generate([4096], H=8, dk=128, dv=128, dtype="bf16", seed=145, gate_scale=0.001)
    o, S = both(split, want_o=True)
    o_ref, S_ref = oracle_replay(split, heads=[0, 5])
    check_out("noalloc split o", o[:, [0, 5]], o_ref, "bf16")
    check_state("noalloc split S", S[:, [0, 5]], S_ref, "bf16")


def test_noalloc_rejects_a_replay_beyond_its_scratch():
    gdn, torch = _gdn()
    # 32768 tokens x 32 heads: ~220 MB of records alone
    T, H = 32768, 32
    k = torch.zeros((T, H, 128), dtype=torch.bfloat16, device="cuda")
    a = torch.ones((T, H), dtype=torch.bfloat16, device="cuda")
    cu = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    with pytest.raises(gdn.GdnError) as e:
        gdn.replay_noalloc(None, k, k, a, a, cu, want_o=False)
    assert e.value.name == "GDN_ERR_WORKSPACE" and "scratch" in e.value.detail
