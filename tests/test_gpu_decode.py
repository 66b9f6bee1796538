"""GPU parity of gdn_decode (one token per sequence from given states).

The oracle is the fp64 sequential replay (page "Tail-Replay: Escaping the
Curse of Linear Attention in Prefix Caching for Hybrid LLMs", section 2
Eq. (1)) over one-token sequences from the same start states.  The kernel
works in fp32 on exact inputs, so the bar is the fp32 tolerance (relative
Frobenius error <= 1e-5) for both input dtypes.
"""
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


def states(N, H, dv, dk, seed):
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal((N, H, dv, dk)) * 0.3).astype(np.float32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_decode_matches_oracle(dtype, dk, dv):
    gdn, torch = _gdn()
    N, H = 5, 3
    inp = workloads.generate([1] * N, H=H, dk=dk, dv=dv, dtype=dtype, seed=101)
    S_in = states(N, H, dv, dk, 102)
    d = dev(inp)
    o, S = gdn.decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S_in=torch.from_numpy(S_in).cuda())
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_replay(inp, S0=S_in.astype(np.float64))
    check_out("decode %s %dx%d o" % (dtype, dv, dk), to_np(o), o_ref, "f32")
    check_state("decode %s %dx%d S" % (dtype, dv, dk), to_np(S), S_ref, "f32")


def test_decode_zero_state_in_place_state_only_and_bf16_output():
    gdn, torch = _gdn()
    N, H = 7, 4
    inp = workloads.generate([1] * N, H=H, dk=128, dv=128, dtype="bf16", seed=103)
    d = dev(inp)
    # zero start state
    o, S = gdn.decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_replay(inp)
    check_out("decode zero state o", to_np(o), o_ref, "f32")
    check_state("decode zero state S", to_np(S), S_ref, "f32")
    # in place, state only
    S_in = states(N, H, 128, 128, 104)
    buf = torch.from_numpy(S_in).cuda()
    o2, S2 = gdn.decode(None, d["k"], d["v"], d["alpha"], d["beta"], S_in=buf, want_o=False, S_out=buf)
    torch.cuda.synchronize()
    assert o2 is None and S2 is buf
    _, S_ref2 = oracle_replay(inp, S0=S_in.astype(np.float64), want_o=False)
    check_state("decode in place", to_np(buf), S_ref2, "f32")
    # bf16 outputs: rounding o to bf16 costs ~2e-3 of relative error
    o3, _ = gdn.decode(d["q"], d["k"], d["v"], d["alpha"], d["beta"], S_in=torch.from_numpy(S_in).cuda(),
                       o_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    o_ref3, _ = oracle_replay(inp, S0=S_in.astype(np.float64))
    assert o3.dtype == torch.bfloat16
    check_out("decode bf16 o", to_np(o3), o_ref3, "f32", o_bf16=True)


def test_replay_then_decode_equals_longer_replay():
    # serving continues after a tail replay: replay T tokens, then decode the next one
    gdn, torch = _gdn()
    H, T = 4, 700
    inp = workloads.generate([T + 1], H=H, dk=128, dv=128, dtype="bf16", seed=105)
    d = dev(inp)
    cu_T = torch.tensor([0, T], dtype=torch.int32, device="cuda")
    _, S_T = gdn.replay(d["q"][:T], d["k"][:T], d["v"][:T], d["alpha"][:T], d["beta"][:T], cu_T, want_o=False)
    o1, S1 = gdn.decode(d["q"][T:], d["k"][T:], d["v"][T:], d["alpha"][T:], d["beta"][T:], S_in=S_T)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_replay(inp)
    check_state("replay then decode S", to_np(S1), S_ref, "bf16")
    check_out("replay then decode o", to_np(o1), o_ref[T:], "bf16")
