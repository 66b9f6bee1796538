"""GPU parity of gdn_chunk_operator and gdn_compose against the fp64 oracle.

T_C / S_local are compared per chunk over the whole output tensors; the
composed state is compared with the oracle's sequential replay over all the
chunks' tokens (the composition adds no approximation of its own, so the
two must agree to the kernels' rounding).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import BLOCK_TOL, TOL_BF16, TOL_F32, check_close, check_state, dev, to_np

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def gpu_ops(inp, bounds, with_v=True):
    gdn, torch = _gdn()
    d = dev(inp)
    cu = torch.from_numpy(np.asarray(bounds, np.int32)).cuda()
    TC, SL = gdn.chunk_operator(d["k"], d["alpha"], d["beta"], cu, v=d["v"] if with_v else None)
    torch.cuda.synchronize()
    return TC, SL


def check_T(label, TC, TC_ref, dtype):
    """T_C [C, H, dk, dk]: one block per (chunk, head)."""
    return check_close(label, TC, TC_ref, 2, TOL_F32 if dtype == "f32" else TOL_BF16, BLOCK_TOL[dtype])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128), (64, 128)])
def test_chunk_operator_uneven_chunks(dtype, dk, dv):
    bounds = np.cumsum([0, 1, 5, 64, 65, 130, 0, 200]).astype(np.int32)
    inp = workloads.generate([int(bounds[-1])], H=2, dk=dk, dv=dv, dtype=dtype, seed=41,
                             gate_scale=0.01)
    TC, SL = gpu_ops(inp, bounds)
    f = inp.f64
    TC_ref, SL_ref = oracle.chunk_operator(f["k"], f["alpha"], f["beta"], bounds, v=f["v"])
    check_T("T_C %s %dx%d" % (dtype, dk, dv), to_np(TC), TC_ref, dtype)
    check_state("S_local %s %dx%d" % (dtype, dk, dv), to_np(SL), SL_ref, dtype)
    # the empty chunk is the identity with a zero local state
    assert np.array_equal(to_np(TC)[5], np.broadcast_to(np.eye(dk), (2, dk, dk)))
    assert not np.any(to_np(SL)[5])


def test_transition_only():
    bounds = np.array([0, 100, 300], np.int32)
    inp = workloads.generate([300], H=2, dk=128, dv=128, dtype="bf16", seed=42, alpha_one=True)
    TC, SL = gpu_ops(inp, bounds, with_v=False)
    assert SL is None
    TC2, _ = gpu_ops(inp, bounds, with_v=True)
    assert np.array_equal(to_np(TC), to_np(TC2))
    f = inp.f64
    TC_ref, _ = oracle.chunk_operator(f["k"], f["alpha"], f["beta"], bounds)
    check_T("T_C only", to_np(TC), TC_ref, "bf16")


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128)])
def test_chunk_operator_item_streams(dk, dv):
    # more (chunk, head) items than two per compute unit (40 chunks x 16
    # heads): each workgroup runs a run of items as one stream of chunks,
    # with runs that start and end inside a chunk's heads; ragged chunks and
    # empty ones (the first, the last and a run of three), each item
    # checked against the oracle on sampled heads
    rng = np.random.Generator(np.random.PCG64(45))
    lengths = rng.integers(1, 300, 40)
    lengths[[0, 7, 8, 9, 39]] = 0
    lengths[12] = 64
    bounds = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    H, heads = 16, [0, 3, 9, 15]
    inp = workloads.generate([int(bounds[-1])], H=H, dk=dk, dv=dv, dtype="bf16", seed=46)
    TC, SL = gpu_ops(inp, bounds)
    f = inp.f64
    TC_ref, SL_ref = oracle.chunk_operator(f["k"][:, heads], f["alpha"][:, heads], f["beta"][:, heads], bounds,
                                           v=f["v"][:, heads])
    check_T("T_C item streams %dx%d" % (dk, dv), to_np(TC)[:, heads], TC_ref, "bf16")
    check_state("S_local item streams %dx%d" % (dk, dv), to_np(SL)[:, heads], SL_ref, "bf16")
    for c in (0, 7, 8, 9, 39):   # empty chunks, every head: identity and zero
        assert np.array_equal(to_np(TC)[c], np.broadcast_to(np.eye(dk), (H, dk, dk)))
        assert not np.any(to_np(SL)[c])
    # one head alone (40 items: one workgroup per item) gives the same bits:
    # the streams change the schedule, not the arithmetic
    gdn, torch = _gdn()
    d = dev(inp)
    cu = torch.from_numpy(bounds).cuda()
    for h in (0, 9):
        one = {key: d[key][:, h:h + 1].contiguous() for key in ("k", "v", "alpha", "beta")}
        TC1, SL1 = gdn.chunk_operator(one["k"], one["alpha"], one["beta"], cu, v=one["v"])
        torch.cuda.synchronize()
        assert torch.equal(TC1[:, 0], TC[:, h]) and torch.equal(SL1[:, 0], SL[:, h])


@pytest.mark.parametrize("gate", ["one", "slow", "workload"])
def test_compose_matches_sequential_replay(gate):
    kw = dict(alpha_one=True) if gate == "one" else (
        dict(gate_scale=0.001) if gate == "slow" else {})
    n_chunks, L = 6, 96
    inp = workloads.generate([n_chunks * L], H=3, dk=128, dv=128, dtype="bf16", seed=43, **kw)
    bounds = workloads.chunk_bounds(n_chunks * L, L)
    gdn, torch = _gdn()
    TC, SL = gpu_ops(inp, bounds)
    rng = np.random.Generator(np.random.PCG64(9))
    S_in = (rng.standard_normal((3, 128, 128)) * 0.2).astype(np.float32)
    S_in_t = torch.from_numpy(S_in).cuda()
    S = gdn.compose(TC, SL, S_in=S_in_t)
    torch.cuda.synchronize()
    f = inp.f64
    _, S_seq = oracle.replay(None, f["k"], f["v"], f["alpha"], f["beta"], [0, n_chunks * L],
                             S0=S_in[None].astype(np.float64), want_o=False)
    print("gate %s ||T_C||/sqrt(d) %.3e" % (gate, np.linalg.norm(to_np(TC)[0, 0]) / np.sqrt(128)), flush=True)
    check_state("composed (gate %s)" % gate, to_np(S), S_seq[0], "bf16")


def test_compose_exact_operators_fp32():
    """Compose alone, fed the oracle's own operators: fp32-level agreement."""
    gdn, torch = _gdn()
    rng = np.random.Generator(np.random.PCG64(10))
    H, dk, dv, C = 2, 128, 64, 9
    inp = workloads.generate([C * 40], H=H, dk=dk, dv=dv, dtype="f32", seed=44, gate_scale=0.01)
    bounds = workloads.chunk_bounds(C * 40, 40)
    f = inp.f64
    TC_ref, SL_ref = oracle.chunk_operator(f["k"], f["alpha"], f["beta"], bounds, v=f["v"])
    TC32, SL32 = TC_ref.astype(np.float32), SL_ref.astype(np.float32)
    S_in = rng.standard_normal((H, dv, dk)).astype(np.float32)
    ref = oracle.compose(TC32, SL32, S_in=S_in)
    S = gdn.compose(torch.from_numpy(TC32).cuda(), torch.from_numpy(SL32).cuda(),
                    S_in=torch.from_numpy(S_in).cuda())
    torch.cuda.synchronize()
    check_state("compose of exact operators", to_np(S), ref, "f32")
    # zero chunks returns the incoming state; in place is allowed
    S_in_t = torch.from_numpy(S_in).cuda()
    S0 = gdn.compose(torch.from_numpy(TC32[:0]).cuda(), torch.from_numpy(SL32[:0]).cuda(),
                     S_in=S_in_t)
    torch.cuda.synchronize()
    assert np.array_equal(to_np(S0), S_in.astype(np.float64))
    S_io = torch.from_numpy(S_in).cuda()
    gdn.compose(torch.from_numpy(TC32).cuda(), torch.from_numpy(SL32).cuda(), S_in=S_io, out=S_io)
    torch.cuda.synchronize()
    assert torch.equal(S_io, S)
