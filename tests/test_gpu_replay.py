"""GPU parity of gdn_replay against the fp64 oracle (through the C ABI).

Bars (tests/gpu_helpers.py): the relative Frobenius error over the whole
output tensor (<= 1e-5 for fp32 inputs, <= 3e-3 for bf16 inputs with an fp32
state) and, per (sequence, head) state and per (token, head) output row, the
element-level bars.  Recurrence: page "Tail-Replay: Escaping the Curse of
Linear Attention in Prefix Caching for Hybrid LLMs", section 2 Eq. (1).
"""
import ctypes

import numpy as np
import pytest

import workloads
from tests.gpu_helpers import check_out, check_replay, check_state, dev, oracle_replay, run_replay, to_np

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def test_workload0_single_head_f32():
    inp = workloads.make_workload(0)
    check_replay("workload 0", inp)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
def test_ragged_multi_tile(dtype, d):
    # lengths span partial chunks, exact multiples and several chunks, plus empties
    inp = workloads.generate([1, 63, 64, 65, 0, 200, 130], H=3, dk=d, dv=d, dtype=dtype, seed=21)
    check_replay("ragged %s d=%d" % (dtype, d), inp)


@pytest.mark.parametrize("dk,dv", [(64, 128), (128, 64)])
def test_rectangular_state(dk, dv):
    inp = workloads.generate([77, 150], H=2, dk=dk, dv=dv, dtype="bf16", seed=22)
    check_replay("rect %dx%d" % (dv, dk), inp)


def test_nonzero_start_state_and_state_only():
    # one recurrence per sequence (no time split), so both calls run the same chain
    inp = workloads.generate([70, 129, 5], H=2, dk=128, dv=128, dtype="bf16", seed=23)
    rng = np.random.Generator(np.random.PCG64(5))
    S0 = rng.standard_normal((3, 2, 128, 128)) * 0.1
    S0 = S0.astype(np.float32).astype(np.float64)
    check_replay("S0", inp, S0=S0, segments=1)
    o1, S1 = run_replay(inp, S0=S0, want_o=True, segments=1)
    o2, S2 = run_replay(inp, S0=S0, want_o=False, segments=1)
    assert o2 is None
    assert np.array_equal(S1, S2)   # the state path does not depend on o


def test_in_place_state_update():
    gdn, torch = _gdn()
    inp = workloads.generate([100, 40], H=2, dk=64, dv=64, dtype="bf16", seed=24)
    d = dev(inp)
    S0 = torch.randn(2, 2, 64, 64, device="cuda") * 0.1
    S0_np = to_np(S0)
    _, S_sep = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=S0.clone(),
                          want_o=False)
    S_io = S0.clone()
    gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=S_io, want_o=False,
               S_out=S_io)
    torch.cuda.synchronize()
    assert torch.equal(S_sep, S_io)
    _, S_ref = oracle_replay(inp, S0=S0_np, want_o=False)
    check_state("in place", to_np(S_io), S_ref, "bf16")


def test_bf16_output():
    _, torch = _gdn()
    inp = workloads.generate([300], H=2, dk=128, dv=128, dtype="bf16", seed=25)
    # rounding o itself to bf16 costs ~1.7e-3 of relative error (whole tensor)
    check_replay("bf16 o", inp, o_dtype=torch.bfloat16)


def test_identity_gate_keeps_state_exactly():
    inp = workloads.generate([150], H=2, dk=128, dv=128, dtype="bf16", seed=26, alpha_one=True,
                             beta_value=0.0)
    rng = np.random.Generator(np.random.PCG64(6))
    S0 = rng.standard_normal((1, 2, 128, 128)).astype(np.float32).astype(np.float64)
    o, S = run_replay(inp, S0=S0)
    assert np.array_equal(S, S0)
    o_ref, _ = oracle_replay(inp, S0=S0)
    check_out("identity gate o", o, o_ref, "bf16")


def test_empty_sequences_return_start_state():
    inp = workloads.generate([0, 10, 0], H=2, dk=64, dv=64, dtype="f32", seed=27)
    rng = np.random.Generator(np.random.PCG64(7))
    S0 = rng.standard_normal((3, 2, 64, 64)).astype(np.float32).astype(np.float64)
    o, S = run_replay(inp, S0=S0)
    assert np.array_equal(S[0], S0[0]) and np.array_equal(S[2], S0[2])
    _, Sz = run_replay(inp, S0=None, want_o=False)
    assert not np.any(Sz[0]) and not np.any(Sz[2])


def test_deterministic():
    inp = workloads.generate([333, 64], H=4, dk=128, dv=128, dtype="bf16", seed=28)
    o1, S1 = run_replay(inp)
    o2, S2 = run_replay(inp)
    assert np.array_equal(o1, o2) and np.array_equal(S1, S2)


def test_repeated_calls_stay_bitwise_identical():
    # Many calls over alternating inputs: every result equal, bit for bit, to
    # that input's first one (a read of a stale or wrong LDS address shows up
    # as one wave's 16 state rows going wrong from some chunk on, now and then).
    import torch
    cases = [(workloads.generate([1, 63, 64, 65, 0, 200, 130], H=3, dk=128, dv=128, dtype="bf16", seed=21), None),
             (workloads.generate([1000], H=2, dk=128, dv=128, dtype="bf16", seed=30, alpha_one=True), None),
             (workloads.generate([300], H=2, dk=128, dv=128, dtype="bf16", seed=25), torch.bfloat16),
             (workloads.generate([500, 77], H=2, dk=64, dv=128, dtype="bf16", seed=63), None)]
    first = [None] * len(cases)
    for _ in range(25):
        for i, (inp, o_dtype) in enumerate(cases):
            o, S = run_replay(inp, o_dtype=o_dtype)
            if first[i] is None:
                first[i] = (o, S)
            else:
                assert np.array_equal(o, first[i][0]) and np.array_equal(S, first[i][1]), "case %d" % i


@pytest.mark.parametrize("n_seqs", [200, 300])
def test_many_sequences(n_seqs):
    # packed batches below and above the longest-first ordering limit (256
    # sequences): lengths 0 .. 200, duplicates and empties included
    rng = np.random.Generator(np.random.PCG64(n_seqs))
    lengths = [int(x) for x in rng.integers(0, 200, size=n_seqs, endpoint=True)]
    inp = workloads.generate(lengths, H=2, dk=64, dv=64, dtype="bf16", seed=n_seqs + 1)
    check_replay("%d sequences" % n_seqs, inp)


def test_varlen_equals_per_sequence_calls():
    inp = workloads.generate([90, 0, 257, 64], H=3, dk=128, dv=128, dtype="bf16", seed=29)
    o, S = run_replay(inp)
    cu = inp.cu_seqlens
    for n in range(4):
        sl = slice(cu[n], cu[n + 1])
        if cu[n + 1] == cu[n]:
            assert not np.any(S[n])
            continue
        sub = workloads.Inputs(dtype=inp.dtype, H=inp.H, dk=inp.dk, dv=inp.dv,
                               cu_seqlens=np.array([0, cu[n + 1] - cu[n]], np.int32),
                               q=inp.q[sl], k=inp.k[sl], v=inp.v[sl], alpha=inp.alpha[sl],
                               beta=inp.beta[sl])
        on, Sn = run_replay(sub)
        assert np.array_equal(Sn[0], S[n])
        assert np.array_equal(on, o[sl])


@pytest.mark.parametrize("gate", ["slow", "one", "strong"])
def test_stress_gate_laws(gate):
    # slow: alpha = exp(-0.001 softplus(x)); one: alpha = 1; strong: alpha =
    # exp(-5 softplus(x)), whose cumulative in-chunk gates underflow fp32
    kw = {"slow": dict(gate_scale=0.001), "one": dict(alpha_one=True), "strong": dict(gate_scale=5.0)}[gate]
    inp = workloads.generate([1000], H=2, dk=128, dv=128, dtype="bf16", seed=30, **kw)
    check_replay("gate %s bf16" % gate, inp)
    inp32 = workloads.generate([700], H=2, dk=128, dv=128, dtype="f32", seed=31, **kw)
    check_replay("gate %s f32" % gate, inp32)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("segments", [1, 3])
def test_non_unit_keys(dtype, segments):
    # keys are used as given: norms in [0.5, 1.2] with beta <= 1 (the
    # transition alpha (I - beta k k^T) then has 1 - beta |k|^2 in [-0.44, 1])
    inp = workloads.generate([700, 190, 1], H=3, dk=128, dv=128, dtype=dtype, seed=32, key_scale=(0.5, 1.2))
    check_replay("non-unit keys %s P=%d" % (dtype, segments), inp, segments=segments)
    check_replay("non-unit keys state only %s P=%d" % (dtype, segments), inp, want_o=False, segments=segments)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("segments", [1, 4])
def test_zero_gates(dtype, segments):
    # alpha = 0 exactly on 3% of (token, head) pairs, under the strong-decay
    # law: the kernels floor log(alpha) at -60, the oracle multiplies by 0
    inp = workloads.generate([900, 64, 3], H=2, dk=128, dv=128, dtype=dtype, seed=33, gate_scale=5.0,
                             alpha_zero_frac=0.03)
    assert np.any(inp.f64["alpha"] == 0.0)
    check_replay("zero gates %s P=%d" % (dtype, segments), inp, segments=segments)
    check_replay("zero gates state only %s P=%d" % (dtype, segments), inp, want_o=False, segments=segments)


def test_front_end_zero_gate_feeds_replay():
    # gdn_front_end turns a log-gate below about -92 into alpha = 0 in bf16;
    # gdn_replay takes that alpha and stays finite and within the bars
    gdn, torch = _gdn()
    raw = workloads.generate_raw([400], H=2, dk=128, dv=128, dtype="bf16", seed=34)
    g = raw.f64("g")
    g[::7] = -200.0                       # rounds exactly in bf16; exp(-200) = 0 in bf16
    g_bits = workloads.bf16_bits(g)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    q, k, alpha, beta = gdn.front_end(t(raw.q_raw), t(raw.k_raw), t(g_bits), t(raw.b))
    v = t(raw.v)
    cu = torch.from_numpy(raw.cu_seqlens).cuda()
    o, S = gdn.replay(q, k, v, alpha, beta, cu)
    torch.cuda.synchronize()
    a_np = to_np(alpha)
    assert np.all(a_np[::7] == 0.0)
    import oracle
    o_ref, S_ref = oracle.replay(to_np(q), to_np(k), raw.f64("v"), a_np, to_np(beta), raw.cu_seqlens)
    check_state("front end -> replay S", to_np(S), S_ref, "bf16")
    check_out("front end -> replay o", to_np(o), o_ref, "bf16")


def test_replay_on_a_side_stream_keeps_its_workspace():
    # The binding allocates the workspace on the stream the call launches on:
    # blocks of the workspace's size that the current stream allocates right
    # after the call (and fills with NaN) are never the workspace that the
    # side stream's kernels are still using.
    gdn, torch = _gdn()
    inp = workloads.generate([3000], H=4, dk=128, dv=128, dtype="bf16", seed=35)
    d = dev(inp)
    o_ref, S_ref = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"])
    torch.cuda.synchronize()
    ws_floats = (gdn.library().gdn_replay_workspace_bytes(1, 3000, 4, 128, 128) + 3) // 4
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    for _ in range(5):
        o, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], stream=side)
        junk = [torch.full((ws_floats,), float("nan"), device="cuda") for _ in range(4)]
        side.synchronize()
        torch.cuda.synchronize()
        del junk
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref)


def test_error_left_by_an_earlier_call_is_not_reported():
    # A failed call of the HIP runtime leaves its error for hipGetLastError;
    # the library reports only the status of its own launches.  The call goes
    # straight through the C ABI so that nothing else runs between the failed
    # runtime call and the library's launches.
    gdn, torch = _gdn()
    lib = gdn.library()
    hip = ctypes.CDLL("libamdhip64.so")
    hip.hipSetDevice.argtypes = [ctypes.c_int]
    inp = workloads.generate([130], H=2, dk=64, dv=64, dtype="bf16", seed=36)
    d = dev(inp)
    o = torch.empty((130, 2, 64), dtype=torch.float32, device="cuda")
    S = torch.empty((1, 2, 64, 64), dtype=torch.float32, device="cuda")
    nbytes = lib.gdn_replay_workspace_bytes(1, 130, 2, 64, 64)
    ws = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    torch.cuda.synchronize()
    p = lambda t: ctypes.c_void_p(t.data_ptr())
    count = ctypes.c_int(0)
    assert hip.hipGetDeviceCount(ctypes.byref(count)) == 0
    assert hip.hipSetDevice(count.value + 7) != 0      # an invalid ordinal: nothing changes
    planted = hip.hipPeekAtLastError()
    try:
        st = lib.gdn_replay(p(d["q"]), p(d["k"]), p(d["v"]), p(d["alpha"]), p(d["beta"]), None, p(d["cu"]), 1, 130,
                            2, 64, 64, 1, p(o), 0, p(S), p(ws), nbytes, ctypes.c_void_p(stream.cuda_stream))
    finally:
        pending = hip.hipGetLastError()                 # leave the thread's error state clean
    print("planted error %d, status %d, pending after the call %d" % (planted, st, pending), flush=True)
    assert st == 0, lib.gdn_last_error()
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_replay(inp)
    check_state("after an earlier error S", to_np(S), S_ref, "bf16")
    check_out("after an earlier error o", to_np(o), o_ref, "bf16")
