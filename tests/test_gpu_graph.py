"""The calls under HIP graph capture.

Every launch of gdn_replay, gdn_chunk_operator, gdn_compose, gdn_front_end,
gdn_decode and the scalar-decay calls is stream-ordered on the caller's
stream with no host synchronisation, memset or copy, so a captured call
replays the same kernels on the same buffers.
Each case captures one call, then replays the graph several times with
eager work (the outputs overwritten) and synchronisations in between; every
replay must reproduce the eager result bit for bit (the kernels are
deterministic).
"""
import numpy as np
import pytest

import workloads
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def _capture_and_check(fn):
    """fn() returns its output tensors; compare graph replays with one eager call."""
    gdn, torch = _gdn()
    eager = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):      # warm-up on a side stream before capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = fn()                    # outputs allocated in capture stay the graph's
    for it in range(3):
        for t in outs:
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for t, e in zip(outs, eager):
            assert torch.equal(t, e), "graph replay %d differs from the eager call" % it


@pytest.mark.parametrize("case", ["packed_with_outputs", "split_state_only", "split_with_outputs"])
def test_replay_under_graph_capture(case):
    gdn, torch = _gdn()
    if case == "packed_with_outputs":
        inp = workloads.generate([300, 0, 700, 65], H=2, dk=128, dv=128, dtype="bf16", seed=81)
        want_o, P = True, None
    else:
        inp = workloads.generate([1000], H=2, dk=128, dv=128, dtype="bf16", seed=82)
        want_o, P = case == "split_with_outputs", 3
    d = dev(inp)

    def call():
        o, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], want_o=want_o, segments=P)
        return [S] + ([o] if want_o else [])
    _capture_and_check(call)


def test_chunk_operator_and_compose_under_graph_capture():
    gdn, torch = _gdn()
    inp = workloads.generate([5 * 128], H=2, dk=128, dv=64, dtype="bf16", seed=83)
    d = dev(inp)
    cu = torch.from_numpy(workloads.chunk_bounds(inp.n_tokens, 128)).cuda()
    S_in = torch.from_numpy(np.random.Generator(np.random.PCG64(84)).standard_normal((2, 64, 128))
                            .astype(np.float32)).cuda()

    def call():
        TC, SL = gdn.chunk_operator(d["k"], d["alpha"], d["beta"], cu, v=d["v"])
        return [TC, SL, gdn.compose(TC, SL, S_in=S_in)]
    _capture_and_check(call)


def test_front_end_decode_and_scalar_ops_under_graph_capture():
    gdn, torch = _gdn()
    raw = workloads.generate_raw([300], H=2, dk=128, dv=128, dtype="bf16", seed=85)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    qr, kr, g, b, v = t(raw.q_raw), t(raw.k_raw), t(raw.g), t(raw.b), t(raw.v)
    cu = torch.from_numpy(workloads.chunk_bounds(300, 128)).cuda()
    S_in = torch.from_numpy(np.random.Generator(np.random.PCG64(86)).standard_normal((300, 2, 128, 128))
                            .astype(np.float32) * 0.1).cuda()

    def call():
        q, k, a, be = gdn.front_end(qr, kr, g, b)
        o, S = gdn.decode(q, k, v, a, be, S_in=S_in)
        gam, SL = gdn.scalar_chunk_operator(k, a, be, cu, v=v)
        return [q, k, a, be, o, S, gam, SL, gdn.scalar_compose(gam, SL)]
    _capture_and_check(call)
