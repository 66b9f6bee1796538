"""The widened calls at the sizes bench.py times, against the oracle.

- decode: 64 requests x 32 heads, d = 128, bf16 (every output);
- front end: 3277 tokens x 32 heads, q and k (every output);
- scalar-decay operators: 64 chunks of 512 tokens x 32 heads, d = 128, on
  sampled heads (heads are independent; the oracle's token loop is slow).
Bars as in the small-size tests: the fp32 tolerance for decode and the
scalar-decay operators, half a bf16 unit per element for the front end.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import TOL_F32, BLOCK_TOL, check_close, check_out, check_state, dev, oracle_replay, to_np

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def test_decode_bench_size():
    gdn, torch = _gdn()
    N, H, d = 64, 32, 128
    inp = workloads.generate([1] * N, H=H, dk=d, dv=d, dtype="bf16", seed=5)
    S_in = (np.random.Generator(np.random.PCG64(6)).standard_normal((N, H, d, d)) * 0.3).astype(np.float32)
    dd = dev(inp)
    o, S = gdn.decode(dd["q"], dd["k"], dd["v"], dd["alpha"], dd["beta"], S_in=torch.from_numpy(S_in).cuda())
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_replay(inp, S0=S_in.astype(np.float64))
    check_out("decode 64 x 32 o", to_np(o), o_ref, "f32")
    check_state("decode 64 x 32 S", to_np(S), S_ref, "f32")


def test_front_end_bench_size():
    gdn, torch = _gdn()
    raw = workloads.generate_raw([workloads.tail_length(32768, "0.1")], H=32, dk=128, dv=128, dtype="bf16", seed=7)

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    outs = gdn.front_end(t(raw.q_raw), t(raw.k_raw), t(raw.g), t(raw.b))
    torch.cuda.synchronize()
    refs = oracle.front_end(raw.f64("q_raw"), raw.f64("k_raw"), raw.f64("g"), raw.f64("b"))
    for name, o, r in zip("q k alpha beta".split(), outs, refs):
        err = np.abs(to_np(o) - r)
        assert np.all(err <= 2.0 ** -8 * np.abs(r) * (1 + 1e-5) + 1e-37), name


def test_scalar_ops_bench_size_sampled_heads():
    gdn, torch = _gdn()
    inp = workloads.make_workload(4)
    d = dev(inp)
    cu_np = workloads.chunk_bounds(inp.n_tokens, 512)
    cu = torch.from_numpy(cu_np).cuda()
    g, SL = gdn.scalar_chunk_operator(d["k"], d["alpha"], d["beta"], cu, v=d["v"])
    S = gdn.scalar_compose(g, SL)
    torch.cuda.synchronize()
    heads = [0, 31]
    f = inp.f64
    g_ref, SL_ref = oracle.scalar_chunk_operator(f["k"][:, heads], f["alpha"][:, heads], f["beta"][:, heads], cu_np,
                                                 v=f["v"][:, heads])
    S_ref = oracle.scalar_compose(g_ref, SL_ref)
    check_close("scalar gamma", to_np(g[:, heads]), g_ref, 0, TOL_F32, BLOCK_TOL["f32"])
    check_state("scalar S_local", to_np(SL[:, heads]), SL_ref, "f32")
    check_state("scalar composed", to_np(S[heads]), S_ref, "f32")
