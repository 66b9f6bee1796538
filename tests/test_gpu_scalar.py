"""GPU parity of the scalar-decay chunk operator and its composition.

The oracle runs the scalar-decay recurrence token by token in float64
(LinearKV, the affine-operator paragraph, with the write term of Tail-Replay
section 2 Eq. (1)).  The kernel takes keys and values exactly (bf16 inputs)
or split into two bf16 parts (fp32 inputs) and the decayed values split,
with fp32 accumulation, so the bar is the fp32 tolerance (relative Frobenius
error <= 1e-5) for both input dtypes.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import TOL_F32, BLOCK_TOL, check_close, check_state, dev, to_np

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


CU = [0, 512, 1000, 1001, 1001, 1700]   # ragged chunks, one empty, one of a single token


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 128), (128, 64), (64, 64)])
def test_scalar_operator_and_compose_match_oracle(dtype, dk, dv):
    gdn, torch = _gdn()
    H = 3
    inp = workloads.generate([CU[-1]], H=H, dk=dk, dv=dv, dtype=dtype, seed=131, gate_scale=0.01)
    d = dev(inp)
    cu = torch.tensor(CU, dtype=torch.int32, device="cuda")
    g, SL = gdn.scalar_chunk_operator(d["k"], d["alpha"], d["beta"], cu, v=d["v"])
    g_only, none = gdn.scalar_chunk_operator(d["k"], d["alpha"], d["beta"], cu)
    S_in = np.random.Generator(np.random.PCG64(132)).standard_normal((H, dv, dk)).astype(np.float32)
    S = gdn.scalar_compose(g, SL, S_in=torch.from_numpy(S_in).cuda())
    torch.cuda.synchronize()
    f = inp.f64
    g_ref, SL_ref = oracle.scalar_chunk_operator(f["k"], f["alpha"], f["beta"], CU, v=f["v"])
    S_ref = oracle.scalar_compose(g_ref, SL_ref, S_in=S_in.astype(np.float64))
    lab = "scalar %s %dx%d" % (dtype, dv, dk)
    check_close(lab + " gamma", to_np(g), g_ref, 0, TOL_F32, BLOCK_TOL["f32"])
    check_state(lab + " S_local", to_np(SL), SL_ref, "f32")
    check_state(lab + " composed", to_np(S), S_ref, "f32")
    assert none is None and torch.equal(g_only, g)
    assert not to_np(SL)[3].any() and np.all(to_np(g)[3] == 1.0)    # the empty chunk


def test_scalar_compose_in_place_zero_start_and_no_chunks():
    gdn, torch = _gdn()
    H, d = 2, 128
    rng = np.random.Generator(np.random.PCG64(133))
    g = torch.from_numpy(rng.uniform(0.0, 1.0, (7, H)).astype(np.float32)).cuda()
    SL = torch.from_numpy(rng.standard_normal((7, H, d, d)).astype(np.float32)).cuda()
    S0 = rng.standard_normal((H, d, d)).astype(np.float32)
    buf = torch.from_numpy(S0).cuda()
    gdn.scalar_compose(g, SL, S_in=buf, out=buf)
    Z = gdn.scalar_compose(g, SL)
    E = gdn.scalar_compose(g[:0], SL[:0], S_in=torch.from_numpy(S0).cuda())
    torch.cuda.synchronize()
    gn, Ln = to_np(g), to_np(SL)
    check_state("scalar compose in place", to_np(buf), oracle.scalar_compose(gn, Ln, S_in=S0), "f32")
    check_state("scalar compose from zero", to_np(Z), oracle.scalar_compose(gn, Ln), "f32")
    assert np.array_equal(to_np(E), S0.astype(np.float64))


def test_last_block_initializer_is_replay_of_the_last_chunk():
    # LinearKV's last-block initializer takes S_local of the last matched
    # chunk: the same state as a replay of that chunk alone from zero
    gdn, torch = _gdn()
    inp = workloads.generate([4 * 512], H=2, dk=128, dv=128, dtype="bf16", seed=134)
    d = dev(inp)
    cu = torch.from_numpy(workloads.chunk_bounds(inp.n_tokens, 512)).cuda()
    _, SL = gdn.chunk_operator(d["k"], d["alpha"], d["beta"], cu, v=d["v"])
    last = slice(3 * 512, 4 * 512)
    cu1 = torch.tensor([0, 512], dtype=torch.int32, device="cuda")
    _, S = gdn.replay(None, d["k"][last].contiguous(), d["v"][last].contiguous(), d["alpha"][last].contiguous(),
                      d["beta"][last].contiguous(), cu1, want_o=False)
    torch.cuda.synchronize()
    f = inp.f64
    S_ref = oracle.replay(f["q"][last], f["k"][last], f["v"][last], f["alpha"][last], f["beta"][last],
                          np.array([0, 512], np.int32), want_o=False)[1]
    check_state("last-block initializer", to_np(SL[3]), S_ref[0], "bf16")
    check_state("replay of the last chunk", to_np(S[0]), S_ref[0], "bf16")


def test_scalar_operator_past_the_dma_size_limit():
    """Keys and values of 2^31 bytes or more go through the generic kernel
    (the load-to-LDS path addresses them with 31-bit offsets): 65536 tokens x
    128 heads at d = 128 in bf16.  Two generated heads are repeated to 128
    (heads are independent); sampled chunks of every kind of head copy are
    checked against the oracle."""
    gdn, torch = _gdn()
    T, Hs, R, d, CH = 65536, 2, 64, 128, 512
    inp = workloads.generate([T], H=Hs, dk=d, dv=d, dtype="bf16", seed=137, gate_scale=0.01)
    dd = dev(inp)
    big = {n: dd[n].repeat(1, R, 1) if dd[n].dim() == 3 else dd[n].repeat(1, R) for n in ("k", "v", "alpha", "beta")}
    H = Hs * R
    assert big["k"].shape == (T, H, d) and big["k"].numel() * 2 >= 2 ** 31
    cu_np = np.arange(0, T + 1, CH, dtype=np.int32)
    g, SL = gdn.scalar_chunk_operator(big["k"], big["alpha"], big["beta"], torch.from_numpy(cu_np).cuda(),
                                      v=big["v"])
    torch.cuda.synchronize()
    f = inp.f64
    for c in (0, 63, T // CH - 1):
        t0, t1 = int(cu_np[c]), int(cu_np[c + 1])
        g_ref, SL_ref = oracle.scalar_chunk_operator(f["k"][t0:t1], f["alpha"][t0:t1], f["beta"][t0:t1],
                                                     [0, t1 - t0], v=f["v"][t0:t1])
        for h in (0, 1, H // 2, H - 1):
            lab = "scalar large chunk %d head %d" % (c, h)
            check_close(lab + " gamma", to_np(g[c, h:h + 1]), g_ref[0, h % Hs:h % Hs + 1], 0, TOL_F32,
                        BLOCK_TOL["f32"])
            check_state(lab + " S_local", to_np(SL[c, h]), SL_ref[0, h % Hs], "f32")
    del big, SL
