"""GPU parity of gdn_front_end (normalised q, k and activated gates).

The oracle is oracle.front_end in float64 (page "Tail-Replay: Escaping the
Curse of Linear Attention in Prefix Caching for Hybrid LLMs", section 3, with
section 2 Eq. (1)).  The kernel computes in fp32 and rounds each result once
to the input dtype, so the element-wise bar is:
- bf16: |out - ref| <= 2^-8 |ref| (half a bf16 unit at most) plus fp32
  rounding; an element may round to the other neighbour of ref when the fp32
  value lies within fp32 rounding of a tie, so the share of elements that
  differ from ref rounded to bf16 is reported and bounded;
- f32: |out - ref| <= 1e-6 (the results lie in [-1, 1]) and 1e-6 relative
  for the gates.
End to end, the front end followed by a replay is checked against the oracle
front end, rounded to bf16 like any bf16 input, followed by the oracle replay
at the bf16 replay tolerance.
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import check_out, check_state, oracle_replay, to_np

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def _t(raw, a):
    import torch
    if raw.dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def _check(out, ref, dtype, what):
    out = to_np(out)
    if dtype == "bf16":
        err = np.abs(out - ref)
        bound = 2.0 ** -8 * np.abs(ref) * (1 + 1e-5) + 1e-37
        assert np.all(err <= bound), "%s: max excess %.3e" % (what, np.max(err - bound))
        rounded = workloads.bf16_to_f64(workloads.bf16_bits(ref))
        share = np.mean(out != rounded)
        print("%s: %.2e of the elements round to the other neighbour" % (what, share), flush=True)
        assert share <= 1e-3
    else:
        err = np.abs(out - ref)
        assert np.all(err <= 1e-6 * np.maximum(1.0, np.abs(ref))), "%s: max error %.3e" % (what, np.max(err))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("dk", [64, 128])
@pytest.mark.parametrize("with_q", [True, False])
def test_front_end_matches_oracle(dtype, dk, with_q):
    gdn, torch = _gdn()
    raw = workloads.generate_raw([1, 0, 77, 300], H=3, dk=dk, dv=64, dtype=dtype, seed=111)
    # a zero key row and a zero query row stay zero
    raw.k_raw[5, 1] = 0
    raw.q_raw[9, 2] = 0
    qr = _t(raw, raw.q_raw) if with_q else None
    q, k, a, b = gdn.front_end(qr, _t(raw, raw.k_raw), _t(raw, raw.g), _t(raw, raw.b))
    torch.cuda.synchronize()
    rq, rk, ra, rb = oracle.front_end(raw.f64("q_raw") if with_q else None, raw.f64("k_raw"), raw.f64("g"),
                                      raw.f64("b"))
    assert (q is None) == (not with_q)
    if with_q:
        _check(q, rq, dtype, "q")
        assert not to_np(q)[9, 2].any()
    _check(k, rk, dtype, "k")
    assert not to_np(k)[5, 1].any()
    _check(a, ra, dtype, "alpha")
    _check(b, rb, dtype, "beta")


def test_front_end_in_place_and_empty():
    gdn, torch = _gdn()
    raw = workloads.generate_raw([513], H=4, dk=128, dv=128, dtype="bf16", seed=112)
    ins = [_t(raw, x) for x in (raw.q_raw, raw.k_raw, raw.g, raw.b)]
    ref = gdn.front_end(*[x.clone() for x in ins])
    outs = gdn.front_end(*ins, out=tuple(ins))
    torch.cuda.synchronize()
    for x, o, r in zip(ins, outs, ref):
        assert o is x and torch.equal(x, r)
    empty = [x[:0] for x in ins]
    q, k, a, b = gdn.front_end(*empty)
    torch.cuda.synchronize()
    assert k.shape == (0, 4, 128) and a.shape == (0, 4)


def test_front_end_then_replay():
    gdn, torch = _gdn()
    raw = workloads.generate_raw([300, 0, 77, 1], H=2, dk=128, dv=128, dtype="bf16", seed=113)
    q, k, a, b = gdn.front_end(_t(raw, raw.q_raw), _t(raw, raw.k_raw), _t(raw, raw.g), _t(raw, raw.b))
    cu = torch.from_numpy(raw.cu_seqlens).cuda()
    o, S = gdn.replay(q, k, _t(raw, raw.v), a, b, cu, want_o=True)
    torch.cuda.synchronize()
    rq, rk, ra, rb = oracle.front_end(raw.f64("q_raw"), raw.f64("k_raw"), raw.f64("g"), raw.f64("b"))
    bits = workloads.bf16_bits
    inp = workloads.Inputs(dtype="bf16", H=2, dk=128, dv=128, cu_seqlens=raw.cu_seqlens, q=bits(rq), k=bits(rk),
                           v=raw.v, alpha=bits(ra), beta=bits(rb))
    o_ref, S_ref = oracle_replay(inp)
    check_out("front end + replay o", to_np(o), o_ref, "bf16")
    check_state("front end + replay S", to_np(S), S_ref, "bf16")
