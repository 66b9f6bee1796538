"""GPU parity of gdn_replay_raw, the front end inside the replay.

The oracle is oracle.front_end on the raw projections (q and k divided by
their norms, alpha = exp(g), beta = sigmoid(b), in float64) followed by
oracle.replay (page "Tail-Replay: Escaping the Curse of Linear Attention in
Prefix Caching for Hybrid LLMs", section 3, with section 2 Eq. (1)).  The
call normalises and activates in fp32 and never rounds those results to
bf16, so it meets the bars of a bf16 replay of exact inputs
(tests/gpu_helpers.py).  Cases cover packed sequences (one workgroup per
sequence and head, records from the prep kernel) and single long sequences
(time split with its fused record prologue, with and without outputs),
zero key and query rows, log-gates below the -60 floor, and keys and
queries whose norms span 0.25 to 4 times sqrt(dk).
"""
import numpy as np
import pytest

import oracle
import workloads
from tests.gpu_helpers import check_out, check_state, rel, to_np

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def _t(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


def _oracle(raw, S0, want_o):
    rq, rk, ra, rb = oracle.front_end(raw.f64("q_raw"), raw.f64("k_raw"), raw.f64("g"), raw.f64("b"))
    return oracle.replay(rq, rk, raw.f64("v"), ra, rb, raw.cu_seqlens, S0=S0, want_o=want_o)


def _run(label, raw, S0=None, want_o=True, o_bf16=False):
    gdn, torch = _gdn()
    cu = torch.from_numpy(raw.cu_seqlens).cuda()
    S0_t = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    o, S = gdn.replay_raw(_t(raw.q_raw), _t(raw.k_raw), _t(raw.v), _t(raw.g), _t(raw.b), cu, S0=S0_t,
                          want_o=want_o, o_dtype=torch.bfloat16 if o_bf16 else None)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(raw, S0, want_o)
    check_state(label + " S_final", to_np(S), S_ref, "bf16")
    if want_o:
        check_out(label + " o", to_np(o), o_ref, "bf16", o_bf16=o_bf16)
    return o, S


CASES = [
    # label, lengths, H, dk, dv, S0, want_o, o_bf16
    ("packed d128 S0 o", [300, 0, 77, 1, 64, 65, 129], 3, 128, 128, True, True, False),
    ("packed dk64 dv128 o bf16", [200, 33, 0, 128], 2, 64, 128, False, True, True),
    ("packed state only dk128 dv64", [500, 7, 64], 3, 128, 64, True, False, False),
    ("long time split o", [4000], 4, 128, 128, True, True, False),
    ("long time split state only", [4000], 4, 128, 128, False, False, False),
]


@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_replay_raw_matches_oracle(case):
    label, lengths, H, dk, dv, with_s0, want_o, o_bf16 = case
    raw = workloads.generate_raw(lengths, H=H, dk=dk, dv=dv, dtype="bf16", seed=300 + len(label))
    S0 = None
    if with_s0:
        rng = np.random.Generator(np.random.PCG64(301))
        S0 = (rng.standard_normal((len(lengths), H, dv, dk)) * 0.2).astype(np.float32).astype(np.float64)
    print(label, lengths, H, dk, dv, flush=True)
    _run(label, raw, S0=S0, want_o=want_o, o_bf16=o_bf16)


def test_replay_raw_zero_rows_and_gate_floor():
    # zero key and query rows give zero normalised rows; log-gates below -60
    # act as -60 (a carried state scaled by e^-60 instead of exactly erased)
    raw = workloads.generate_raw([150, 90], H=2, dk=128, dv=128, dtype="bf16", seed=320, gate_scale=5.0)
    raw.k_raw[5, 1] = 0
    raw.k_raw[170, 0] = 0
    raw.q_raw[9, 0] = 0
    bits = workloads.bf16_bits
    raw.g[40, 0] = bits(np.array(-100.0))
    raw.g[200, 1] = bits(np.array(-80.0))
    o, _ = _run("zero rows, gate floor", raw, want_o=True)
    assert not to_np(o)[9, 0].any()


def test_replay_raw_against_front_end_then_replay():
    """Against the two-call path (gdn_front_end, then gdn_replay): both
    compute the same composition, but the two-call path rounds the
    normalised q, k and the gates to bf16 in between (half a bf16 unit per
    element), which moves its results by a few 1e-3 of their norm; the
    fused call skips that rounding and stays at the replay's own rounding
    level against the exact composition."""
    gdn, torch = _gdn()
    raw = workloads.generate_raw([1000, 300], H=4, dk=128, dv=128, dtype="bf16", seed=330)
    cu = torch.from_numpy(raw.cu_seqlens).cuda()
    o1, S1 = gdn.replay_raw(_t(raw.q_raw), _t(raw.k_raw), _t(raw.v), _t(raw.g), _t(raw.b), cu, want_o=True)
    q, k, a, b = gdn.front_end(_t(raw.q_raw), _t(raw.k_raw), _t(raw.g), _t(raw.b))
    o2, S2 = gdn.replay(q, k, _t(raw.v), a, b, cu, want_o=True)
    torch.cuda.synchronize()
    o_ref, S_ref = _oracle(raw, None, True)
    e_fused = max(rel(to_np(o1), o_ref), rel(to_np(S1), S_ref))
    e_two = max(rel(to_np(o2), o_ref), rel(to_np(S2), S_ref))
    gap = max(rel(to_np(o1), to_np(o2)), rel(to_np(S1), to_np(S2)))
    print("against the exact composition: fused %.2e, two calls %.2e; fused vs two calls %.2e"
          % (e_fused, e_two, gap), flush=True)
    assert e_fused <= 1e-4 and e_fused <= 0.1 * e_two
    assert gap <= 1e-2
