"""GPU parity at the edges of the supported sizes.

- the largest head count (65536): every head is an independent workgroup,
  and 32-bit in-chunk byte offsets span 63 tokens of 65536 heads;
- a long packed sequence (300,001 tokens, with outputs): the time split with
  outputs (three passes) over thousands of chunks, a ragged last chunk.

Checked against the fp64 oracle (page "Tail-Replay: Escaping the Curse of
Linear Attention in Prefix Caching for Hybrid LLMs", section 2 Eq. (1)) at
the bf16 tolerance: on sampled heads for the head count, on every output
for the long sequence.
"""
import pytest

import workloads
from tests.gpu_helpers import check_out, check_state, dev, oracle_replay, to_np

pytestmark = pytest.mark.gpu


def _gdn():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    return gdn, torch


def test_largest_head_count():
    gdn, torch = _gdn()
    H = 65536
    inp = workloads.generate([3, 70], H=H, dk=64, dv=64, dtype="bf16", seed=91)
    d = dev(inp)
    o, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], want_o=True)
    torch.cuda.synchronize()
    heads = [0, 1, 12345, 40000, H - 1]
    o_ref, S_ref = oracle_replay(inp, heads=heads)
    check_out("H=%d o heads %s" % (H, heads), to_np(o[:, heads]), o_ref, "bf16")
    check_state("H=%d S_final heads %s" % (H, heads), to_np(S[:, heads]), S_ref, "bf16")


def test_long_sequence_with_outputs():
    gdn, torch = _gdn()
    inp = workloads.generate([300001], H=2, dk=64, dv=64, dtype="bf16", seed=92, gate_scale=0.01)
    d = dev(inp)
    o, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], want_o=True)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle_replay(inp)
    check_out("T=300001 o", to_np(o), o_ref, "bf16")
    check_state("T=300001 S_final", to_np(S), S_ref, "bf16")
