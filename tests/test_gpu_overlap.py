"""A replay beside a host-to-device copy on another stream.

The Tail-Replay page (section 3) overlaps the transfer of the attention
layers' cached keys and values with the replay, on a copy stream that is
waited for only before the query's forward.  The calls only launch on the
caller's stream, so the replay's results must not depend on the copy: the
overlapped replay equals the serial one bit for bit, and the copy lands
whole.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_helpers import dev

pytestmark = pytest.mark.gpu


def test_replay_beside_pinned_copy():
    import torch
    assert torch.cuda.is_available()
    import gated_deltanet_state_amd as gdn
    inp = workloads.generate([1500, 700], H=4, dk=128, dv=128, dtype="bf16", seed=121)
    d = dev(inp)
    n = 16 << 20
    host = torch.empty(n, dtype=torch.uint8, pin_memory=True)
    host.copy_(torch.from_numpy(np.random.Generator(np.random.PCG64(122)).integers(0, 256, n, dtype=np.uint8)))
    dst = torch.zeros(n, dtype=torch.uint8, device="cuda")
    o_ref, S_ref = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], want_o=True)
    torch.cuda.synchronize()
    comp = torch.cuda.current_stream()
    copy = torch.cuda.Stream()
    for it in range(3):
        dst.zero_()
        start = torch.cuda.Event()
        start.record(comp)
        copy.wait_event(start)
        with torch.cuda.stream(copy):
            dst.copy_(host, non_blocking=True)
        done = torch.cuda.Event()
        done.record(copy)
        o, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], want_o=True)
        comp.wait_event(done)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref) and torch.equal(S, S_ref), "overlapped replay %d differs" % it
        assert torch.equal(dst.cpu(), host), "copy %d incomplete" % it
