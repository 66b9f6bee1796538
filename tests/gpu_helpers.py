"""Helpers for the GPU tests: move seeded inputs to the device, run the
library through its binding and compare with the oracle.  Imported only by
tests marked ``gpu``.

Every comparison asserts two kinds of bar against the fp64 oracle:
  * the contract: the relative Frobenius error over the whole output tensor
    (<= 1e-5 for fp32 inputs, <= 3e-3 for bf16 inputs with an fp32 state);
  * element-level bars that a localised mistake cannot hide under: the worst
    relative error of any one (sequence, head) state, (chunk, head) operator
    or (token, head) output row (oracle.rel_fro_blocks).  Output rows are
    measured against max(|row|, ROW_FLOOR x the root mean square row norm):
    the first rows of a sequence can be tiny next to the rest while the
    kernel's rounding scales with the state.  The element bars sit five to
    ten times above the worst errors measured on MI355X over every GPU test
    and the seeded fuzz (bf16 inputs: states 1.1e-5, rows 9.8e-5; fp32
    inputs: states 7.7e-6, rows 3.3e-5, both under the strong-decay law,
    where the fp32 cumulative log-gates of a chunk reach |g| ~ 400 and their
    rounding sets the decays' relative accuracy near 1e-5), so one wrong
    row, tile or chunk fails them by orders of magnitude.
"""
import numpy as np

import oracle

TOL_F32 = 1e-5   # relative Frobenius error, whole tensor, fp32 inputs
TOL_BF16 = 3e-3  # relative Frobenius error, whole tensor, bf16 inputs with fp32 state
BLOCK_TOL = {"f32": 5e-5, "bf16": 1e-4}   # worst (sequence, head) state / (chunk, head) operator
ROW_TOL = {"f32": 3e-4, "bf16": 1e-3}     # worst (token, head) output row
ROW_FLOOR = 0.05
BF16_UNIT_ROUNDOFF = 2.0 ** -8            # relative error of rounding to bf16 (outputs stored in bf16)


def tol_for(inp):
    return TOL_F32 if inp.dtype == "f32" else TOL_BF16


def dev(inp, device="cuda:0"):
    """Device tensors for an Inputs batch (bf16 via their bit patterns)."""
    import torch

    def t(a):
        if inp.dtype == "bf16":
            return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(device)
        return torch.from_numpy(np.ascontiguousarray(a)).to(device)
    return dict(q=t(inp.q), k=t(inp.k), v=t(inp.v), alpha=t(inp.alpha), beta=t(inp.beta),
                cu=torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(device))


def oracle_replay(inp, S0=None, want_o=True, heads=None):
    """Oracle on all heads, or on the listed heads only (heads are independent)."""
    f = inp.f64
    sel = slice(None) if heads is None else list(heads)
    S0s = None if S0 is None else np.asarray(S0)[:, sel]
    return oracle.replay(f["q"][:, sel], f["k"][:, sel], f["v"][:, sel], f["alpha"][:, sel],
                         f["beta"][:, sel], inp.cu_seqlens, S0=S0s, want_o=want_o)


def rel(x, ref):
    return oracle.rel_fro(np.asarray(x, np.float64), ref)


def to_np(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def check_close(label, got, ref, nred, whole_tol, block_tol, floor=0.0):
    """Assert the whole-tensor and the worst per-block relative error."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (label, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "%s: non-finite values" % label
    whole = oracle.rel_fro(got, ref)
    blocks = oracle.rel_fro_blocks(got, ref, nred, floor)
    worst = float(blocks.max()) if blocks.size else 0.0
    where = tuple(int(i) for i in np.unravel_index(int(np.argmax(blocks)), blocks.shape)) if blocks.size else ()
    print("%s: whole %.2e (bar %.0e), worst block %.2e at %s (bar %.0e)"
          % (label, whole, whole_tol, worst, where, block_tol), flush=True)
    assert whole <= whole_tol, "%s: whole-tensor error %.3e > %.1e" % (label, whole, whole_tol)
    assert worst <= block_tol, "%s: block %s error %.3e > %.1e" % (label, where, worst, block_tol)
    return whole, worst


def check_state(label, S, S_ref, dtype, whole_tol=None, block_tol=None):
    """States [..., dv, dk]: one block per leading index (sequence, head)."""
    whole = (TOL_F32 if dtype == "f32" else TOL_BF16) if whole_tol is None else whole_tol
    return check_close(label, S, S_ref, 2, whole, BLOCK_TOL[dtype] if block_tol is None else block_tol)


def check_out(label, o, o_ref, dtype, o_bf16=False, whole_tol=None, row_tol=None):
    """Outputs [T, H, dv]: one block per (token, head) row.  Outputs stored in
    bf16 carry their own rounding on top (at most 2^-8 of each element, so of
    each row)."""
    whole = (TOL_F32 if dtype == "f32" else TOL_BF16) if whole_tol is None else whole_tol
    row = ROW_TOL[dtype] if row_tol is None else row_tol
    if o_bf16:
        whole, row = max(whole, TOL_BF16), row + BF16_UNIT_ROUNDOFF
    return check_close(label, o, o_ref, 1, whole, row, floor=ROW_FLOOR)


def run_replay(inp, S0=None, want_o=True, o_dtype=None, segments=None):
    """One replay of an Inputs batch on cuda:0; returns numpy float64 (o or None, S)."""
    import torch
    import gated_deltanet_state_amd as gdn
    d = dev(inp)
    S0_t = None if S0 is None else torch.from_numpy(np.asarray(S0, np.float32)).cuda()
    o, S = gdn.replay(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["cu"], S0=S0_t,
                      want_o=want_o, o_dtype=o_dtype, segments=segments)
    torch.cuda.synchronize()
    return (None if o is None else to_np(o)), to_np(S)


def check_replay(label, inp, S0=None, want_o=True, o_dtype=None, segments=None):
    """Replay on the GPU and the oracle; assert every bar.  Returns (o, S)."""
    import torch
    o, S = run_replay(inp, S0=S0, want_o=want_o, o_dtype=o_dtype, segments=segments)
    o_ref, S_ref = oracle_replay(inp, S0=S0, want_o=want_o)
    check_state(label + " S_final", S, S_ref, inp.dtype)
    if want_o:
        check_out(label + " o", o, o_ref, inp.dtype, o_bf16=o_dtype == torch.bfloat16)
    return o, S
