"""Helpers for the GPU tests: move seeded inputs to the device and compare
with the oracle.  Imported only by tests marked ``gpu``."""
import numpy as np

import oracle

TOL_F32 = 1e-5   # relative Frobenius error, fp32 inputs
TOL_BF16 = 3e-3  # relative Frobenius error, bf16 inputs with fp32 state


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
