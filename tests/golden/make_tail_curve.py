"""Write tests/golden/tail_curve.json: the fp64 oracle's tail-replay state
error as a function of the replayed fraction (calls only oracle/ and the
input generator; run from the repository root: python tests/golden/make_tail_curve.py).

Sources:
- "Tail-Replay: Escaping the Curse of Linear Attention in Prefix Caching for
  Hybrid LLMs", section 3 (Independent Tail-Replay): the state at the end of
  an m-token matched prefix is rebuilt by replaying only its latest k tokens
  from a zero state.
- "LinearKV: One Cached State Suffices for Position-Independent Caching in
  Hybrid LLMs", the probe of a constructed state against the full-prefix
  state (Figure 3 discussion): relative Frobenius error
  ||S_tail - S_full|| / ||S_full||.

Bound (from the affine chunk operator of the LinearKV page, applied to the
tail as one chunk): S_full = S_head T_tail + S_tail exactly, with S_head the
state after the first m - k tokens, so ||S_full - S_tail|| = ||S_head T_tail||.
Each factor alpha_t (I - beta_t k_t k_t^T) of T_tail has spectral norm at most
alpha_t when 0 <= beta_t ||k_t||^2 <= 2, hence per head
||S_full - S_tail||_F <= ||S_head||_F prod_tail alpha_t; the stored bound is
sqrt(sum_h (||S_head,h||_F prod_tail alpha_h)^2) / ||S_full||_F.

Inputs: the 32768-token, 32-head, d = 128 bf16 prefill inputs (seed 3) with the
workload gate law alpha = exp(-0.1 softplus(x)), and the same draw with the
slow law alpha = exp(-0.001 softplus(x)) as a supplement (the workload law
forgets the head of the prefix within a few hundred tokens, so its 5% and 10%
points are exactly zero in real arithmetic).
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402

M = workloads.TAIL_CURVE_M
KS = workloads.TAIL_CURVE_KS
LAWS = workloads.TAIL_CURVE_LAWS
OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tail_curve.json")


def curve(inp, ks=KS):
    """Oracle tail errors and bounds for every tail length in ks (one sequence)."""
    f = inp.f64
    k, v, a, b = (f[n] for n in ("k", "v", "alpha", "beta"))
    m = k.shape[0]
    # states after m - k tokens for every k, by split resumption, then the full state
    heads_S = {}
    S, t = None, 0
    for kk in sorted(ks, reverse=True):
        e = m - kk
        _, S = oracle.replay(None, k[t:e], v[t:e], a[t:e], b[t:e], [0, e - t], S0=S, want_o=False)
        heads_S[kk], t = S, e
    _, S_full = oracle.replay(None, k[t:], v[t:], a[t:], b[t:], [0, m - t], S0=S, want_o=False)
    # every tail from zero, packed in one call
    cu = np.concatenate([[0], np.cumsum(ks)]).astype(np.int32)
    cat = lambda x: np.concatenate([x[m - kk:] for kk in ks])  # noqa: E731
    _, S_tail = oracle.replay(None, cat(k), cat(v), cat(a), cat(b), cu, want_o=False)
    full_norm = float(np.linalg.norm(S_full))
    out = {"err": [], "bound": [], "err_per_head": []}
    for i, kk in enumerate(ks):
        d = S_tail[i] - S_full[0]
        out["err"].append(float(np.linalg.norm(d)) / full_norm)
        out["err_per_head"].append([float(np.linalg.norm(d[h]) / np.linalg.norm(S_full[0, h]))
                                    for h in range(d.shape[0])])
        prod_a = np.exp(np.sum(np.log(a[m - kk:]), axis=0))                   # [H]
        hn = np.linalg.norm(heads_S[kk][0].reshape(d.shape[0], -1), axis=1)   # [H]
        out["bound"].append(float(np.sqrt(np.sum((hn * prod_a) ** 2))) / full_norm)
    return out


def main():
    res = {
        "source": ("Tail-Replay (section 3, Independent Tail-Replay: replay the latest k tokens of an m-token "
                   "prefix from zero) and LinearKV (relative state error against the full-prefix state, "
                   "Figure 3 discussion); bound from the affine chunk operator, see make_tail_curve.py"),
        "generated_by": "tests/golden/make_tail_curve.py (fp64 oracle only)",
        "inputs": "workloads.tail_curve_inputs(law): generate([32768], H=32, dk=128, dv=128, dtype='bf16', seed=3, gate_scale=c)",
        "m": M, "k": KS, "fraction": [kk / M for kk in KS], "laws": {},
    }
    for law, c in LAWS.items():
        r = curve(workloads.tail_curve_inputs(law))
        r["gate_scale"] = c
        res["laws"][law] = r
        print(law, " ".join("%d:%.2e" % (kk, e) for kk, e in zip(KS, r["err"])), flush=True)
    with open(OUT, "w") as fh:
        json.dump(res, fh, indent=1)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
