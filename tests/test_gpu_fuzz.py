"""Seeded randomized parity of gdn_replay against the fp64 oracle.

Each case draws, from its own seed: 1 .. 8 sequences of 0 .. 300 tokens
(mostly 1 .. 300), 1 .. 4 heads, dk and dv from {64, 128}, the input dtype,
a start state or none, outputs or none (fp32 or bf16), a gate law (the
workload law, slow decay, alpha = 1, strong decay, strong decay with some
gates exactly 0), unit or non-unit keys, and for bf16 inputs the cost model
or a forced time split.  Every case must meet the bars of
tests/gpu_helpers.py (page "Tail-Replay: Escaping the Curse of Linear
Attention in Prefix Caching for Hybrid LLMs", section 2 Eq. (1)); the test
stops at the first case that does not and names it.
"""
import numpy as np
import pytest

import workloads
from tests.gpu_helpers import check_replay

pytestmark = pytest.mark.gpu

N_CASES = 48
LAWS = {
    "workload": dict(),
    "slow": dict(gate_scale=0.001),
    "alpha1": dict(alpha_one=True),
    "strong": dict(gate_scale=5.0),
    "strong+zeros": dict(gate_scale=5.0, alpha_zero_frac=0.03),
}


def draw_case(seed):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    n = int(rng.integers(1, 9))
    lengths = [int(x) if rng.uniform() > 0.1 else 0 for x in rng.integers(1, 301, size=n)]
    case = dict(
        lengths=lengths,
        H=int(rng.integers(1, 5)),
        dk=int(rng.choice([64, 128])),
        dv=int(rng.choice([64, 128])),
        dtype=str(rng.choice(["bf16", "f32"], p=[0.75, 0.25])),
        S0=bool(rng.uniform() < 0.4),
        want_o=bool(rng.uniform() < 0.6),
        o_bf16=bool(rng.uniform() < 0.25),
        law=str(rng.choice(sorted(LAWS))),
        key_scale=bool(rng.uniform() < 0.35),
        segments=None if rng.uniform() < 0.5 else int(rng.integers(1, 6)),
    )
    return case


def test_seeded_fuzz():
    import torch
    assert torch.cuda.is_available()
    for seed in range(N_CASES):
        c = draw_case(seed)
        label = "fuzz case %d %s" % (seed, c)
        print(label, flush=True)
        inp = workloads.generate(c["lengths"], H=c["H"], dk=c["dk"], dv=c["dv"], dtype=c["dtype"], seed=2000 + seed,
                                 key_scale=(0.5, 1.2) if c["key_scale"] else None, **LAWS[c["law"]])
        S0 = None
        if c["S0"]:
            rng = np.random.Generator(np.random.PCG64(3000 + seed))
            S0 = (rng.standard_normal((len(c["lengths"]), c["H"], c["dv"], c["dk"])) * 0.2).astype(np.float32)
            S0 = S0.astype(np.float64)
        check_replay("case %d" % seed, inp, S0=S0, want_o=c["want_o"],
                     o_dtype=torch.bfloat16 if c["o_bf16"] else None, segments=c["segments"])
