"""Plant plausible mistakes in copies of the oracle (on the CPU only) and
check that the pins catch every one of them.

Each mutant is a textual edit of gdn_oracle.c (the recurrence) or of the
package's __init__.py (the numpy front end and scalar-decay functions) in a
copy in a temporary directory; the real oracle is never touched.
"""
import importlib.util
import os
import shutil
import sys

import pytest

from tests.oracle_pins import ALL_PINS

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

MUTANTS = {
    # wrong sign of the delta-rule correction
    "delta_sign": ("double delta = beta * (v[i] - alpha * y);",
                   "double delta = beta * (v[i] + alpha * y);"),
    # the gate dropped from the read of the old state
    "drop_alpha_in_read": ("double delta = beta * (v[i] - alpha * y);",
                           "double delta = beta * (v[i] - y);"),
    # the gate not applied to the kept state
    "no_decay": ("row[j] = alpha * row[j] + delta * k[j];",
                 "row[j] = row[j] + delta * k[j];"),
    # output read from the wrong side (transposed state) -- only differs for dk != dv
    "o_before_update": (
        "token_update(S, dk, dv, k + th * dk, v + th * dv, alpha[th], beta[th]);\n"
        "      if (o) state_times(S, dk, dv, q + th * dk, o + th * dv);",
        "if (o) state_times(S, dk, dv, q + th * dk, o + th * dv);\n"
        "      token_update(S, dk, dv, k + th * dk, v + th * dv, alpha[th], beta[th]);"),
    # transition product taken in reverse (anti-chronological) order
    "operator_reversed": (
        "for (int j = 0; j < dk; ++j) acc += P[(size_t)i * dk + j] * kt[j];",
        "for (int j = 0; j < dk; ++j) acc += P[(size_t)j * dk + i] * kt[j];"),
    # the transition's gate dropped
    "operator_no_gate": (
        "P[(size_t)i * dk + j] = a * (P[(size_t)i * dk + j] - b * y[i] * kt[j]);",
        "P[(size_t)i * dk + j] = (P[(size_t)i * dk + j] - b * y[i] * kt[j]);"),
    # composition with the operator on the wrong side
    "compose_transposed": (
        "acc += S[(size_t)i * dk + m] * T[(size_t)m * dk + j];",
        "acc += S[(size_t)i * dk + m] * T[(size_t)j * dk + m];"),
    # local state dropped in the composition
    "compose_no_local": ("double acc = L[(size_t)i * dk + j];", "double acc = 0.0;"),
}


PY_MUTANTS = {
    # the norm's square root dropped
    "front_no_sqrt": ("n = np.sqrt(np.sum(x * x, axis=-1, keepdims=True))",
                      "n = np.sum(x * x, axis=-1, keepdims=True)"),
    # sigmoid of the negated logit
    "front_sigmoid_sign": ("1.0 / (1.0 + np.exp(-_f64(b)))", "1.0 / (1.0 + np.exp(_f64(b)))"),
    # decay from the negated log-gate
    "front_gate_sign": ("np.exp(_f64(g)), 1.0", "np.exp(-_f64(g)), 1.0"),
    # the scalar decay not applied to the kept state
    "scalar_no_decay": ("SL[c] = a[t][:, None, None] * SL[c] + b[t]", "SL[c] = SL[c] + b[t]"),
    # the write strength dropped
    "scalar_no_beta": ("+ b[t][:, None, None] * v[t]", "+ v[t]"),
    # gamma as a sum instead of a product
    "scalar_gamma_sum": ("gamma[c] *= a[t]", "gamma[c] += a[t] - 1"),
    # composition without the decay of the incoming state
    "scalar_compose_no_decay": ("S = g[c][:, None, None] * S + SL[c]", "S = S + SL[c]"),
    # the error measure as a difference of norms instead of the norm of the difference
    "rel_fro_norm_difference": ("num = float(np.linalg.norm((x - ref).ravel()))",
                                "num = abs(float(np.linalg.norm(x.ravel())) - den)"),
    # the error measure not divided by the reference norm
    "rel_fro_absolute": ("return num / den if den > 0 else num", "return num"),
    # per-block errors divided by the whole tensor's norm
    "blocks_global_denominator": ("den = np.asarray(np.sqrt(np.sum(r * r, axis=-1)))",
                                  "den = np.full(num.shape, np.sqrt(np.sum(r * r)))"),
    # per-block errors with the floor ignored
    "blocks_no_floor": ("den = np.maximum(den, floor * np.sqrt(np.mean(den * den)))", "den = den"),
    # per-block errors reduced over the wrong axes (leading instead of trailing)
    "blocks_wrong_axes": ("lead = ref.shape[:ref.ndim - nred]", "lead = ref.shape[nred:]"),
}


def _load_mutant(tmp_path, name, old, new, fname="gdn_oracle.c"):
    d = tmp_path / ("oracle_" + name)
    shutil.copytree(os.path.join(ROOT, "oracle"), d,
                    ignore=shutil.ignore_patterns("*.so", "__pycache__", "*.tmp*"))
    src = (d / fname).read_text()
    assert src.count(old) == 1, name
    (d / fname).write_text(src.replace(old, new))
    modname = "oracle_mutant_" + name
    spec = importlib.util.spec_from_file_location(modname, d / "__init__.py")
    mod = importlib.util.module_from_spec(spec)
    sys.modules[modname] = mod
    spec.loader.exec_module(mod)
    mod.build(force=True)
    return mod


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_catch_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    mod = _load_mutant(tmp_path, name, old, new)
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no pin caught mutant %s" % name


@pytest.mark.parametrize("name", sorted(PY_MUTANTS))
def test_pins_catch_python_mutant(tmp_path, name):
    old, new = PY_MUTANTS[name]
    mod = _load_mutant(tmp_path, name, old, new, fname="__init__.py")
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            caught.append(pin.__name__)
    assert caught, "no pin caught mutant %s" % name
