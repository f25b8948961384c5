"""The oracle's pins have teeth: plant plausible mistakes in a copy of the
oracle's C source (on the CPU), rebuild it, and check that the pin suite
rejects every mutant.  The real oracle is never modified."""
import os
import subprocess

import numpy as np
import pytest

import oracle
from oracle import oracle as oracle_mod
import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle_mod.__file__), "lora_oracle.c")

# (name, text in the source, replacement) -- each is a mistake a port could make.
MUTANTS = [
    ("drop_base", "yt[n] = yt[n] + s * d;", "yt[n] = s * d;"),
    ("drop_lora", "yt[n] = yt[n] + s * d;", "yt[n] = yt[n];"),
    ("sign", "yt[n] = yt[n] + s * d;", "yt[n] = yt[n] - s * d;"),
    ("scale_inverted", "const double s = alpha[i] / (double)r;", "const double s = (double)r / alpha[i];"),
    ("scale_no_rank", "const double s = alpha[i] / (double)r;", "const double s = alpha[i];"),
    ("W_transposed", "const double *wn = W + (size_t)n * d_in;\n            double acc = 0.0;\n            for (int k = 0; k < d_in; ++k)\n                acc += xt[k] * wn[k];",
     "double acc = 0.0;\n            for (int k = 0; k < d_in && k < d_out && n < d_in; ++k)\n                acc += xt[k] * W[(size_t)k * d_in + n];"),
    ("B_transposed", "d += h[j] * bn[j];", "d += h[j] * Bi[(size_t)j * d_out + n];"),
    ("wrong_slot", "int32_t i = idx[t];", "int32_t i = (idx[t] >= 0 && idx[t] + 1 < S) ? idx[t] + 1 : idx[t];"),
    ("base_only_gets_lora", "if (is_base_only)\n            continue;", "if (is_base_only)\n            i = 0;"),
    ("unstable_route", "perm[next[k]] = t;\n        next[k] += 1;", "perm[offsets[k] + counts[k] - 1 - (next[k] - offsets[k])] = t;\n        next[k] += 1;"),
    ("theta_ge", "(counts[k] > theta)", "(counts[k] >= theta)"),
    ("inactive_is_base", "    return S + 1;\n}", "    return (idx >= 0 && idx < S) ? S : S + 1;\n}"),
]

PIN_TESTS = [
    pins.test_apply_worked_example,
    pins.test_apply_selection_matrix_base,
    pins.test_apply_one_hot_adapter_closed_form,
    pins.test_apply_base_only_is_library_matmul,
    pins.test_apply_exact_rational_small_integers,
    pins.test_linear_in_alpha_and_base_untouched,
    pins.test_invalid_tokens_are_nan_and_counted,
    pins.test_route_worked_example,
    lambda: pins.test_route_matches_numpy_stable_sort("random0"),
    lambda: pins.test_route_modes(0, 4, [2, 1, 0]),
]


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new, tmp_path, monkeypatch):
    src = open(SRC).read()
    assert src.count(old) >= 1, "mutation anchor not found: " + name
    mutated = src.replace(old, new, 1)
    c = tmp_path / "mut.c"
    c.write_text(mutated)
    so = tmp_path / "libmut.so"
    subprocess.run(["gcc", "-std=c99", "-O1", "-fopenmp", "-fPIC", "-shared", "-w",
                    "-o", str(so), str(c), "-lm"], check=True)
    monkeypatch.setattr(oracle_mod, "_lib", None)
    monkeypatch.setattr(oracle_mod, "LIB_PATH", str(so))
    caught = 0
    for fn in PIN_TESTS:
        try:
            fn()
        except Exception:
            caught += 1
    assert caught > 0, "no pin rejects mutant " + name
