"""Planted mistakes in the oracle must fail its pins.

Each mutant is a one-token edit of ``oracle/kda_oracle.c`` (a dropped term, a
wrong sign, a wrong operand or index, a wrong clamp bound), compiled on the CPU
into a temporary library and run through every pin check.  A mutant that no
check catches would mean the pins do not constrain that part of the oracle.
"""
import functools
import os
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_pins as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "kda_oracle.c")

MUTANTS = {
    "no_forget": ("S[i * nc + j] *= alpha[i];", ";"),
    "delta_sign": ("((double)vt[cols[c0 + j]] - w[j])", "((double)vt[cols[c0 + j]] + w[j])"),
    "no_beta": ("u[j] = bt * (", "u[j] = ("),
    "predict_with_q": ("w[j] += (double)kt[i] * S[i * nc + j];", "w[j] += (double)qt[i] * S[i * nc + j];"),
    "write_with_q": ("S[i * nc + j] += (double)kt[i] * u[j];", "S[i * nc + j] += (double)qt[i] * u[j];"),
    "readout_with_k": ("ot[j] += (double)qt[i] * S[i * nc + j];", "ot[j] += (double)kt[i] * S[i * nc + j];"),
    "lower_clamp": ("if (x < -5.0) x = -5.0;", "if (x < -6.0) x = -6.0;"),
    "no_upper_clamp": ("if (x > 0.0) x = 0.0;", ";"),
    "gate_not_exp": ("return exp(x);", "return 1.0 + x;"),
    "value_column_index": ("vt[cols[c0 + j]]", "vt[c0 + j]"),
    "ignore_s0": ("S[i * nc + j] = s0 ? s0[((n * H + h) * Dk + i) * Dv + cols[c0 + j]] : 0.0;",
                  "S[i * nc + j] = 0.0;"),
    "s0_transposed": ("s0[((n * H + h) * Dk + i) * Dv + cols[c0 + j]]", "s0[((n * H + h) * Dv + cols[c0 + j]) * Dk + i]"),
    "decay_by_value_channel": ("S[i * nc + j] *= alpha[i];", "S[i * nc + j] *= alpha[j % Dk];"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, tmp_path):
    src = open(SRC).read()
    old, new = MUTANTS[name]
    assert src.count(old) >= 1, f"mutation site for {name} not found"
    c = tmp_path / f"{name}.c"
    c.write_text(src.replace(old, new))
    so = tmp_path / f"{name}.so"
    subprocess.run(["gcc", "-O1", "-fopenmp", "-fPIC", "-shared", "-std=c11", str(c), "-o", str(so), "-lm"],
                   check=True)
    fwd = functools.partial(oracle.forward, _lib=oracle.load(str(so)))
    caught = []
    for check in pins.ALL_CHECKS:
        try:
            check(fwd=fwd)
        except (AssertionError, RuntimeError, ValueError):
            caught.append(check.__name__)
    assert caught, f"no pin catches mutant {name}"
