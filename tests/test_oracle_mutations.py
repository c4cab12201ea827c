"""Plant plausible mistakes in a copy of the oracle's loop and check that the pins
catch each one.  The mutants run on the CPU only; the oracle module itself is
never modified.
"""
import inspect
import json
import os

import numpy as np
import pytest

import oracle as O
import oracle.gptq_oracle as G
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")

MUTANTS = {
    "no_divide_by_U_jj": ("e = (w - q) / Ub[j, j]", "e = (w - q)"),
    "wrong_sign_in_block": ("W1[:, j:] -= np.outer(e, Ub[j, j:])",
                            "W1[:, j:] += np.outer(e, Ub[j, j:])"),
    "transposed_U_in_block": ("W1[:, j:] -= np.outer(e, Ub[j, j:])",
                              "W1[:, j:] -= np.outer(e, Ub[j:, j])"),
    "update_skips_next_column": ("W1[:, j:] -= np.outer(e, Ub[j, j:])",
                                 "W1[:, j + 2:] -= np.outer(e, Ub[j, j + 2:])"),
    "dropped_out_of_block_update": ("        W[:, i2:] -= E @ U[i1:i2, i2:]\n", "        pass\n"),
    "out_of_block_uses_U_transpose": ("        W[:, i2:] -= E @ U[i1:i2, i2:]\n",
                                      "        W[:, i2:] -= E @ U[i2:, i1:i2].T\n"),
    "error_not_divided_stored": ("            E[:, j] = e\n", "            E[:, j] = e * Ub[j, j]\n"),
}


def _mutant(name):
    old, new = MUTANTS[name]
    src = inspect.getsource(G.gptq_quantize)
    assert src.count(old) == 1, name
    ns = dict(vars(G))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["gptq_quantize"]


def _pins_pass(fn):
    """The loop pins from test_oracle_pins, against an arbitrary implementation."""
    with open(os.path.join(GOLD, "hand_example_4col.json")) as f:
        g = json.load(f)
    r = fn(np.array(g["W0"]), np.array(g["U"]), g["bits"], 0, 2)
    if not np.array_equal(r.codes, g["codes"]):
        return False
    if not np.isclose(r.err_sq_sum, np.sum(np.square(g["E"])), rtol=1e-12):
        return False
    w, x = wl.tiny_case(5, 6, 8, 64, 0.8)
    H_lam, lam = O.damp(O.hessian([x]), 0.01)
    U = O.inv_hessian_factor(H_lam)
    for bits in (2, 3, 4):
        codes, _ = O.obq_fixed_order(w, H_lam, bits, 0, "inverse")
        if not np.array_equal(fn(w, U, bits, 0, 3).codes, codes):
            return False
    w, x = wl.tiny_case(11, 20, 70, 200, 0.8)
    H_lam, lam = O.damp(O.hessian([x]), 0.01)
    U = O.inv_hessian_factor(H_lam)
    r1, r2 = fn(w, U, 4, 0, 1), fn(w, U, 4, 0, 16)
    if not np.array_equal(r1.codes, r2.codes):
        return False
    D = w - r2.w_hat
    if not np.isclose(0.5 * r2.err_sq_sum, 0.5 * np.sum((D @ H_lam) * D), rtol=1e-9):
        return False
    return True


def test_unmutated_loop_passes_the_pins():
    assert _pins_pass(G.gptq_quantize)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_planted_mistake_is_caught(name):
    assert not _pins_pass(_mutant(name))
