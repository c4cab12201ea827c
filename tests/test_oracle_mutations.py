"""Plant plausible mistakes in a copy of the oracle's loop (and of its forced
replay) and check that the pins catch each one.  The mutants run on the CPU only;
the oracle module itself is never modified.
"""
import inspect
import json
import os

import numpy as np
import pytest

import oracle as O
import oracle.gptq2d as Q2
import oracle.gptq_oracle as G
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")

# (function, original text, planted text)
MUTANTS = {
    "no_divide_by_U_jj": ("gptq_quantize", "Eb[:, done] = (w - dequant(c, s, z)) / U[j, j]",
                          "Eb[:, done] = (w - dequant(c, s, z))"),
    "error_scaled_by_U_jj_squared": ("gptq_quantize", "Eb[:, done] = (w - dequant(c, s, z)) / U[j, j]",
                                     "Eb[:, done] = (w - dequant(c, s, z)) / U[j, j] ** 2"),
    "wrong_sign_in_block": ("gptq_quantize", "return Wr[:, k0:k1] - Eb[:, :done] @ U[b0:b0 + done, k0:k1]",
                            "return Wr[:, k0:k1] + Eb[:, :done] @ U[b0:b0 + done, k0:k1]"),
    "transposed_U_in_block": ("gptq_quantize", "return Wr[:, k0:k1] - Eb[:, :done] @ U[b0:b0 + done, k0:k1]",
                              "return Wr[:, k0:k1] - Eb[:, :done] @ U[k0:k1, b0:b0 + done].T"),
    "in_block_skips_previous_column": (
        "gptq_quantize", "return Wr[:, k0:k1] - Eb[:, :done] @ U[b0:b0 + done, k0:k1]",
        "return Wr[:, k0:k1] - Eb[:, :max(done - 1, 0)] @ U[b0:b0 + max(done - 1, 0), k0:k1]"),
    "dropped_out_of_block_update": ("gptq_quantize", "        Wr[:, b1:] -= Eb @ U[b0:b1, b1:]\n",
                                    "        pass\n"),
    "out_of_block_uses_U_transpose": ("gptq_quantize", "        Wr[:, b1:] -= Eb @ U[b0:b1, b1:]\n",
                                      "        Wr[:, b1:] -= Eb @ U[b1:, b0:b1].T\n"),
    "group_grid_from_stale_weights": ("gptq_quantize",
                                      "set_grid(gi, current(j, min(j + g, d_col), done))",
                                      "set_grid(gi, Wr[:, j:min(j + g, d_col)])"),
    "zero_replay_tie_at_integer": ("_replay_zero", "tie = np.minimum(rz[diff], z[diff]) + 0.5",
                                   "tie = np.minimum(rz[diff], z[diff])"),
    "code_replay_tie_at_integer": ("_replay_code", "tie = np.minimum(rc[diff], c[diff]) - z[diff] + 0.5",
                                   "tie = np.minimum(rc[diff], c[diff]) - z[diff]"),
}


def _mutant(name):
    """gptq_quantize with one planted mistake in it or in a helper it calls."""
    fn, old, new = MUTANTS[name]
    src = inspect.getsource(getattr(G, fn))
    assert src.count(old) == 1, name
    ns = dict(vars(G))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    if fn != "gptq_quantize":   # re-bind the loop to the planted helper
        exec(compile(inspect.getsource(G.gptq_quantize), "<loop>", "exec"), ns)
    return ns["gptq_quantize"]


def _replay_pins_pass(fn):
    """Forced replay must adopt a supplied zero-point / code only at a tie."""
    from test_oracle_pins import zero_tie_case, code_tie_case
    w, U, bits, g, B, zrow, z_adopt, z_reject = zero_tie_case()
    try:
        fn(w, U, bits, g, B, replay_zeros=z_reject)
        return False
    except O.ReplayMismatch:
        pass
    try:
        r = fn(w, U, bits, g, B, replay_zeros=z_adopt)
    except O.ReplayMismatch:
        return False
    if r.adopted_zeros != 1 or not np.array_equal(r.zeros, z_adopt):
        return False
    w, U, bits, B, codes_adopt, codes_reject = code_tie_case()
    try:
        fn(w, U, bits, 0, B, replay_codes=codes_reject)
        return False
    except O.ReplayMismatch:
        pass
    try:
        r = fn(w, U, bits, 0, B, replay_codes=codes_adopt)
    except O.ReplayMismatch:
        return False
    return r.adopted_codes >= 1


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
    # groups of 2 inside blocks of 4 (parameters from the in-block updated weights)
    codes, _ = O.obq_fixed_order(w, H_lam, 3, 2, "inverse")
    if not np.array_equal(fn(w, U, 3, 2, 4).codes, codes):
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
    return _replay_pins_pass(fn)


def test_unmutated_loop_passes_the_pins():
    assert _pins_pass(G.gptq_quantize)


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_each_planted_mistake_is_caught(name):
    assert not _pins_pass(_mutant(name))


# ---------------------------------------------------------------- GPTQ-2D replay
MUTANTS_2D = {
    "tie_test_at_integer": ("near = abs(abs(t - np.floor(t)) - 0.5) <= replay_tol",
                            "near = abs(t - np.floor(t)) <= replay_tol"),
    "adopts_without_tie_test": ("if not (near and int(replay_codes[i, j]) in cand):",
                                "if not (int(replay_codes[i, j]) in cand):"),
}


def _mutant_2d(name):
    old, new = MUTANTS_2D[name]
    src = inspect.getsource(Q2.gptq2d)
    assert src.count(old) == 1, name
    ns = dict(vars(Q2))
    exec(compile(src.replace(old, new), "<mutant>", "exec"), ns)
    return ns["gptq2d"]


def _pins_2d_pass(fn):
    from test_oracle_gptq2d import tie_case_2d
    X, U_Q, U_P, bits, adopt, reject = tie_case_2d()
    try:
        r = fn(X, U_Q, U_P, bits, replay_codes=adopt)
    except O.ReplayMismatch:
        return False
    if r.adopted_codes != 1:
        return False
    try:
        fn(X, U_Q, U_P, bits, replay_codes=reject)
        return False
    except O.ReplayMismatch:
        return True


def test_unmutated_2d_replay_passes_the_pins():
    assert _pins_2d_pass(Q2.gptq2d)


@pytest.mark.parametrize("name", sorted(MUTANTS_2D))
def test_each_planted_2d_replay_mistake_is_caught(name):
    assert not _pins_2d_pass(_mutant_2d(name))
