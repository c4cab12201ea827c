"""Pins of the oracle's act-order (wiki "GPTQ", section "실무 변형": quantize the
columns with the largest Hessian diagonal first; with groups a column-to-group
map is needed).  CPU only."""
import numpy as np
import pytest

import oracle as O
import workloads as wl


def _case(seed, d_row, d_col, n=96, corr=0.8):
    w, x = wl.tiny_case(seed, d_row, d_col, n, corr)
    # give the columns clearly different scales so the order is not the identity
    rng = np.random.default_rng(seed + 1)
    x = x * rng.uniform(0.3, 3.0, d_col)[None, :]
    return w, x


def test_perm_hand_example_ties_and_nan():
    H = np.diag([1.0, 3.0, 3.0, 2.0, np.nan, 3.0])
    np.testing.assert_array_equal(O.act_order_perm(H), [1, 2, 5, 3, 0, 4])
    # compared in H's own precision: equal in fp32, different in fp64
    H64 = np.diag([1.0, 1.0 + 1e-9])
    np.testing.assert_array_equal(O.act_order_perm(H64), [1, 0])
    np.testing.assert_array_equal(O.act_order_perm(H64.astype(np.float32)), [0, 1])


@pytest.mark.parametrize("group,B", [(0, 16), (8, 4), (8, 16)])
def test_descending_diagonal_gives_natural_order(group, B):
    """When diag(H) already decreases, act-order is the natural order, bitwise."""
    w, x = _case(3, 12, 40)
    perm0 = O.act_order_perm(O.hessian([x]))
    w2, x2 = w[:, perm0], x[:, perm0]
    H2 = O.hessian([x2])
    np.testing.assert_array_equal(O.act_order_perm(H2), np.arange(40))
    a = O.solve_layer_act_order(w2, [x2], 4, group, B)
    b = O.solve_layer(w2, [x2], 4, group, B)
    np.testing.assert_array_equal(a.result.codes, b.result.codes)
    np.testing.assert_array_equal(a.result.w_hat, b.result.w_hat)
    np.testing.assert_array_equal(a.result.scales, b.result.scales)
    np.testing.assert_array_equal(a.result.g_idx, np.arange(40) // (group or 40))
    assert a.err == b.err


@pytest.mark.parametrize("group,B", [(0, 8), (4, 4), (8, 4)])
def test_feature_permutation_equivariance(group, B):
    """Renaming the input features renames the result: the order follows the
    diagonal, not the column index."""
    w, x = _case(5, 10, 32)
    Q = np.random.default_rng(9).permutation(32)
    a = O.solve_layer_act_order(w, [x], 3, group, B)
    b = O.solve_layer_act_order(w[:, Q], [x[:, Q]], 3, group, B)
    np.testing.assert_array_equal(b.result.codes, a.result.codes[:, Q])
    np.testing.assert_array_equal(b.result.g_idx, a.result.g_idx[Q])
    np.testing.assert_allclose(b.result.w_hat, a.result.w_hat[:, Q], rtol=0, atol=1e-12)
    np.testing.assert_allclose(b.result.scales, a.result.scales, rtol=1e-12, atol=0)
    assert b.err == pytest.approx(a.err, rel=1e-10)


@pytest.mark.parametrize("group", [0, 8])
def test_diagonal_hessian_is_rtn_in_that_order(group):
    """No compensation with a diagonal H: act-order GPTQ is RTN over the columns
    taken in descending-diagonal order (groups formed in that order)."""
    rng = np.random.default_rng(21)
    w = 0.02 * rng.standard_normal((16, 48))
    H = np.diag(rng.uniform(0.5, 5.0, 48))
    perm = O.act_order_perm(H)
    U = O.inv_hessian_factor(O.damp(H[np.ix_(perm, perm)])[0])
    r = O.gptq_quantize_act_order(w, U, perm, 4, group, 16)
    rc, rw = O.rtn(w[:, perm], 4, group)
    inv = np.argsort(perm)
    np.testing.assert_array_equal(r.codes, rc[:, inv])
    np.testing.assert_allclose(r.w_hat, rw[:, inv], rtol=0, atol=1e-15)


def test_g_idx_rebuilds_w_hat():
    """Every column dequantizes with the parameters of its group g_idx[j]."""
    w, x = _case(7, 9, 48)
    r = O.solve_layer_act_order(w, [x], 4, 8, 16).result
    assert not np.array_equal(r.perm, np.arange(48))
    rebuilt = O.dequant(r.codes.astype(np.float64), r.scales[:, r.g_idx], r.zeros[:, r.g_idx])
    np.testing.assert_array_equal(rebuilt, r.w_hat)
    # each group holds group_size columns
    np.testing.assert_array_equal(np.bincount(r.g_idx), np.full(6, 8))


@pytest.mark.parametrize("group", [0, 2])
def test_act_order_equals_obq_in_that_order(group):
    """OBQ's compensation with explicit inverses of the reordered H_lambda
    (wiki 'OBQ에서 GPTQ로'), applied in the act-order column order, gives the
    same codes as the Cholesky / lazy-batch loop with the reordered factor."""
    w, x = _case(31, 5, 8)
    H = O.hessian([x])
    perm = O.act_order_perm(H)
    assert not np.array_equal(perm, np.arange(8))
    H_lam = O.damp(H[np.ix_(perm, perm)])[0]
    r = O.gptq_quantize_act_order(w, O.inv_hessian_factor(H_lam), perm, 3, group, 2)
    codes, w_hat = O.obq_fixed_order(w[:, perm], H_lam, 3, group, "inverse")
    inv = np.argsort(perm)
    np.testing.assert_array_equal(r.codes, codes[:, inv])
    np.testing.assert_allclose(r.w_hat, w_hat[:, inv], rtol=0, atol=1e-12)


def test_act_order_error_identity():
    """1/2 ||E||^2 - 1/2 lambda ||dW||^2 equals ||X dW^T||^2 in any column order."""
    w, x = _case(11, 14, 36, n=300)
    sol = O.solve_layer_act_order(w, [x], 3, 12, 12)
    dW = w - sol.result.w_hat
    lhs = 0.5 * sol.result.err_sq_sum - 0.5 * sol.lam * float(np.sum(dW * dW))
    assert lhs == pytest.approx(sol.err, rel=1e-9)
    assert sol.err == pytest.approx(O.output_error_direct(w, sol.result.w_hat, x), rel=1e-9)


def test_pins_catch_planted_mistakes():
    """A factor of the un-reordered H, or a group map built from perm instead of
    its inverse, fails the pins above."""
    w, x = _case(31, 5, 8)
    H = O.hessian([x])
    perm = O.act_order_perm(H)
    H_lam = O.damp(H[np.ix_(perm, perm)])[0]
    codes, _ = O.obq_fixed_order(w[:, perm], H_lam, 3, 0, "inverse")
    inv = np.argsort(perm)
    wrong_U = O.inv_hessian_factor(O.damp(H)[0])
    bad = O.gptq_quantize_act_order(w, wrong_U, perm, 3, 0, 2)
    assert not np.array_equal(bad.codes, codes[:, inv])
    w2, x2 = _case(7, 9, 48)
    r = O.solve_layer_act_order(w2, [x2], 4, 8, 16).result
    wrong_g = r.perm // 8
    rebuilt = O.dequant(r.codes.astype(np.float64), r.scales[:, wrong_g], r.zeros[:, wrong_g])
    assert not np.array_equal(rebuilt, r.w_hat)
