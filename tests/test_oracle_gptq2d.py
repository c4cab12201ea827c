"""Pins of the two-sided adaptive rounding oracle (GPTQ-2D review page, sections
1-3: the two-sided metric ||A (Z - X) B||_F^2, its Kronecker vectorisation, the
anti-diagonal sweep).  CPU only."""
import numpy as np
import pytest

import oracle as O

Q2 = O.gptq2d


def _case(seed, m, n, corr=0.7):
    rng = np.random.default_rng(seed)
    X = 0.02 * rng.standard_normal((m, n))
    A = np.eye(m) + corr * rng.standard_normal((m, m)) / np.sqrt(m)
    B = np.eye(n) + corr * rng.standard_normal((n, n)) / np.sqrt(n)
    U_Q = O.inv_hessian_factor(A.T @ A)
    U_P = O.inv_hessian_factor(B @ B.T)
    return X, A, B, U_Q, U_P


@pytest.mark.parametrize("m,n,bits", [(5, 7, 3), (8, 6, 4), (1, 9, 2), (7, 1, 4), (6, 6, 8)])
def test_equals_one_sided_rounding_of_the_vectorised_matrix(m, n, bits):
    """The sweep equals the one-sided lazy-batch loop run on vec(X) (column-major)
    with U = U_P kron U_Q, one grid for the whole row."""
    X, A, B, U_Q, U_P = _case(m * 10 + n, m, n)
    r = Q2.gptq2d(X, U_Q, U_P, bits)
    v = X.reshape(-1, order="F")[None, :]
    one = O.gptq_quantize(v, np.kron(U_P, U_Q), bits, 0, 1)
    np.testing.assert_array_equal(r.codes.reshape(-1, order="F"), one.codes[0])
    np.testing.assert_allclose(r.w_hat.reshape(-1, order="F"), one.w_hat[0], rtol=0, atol=1e-15)
    assert r.err == pytest.approx(one.err_sq_sum, rel=1e-10)


def test_kronecker_vectorisation_of_the_metric():
    """||A D B||^2 = vec(D)^T (B B^T kron A^T A) vec(D) (column-major vec)."""
    X, A, B, _, _ = _case(3, 4, 5)
    D = np.random.default_rng(4).standard_normal(X.shape)
    v = D.reshape(-1, order="F")
    assert Q2.two_sided_metric(X, X + D, A, B) == pytest.approx(v @ np.kron(B @ B.T, A.T @ A) @ v, rel=1e-12)


def test_the_metric_is_the_sum_of_squared_scaled_errors():
    X, A, B, U_Q, U_P = _case(5, 9, 11)
    r = Q2.gptq2d(X, U_Q, U_P, 3)
    assert Q2.two_sided_metric(X, r.w_hat, A, B) == pytest.approx(r.err, rel=1e-9)


def test_entries_of_an_anti_diagonal_are_independent():
    """Rounding a diagonal's entries in reverse order, each feeding back at once,
    changes nothing: none reads another's feedback."""
    X, _, _, U_Q, U_P = _case(7, 10, 8)
    a = Q2.gptq2d(X, U_Q, U_P, 4)
    b = Q2.gptq2d(X, U_Q, U_P, 4, reverse_within_diagonal=True)
    np.testing.assert_array_equal(a.codes, b.codes)
    np.testing.assert_array_equal(a.E, b.E)


def test_identity_sides_give_round_to_nearest():
    X, _, _, _, _ = _case(9, 6, 7)
    r = Q2.gptq2d(X, np.eye(6), np.eye(7), 3)
    s, z = Q2.tensor_grid(X, 3)
    np.testing.assert_array_equal(r.codes, O.quant_codes(X, s, z, 7).astype(np.uint8))


def test_identity_right_side_rounds_columns_independently():
    """With B = I every column is its own one-sided problem (the same grid)."""
    X, A, _, U_Q, _ = _case(11, 8, 5)
    grid = Q2.tensor_grid(X, 4)
    full = Q2.gptq2d(X, U_Q, np.eye(5), 4)
    for j in range(5):
        col = Q2.gptq2d(X[:, [j]], U_Q, np.eye(1), 4, grid=grid)
        np.testing.assert_array_equal(full.codes[:, [j]], col.codes)


def test_better_than_round_to_nearest():
    X, A, B, U_Q, U_P = _case(13, 24, 20, corr=1.5)
    r = Q2.gptq2d(X, U_Q, U_P, 3)
    s, z = Q2.tensor_grid(X, 3)
    rtn = O.dequant(O.quant_codes(X, s, z, 7), s, z)
    assert Q2.two_sided_metric(X, r.w_hat, A, B) < 0.8 * Q2.two_sided_metric(X, rtn, A, B)


def test_replay_adopts_only_ties():
    X, _, _, U_Q, U_P = _case(15, 6, 6)
    r = Q2.gptq2d(X, U_Q, U_P, 4)
    assert Q2.gptq2d(X, U_Q, U_P, 4, replay_codes=r.codes).adopted_codes == 0
    bad = r.codes.copy()
    bad[2, 3] = (int(bad[2, 3]) + 3) % 16
    with pytest.raises(O.ReplayMismatch):
        Q2.gptq2d(X, U_Q, U_P, 4, replay_codes=bad)


def tie_case_2d():
    """Entry (2, 3) of a 5 x 6 matrix is placed so that the value it is rounded
    from, divided by the scale, is (k + 0.5) + 2e-4; entry (4, 1) sits at k' + 0.3.
    Identity side factors (no feedback).  Returns (X, U_Q, U_P, bits, codes with
    (2, 3) moved to the other side of its tie, codes with (4, 1) moved to its
    other neighbour)."""
    rng = np.random.default_rng(47)
    X = 0.02 * rng.standard_normal((5, 6))
    s, z = Q2.tensor_grid(X, 4)
    X[2, 3] = s * (1 + 0.5 + 2e-4)
    X[4, 1] = s * (-2 + 0.3)
    assert Q2.tensor_grid(X, 4) == (s, z)
    base = Q2.gptq2d(X, np.eye(5), np.eye(6), 4)
    assert base.codes[2, 3] == 2 + z and base.codes[4, 1] == -2 + z
    adopt, reject = base.codes.copy(), base.codes.copy()
    adopt[2, 3] = 1 + z
    reject[4, 1] = -1 + z
    return X, np.eye(5), np.eye(6), 4, adopt, reject


def test_replay_adopts_the_last_decision_at_a_tie_with_real_factors():
    """With real side factors the last entry (m-1, n-1) is rounded from
    X - (U_Q^T M) with M built from every other entry; X[m-1, n-1] is moved so that
    this value sits 2e-4 past a tie (no other entry reads it, and the grid is
    unchanged).  Replay adopts the other side of the tie, and the reported error
    is still the metric of the adopted result."""
    X, A, B, U_Q, U_P = _case(18, 6, 7)
    s, z = Q2.tensor_grid(X, 4)
    r = Q2.gptq2d(X, U_Q, U_P, 4)
    M = np.zeros_like(X)
    for i in range(6):
        for j in range(7):
            if (i, j) != (5, 6):
                M[i, j:] += r.E[i, j] * U_P[j, j:]
    corr = U_Q[:, 5] @ M[:, 6]
    others = np.delete(X.ravel(), -1)
    assert others.min() == X.min() and others.max() == X.max()   # X[5, 6] is no extreme
    k = int(np.floor((0.5 * (X.min() + X.max()) - corr) / s))
    X[5, 6] = corr + s * (k + 0.5 + 2e-4)
    assert 0 < k + z < 14
    assert Q2.tensor_grid(X, 4) == (s, z)
    base = Q2.gptq2d(X, U_Q, U_P, 4)
    np.testing.assert_array_equal(np.delete(base.codes.ravel(), -1), np.delete(r.codes.ravel(), -1))
    assert base.codes[5, 6] == k + 1 + z
    flipped = base.codes.copy()
    flipped[5, 6] = k + z
    rr = Q2.gptq2d(X, U_Q, U_P, 4, replay_codes=flipped)
    assert rr.adopted_codes == 1 and rr.codes[5, 6] == k + z
    assert Q2.two_sided_metric(X, rr.w_hat, A, B) == pytest.approx(rr.err, rel=1e-9)
    assert rr.err != pytest.approx(base.err, rel=1e-12)
    with pytest.raises(O.ReplayMismatch):
        Q2.gptq2d(X, U_Q, U_P, 4, replay_codes=flipped, replay_tol=1e-4)


def test_replay_2d_adopts_only_at_the_tie():
    X, U_Q, U_P, bits, adopt, reject = tie_case_2d()
    r = Q2.gptq2d(X, U_Q, U_P, bits, replay_codes=adopt)
    assert r.adopted_codes == 1
    np.testing.assert_array_equal(r.codes, adopt)
    with pytest.raises(O.ReplayMismatch):
        Q2.gptq2d(X, U_Q, U_P, bits, replay_codes=reject)
    with pytest.raises(O.ReplayMismatch):
        Q2.gptq2d(X, U_Q, U_P, bits, replay_codes=adopt, replay_tol=1e-4)
