"""Pins for the fp64 oracle: closed forms, brute force, the OBQ form, invariants.

Each test names the page and section whose statement it checks.
"""
import json
import os

import numpy as np
import pytest

import oracle as O
import workloads as wl

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _spd(d, seed, cond_boost=1.0):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((3 * d, d))
    return a.T @ a + cond_boost * np.eye(d)


def _tiny(seed, d_row, d_col, n=64, corr=0.8):
    w, x = wl.tiny_case(seed, d_row, d_col, n, corr)
    H = O.hessian([x])
    H_lam, lam = O.damp(H, 0.01)
    return w, x, H, H_lam, lam


# ---------------------------------------------------------------- Hessian
def test_hessian_matches_python_loops_exactly():
    """Blog section 3 / wiki sketch: H = 2 X^T X, as explicit sums."""
    rng = np.random.default_rng(3)
    x = rng.integers(-4, 5, size=(7, 3)).astype(np.float64)
    H = O.hessian([x])
    for i in range(3):
        for j in range(3):
            s = 0.0
            for k in range(7):
                s += 2.0 * x[k, i] * x[k, j]
            assert H[i, j] == s


def test_hessian_is_a_sum_over_chunks():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 6)).astype(np.float16)
    full = O.hessian([x])
    parts = O.hessian([x[:13], x[13:31], x[31:]])
    np.testing.assert_allclose(parts, full, rtol=1e-13, atol=1e-13)
    np.testing.assert_array_equal(full, full.T)


def test_damp_closed_form():
    """Wiki three-changes table: lambda = 1% of the mean diagonal."""
    H = np.diag([1.0, 2.0, 3.0, 6.0]) + 0.5
    Hl, lam = O.damp(H, 0.01)
    assert lam == pytest.approx(0.01 * np.mean([1.5, 2.5, 3.5, 6.5]), rel=1e-15)
    np.testing.assert_allclose(Hl - H, lam * np.eye(4), rtol=0, atol=1e-15)


# ---------------------------------------------------------------- factor
@pytest.mark.parametrize("route", [O.inv_hessian_factor, O.inv_hessian_factor_reverse])
def test_factor_recovers_known_U(route):
    """Algorithm 1: U upper with U^T U = H^-1; given U, H = (U^T U)^-1 returns it."""
    rng = np.random.default_rng(5)
    d = 9
    U = np.triu(rng.standard_normal((d, d)) * 0.3)
    U[np.diag_indices(d)] = rng.uniform(0.5, 2.0, d)
    H = np.linalg.inv(U.T @ U)
    np.testing.assert_allclose(route(H), U, rtol=0, atol=1e-10)


def test_factor_routes_agree_and_residuals():
    for seed, d in [(1, 5), (2, 40), (3, 130)]:
        Hl, _ = O.damp(_spd(d, seed, 0.0), 0.01)
        U1 = O.inv_hessian_factor(Hl)
        U2 = O.inv_hessian_factor_reverse(Hl)
        assert np.allclose(np.tril(U1, -1), 0) and np.all(np.diag(U1) > 0)
        np.testing.assert_allclose(U2, U1, rtol=0, atol=1e-12 * np.abs(U1).max())
        np.testing.assert_allclose(U1.T @ U1 @ Hl, np.eye(d), atol=1e-10)


def test_factor_not_pd_raises():
    H = np.zeros((4, 4))
    with pytest.raises(O.NotPositiveDefinite):
        O.inv_hessian_factor(H)


# ---------------------------------------------------------------- grid / quantizer
def test_hand_worked_example():
    """Hand-worked Algorithm 1 on one row (tests/golden/hand_example_4col.json)."""
    with open(os.path.join(GOLD, "hand_example_4col.json")) as f:
        g = json.load(f)
    W0 = np.array(g["W0"])
    U = np.array(g["U"])
    s, z = O.grid_params(W0, g["bits"])
    np.testing.assert_allclose(s, g["scale"], rtol=1e-15)
    np.testing.assert_array_equal(z, g["zero"])
    for B in (1, 2, 3, 4, 128):
        r = O.gptq_quantize(W0, U, g["bits"], 0, B)
        np.testing.assert_array_equal(r.codes, g["codes"])
        np.testing.assert_allclose(r.w_hat, g["w_hat"], rtol=0, atol=1e-15)
        assert r.err_sq_sum == pytest.approx(float(np.sum(np.square(g["E"]))), rel=1e-12)
    rc, _ = O.rtn(W0, g["bits"])
    np.testing.assert_array_equal(rc, g["rtn_codes"])


def test_quantizer_round_half_even_and_clamp():
    """The sketch uses torch.round (half to even), then + zero, then clamp."""
    w = np.array([0.5, 1.5, 2.5, -0.5, 100.0, -100.0])
    c = O.quant_codes(w, 1.0, 3.0, 7)
    np.testing.assert_array_equal(c, [3, 5, 5, 3, 7, 0])


def test_grid_floor_on_constant_row():
    s, z = O.grid_params(np.array([[0.25, 0.25, 0.25]]), 4)
    assert s[0] == pytest.approx(1e-8 / 15)


# ---------------------------------------------------------------- loop
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("d_col", [3, 5, 8])
def test_obq_fixed_order_equals_gptq(bits, d_col):
    """Wiki 'OBQ에서 GPTQ로': OBQ's delta_F and elimination downdate, applied in the
    same natural order, give the same codes as the Cholesky/lazy-batch form."""
    w, x, H, H_lam, lam = _tiny(10 * bits + d_col, 6, d_col)
    U = O.inv_hessian_factor(H_lam)
    ref = O.gptq_quantize(w, U, bits, 0, 128)
    for dd in ("inverse", "gauss"):
        codes, w_hat = O.obq_fixed_order(w, H_lam, bits, 0, dd)
        np.testing.assert_array_equal(codes, ref.codes)
        np.testing.assert_allclose(w_hat, ref.w_hat, rtol=0, atol=1e-12)
    for B in (1, 2, 3):
        np.testing.assert_array_equal(O.gptq_quantize(w, U, bits, 0, B).codes, ref.codes)


def test_obq_fixed_order_equals_gptq_groups():
    w, x, H, H_lam, lam = _tiny(77, 5, 8)
    U = O.inv_hessian_factor(H_lam)
    for g, B in [(2, 2), (2, 4), (4, 2), (4, 8), (8, 8)]:
        ref = O.gptq_quantize(w, U, 3, g, B)
        codes, w_hat = O.obq_fixed_order(w, H_lam, 3, g, "inverse")
        np.testing.assert_array_equal(codes, ref.codes)
        np.testing.assert_allclose(w_hat, ref.w_hat, rtol=0, atol=1e-12)


def test_block_size_invariance_ragged():
    """Wiki three-changes table, lazy batch: the block size changes speed, not the
    result (B = 1 equals B = 128 equals any B, ragged final block included)."""
    w, x, H, H_lam, lam = _tiny(11, 40, 70, n=200)
    U = O.inv_hessian_factor(H_lam)
    ref = O.gptq_quantize(w, U, 4, 0, 1)
    for B in (3, 16, 64, 128):
        r = O.gptq_quantize(w, U, 4, 0, B)
        np.testing.assert_array_equal(r.codes, ref.codes)
        np.testing.assert_allclose(r.w_hat, ref.w_hat, rtol=0, atol=1e-12)
        assert r.err_sq_sum == pytest.approx(ref.err_sq_sum, rel=1e-10)
    refg = O.gptq_quantize(w, U, 3, 8, 1)
    for B in (2, 8, 16, 32):
        np.testing.assert_array_equal(O.gptq_quantize(w, U, 3, 8, B).codes, refg.codes)
    # g > B: group parameters at a block start read fully updated columns
    refg = O.gptq_quantize(w, U, 3, 32, 1)
    np.testing.assert_array_equal(O.gptq_quantize(w, U, 3, 32, 16).codes, refg.codes)


@pytest.mark.parametrize("group", [0, 16])
def test_diagonal_hessian_equals_rtn(group):
    """With a diagonal H no error can be compensated: GPTQ reduces to RTN
    (wiki '문제 설정' contrasts the two)."""
    rng = np.random.default_rng(12)
    w = 0.02 * rng.standard_normal((20, 48))
    H = np.diag(rng.uniform(0.5, 5.0, 48))
    U = O.inv_hessian_factor(O.damp(H)[0])
    assert np.allclose(np.triu(U, 1), 0)
    r = O.gptq_quantize(w, U, 4, group, 16)
    rc, rw = O.rtn(w, 4, group)
    np.testing.assert_array_equal(r.codes, rc)
    np.testing.assert_allclose(r.w_hat, rw, rtol=0, atol=1e-15)


def test_weights_on_grid_are_kept():
    rng = np.random.default_rng(13)
    bits, d = 3, 24
    scale = 2.0 ** -6
    zero = 3
    c = rng.integers(0, 8, size=(10, d)).astype(np.float64)
    c[:, 0], c[:, 1] = 0, 7
    w = scale * (c - zero)
    w, x, H, H_lam, lam = (w,) + _tiny(14, 10, d)[1:]
    U = O.inv_hessian_factor(H_lam)
    r = O.gptq_quantize(w, U, bits, 0, 8)
    np.testing.assert_array_equal(r.codes, c)
    np.testing.assert_array_equal(r.w_hat, w)
    assert O.output_error(w, r.w_hat, H) == 0.0


def test_hessian_scale_invariance():
    w, x, H, H_lam, lam = _tiny(15, 12, 33)
    r1 = O.gptq_quantize(w, O.inv_hessian_factor(H_lam), 4, 0, 8)
    r2 = O.gptq_quantize(w, O.inv_hessian_factor(7.25 * H_lam), 4, 0, 8)
    np.testing.assert_array_equal(r1.codes, r2.codes)


def test_error_identities():
    """1/2 ||E||^2 equals the damped objective (OBS increments, wiki OBQ equation);
    the undamped objective equals ||X dW^T||^2 evaluated from the rows."""
    w, x, H, H_lam, lam = _tiny(16, 9, 30, n=90)
    U = O.inv_hessian_factor(H_lam)
    for g, B in [(0, 1), (0, 8), (10, 10), (5, 10)]:
        r = O.gptq_quantize(w, U, 3, g, B)
        D = w - r.w_hat
        damped = 0.5 * np.sum((D @ H_lam) * D)
        assert 0.5 * r.err_sq_sum == pytest.approx(damped, rel=1e-10)
        e1 = O.output_error(w, r.w_hat, H)
        e2 = O.output_error_direct(w, r.w_hat, x)
        assert e1 == pytest.approx(e2, rel=1e-10)
        assert e1 == pytest.approx(0.5 * r.err_sq_sum - 0.5 * lam * np.sum(D * D), rel=1e-9)


def test_outputs_on_grid():
    w, x, H, H_lam, lam = _tiny(17, 16, 64, n=128)
    U = O.inv_hessian_factor(H_lam)
    for bits, g in [(2, 0), (3, 16), (8, 32)]:
        r = O.gptq_quantize(w, U, bits, g, 16)
        assert r.codes.max() <= (1 << bits) - 1
        gg = g or 64
        for gi in range(64 // gg):
            sl = slice(gi * gg, (gi + 1) * gg)
            np.testing.assert_array_equal(
                r.w_hat[:, sl],
                r.scales[:, gi:gi + 1] * (r.codes[:, sl].astype(np.float64) - r.zeros[:, gi:gi + 1]))


def test_exhaustive_optimum_is_a_lower_bound():
    for seed, d in [(20, 3), (21, 5), (22, 6)]:
        w, x, H, H_lam, lam = _tiny(seed, 4, d, n=32, corr=0.9)
        U = O.inv_hessian_factor(H_lam)
        r = O.gptq_quantize(w, U, 2, 0, 4)
        opt = O.exhaustive_optimum(w, H, 2)
        e = O.output_error(w, r.w_hat, H)
        _, rw = O.rtn(w, 2)
        assert opt <= e * (1 + 1e-12)
        assert opt <= O.output_error(w, rw, H) * (1 + 1e-12)


def test_gptq_beats_rtn_on_correlated_512():
    """Wiki '최소 구현': on correlated random 512-dim inputs with 2048 samples, GPTQ's
    output squared error is below (the page says under half of) RTN's."""
    spec = wl.workload_layers(1)[0]
    W = wl.make_weight(spec)
    X = wl.make_x(spec)
    sol = O.solve_layer(W, [X], 4, 0, 128)
    _, rw = O.rtn(W, 4)
    ratio = sol.err / O.output_error(W, rw, sol.H)
    assert ratio < 0.5


# ---------------------------------------------------------------- forced replay
def test_replay_with_own_codes_is_identity():
    w, x, H, H_lam, lam = _tiny(30, 20, 48, n=100)
    U = O.inv_hessian_factor(H_lam)
    r = O.gptq_quantize(w, U, 4, 16, 16)
    rr = O.gptq_quantize(w, U, 4, 16, 16, replay_codes=r.codes, replay_zeros=r.zeros)
    assert rr.adopted_codes == 0 and rr.adopted_zeros == 0
    np.testing.assert_array_equal(rr.codes, r.codes)


def test_replay_rejects_non_boundary_mismatch():
    w, x, H, H_lam, lam = _tiny(31, 20, 48, n=100)
    U = O.inv_hessian_factor(H_lam)
    r = O.gptq_quantize(w, U, 4, 0, 16)
    bad = r.codes.copy()
    bad[3, 5] = (int(bad[3, 5]) + 2) % 16
    with pytest.raises(O.ReplayMismatch):
        O.gptq_quantize(w, U, 4, 0, 16, replay_codes=bad)


def test_replay_accepts_only_near_boundary_flip():
    """Flip the last column's decision closest to a tie (no later column can
    cascade); replay adopts it only when the tie distance is within tolerance."""
    w, x, H, H_lam, lam = _tiny(32, 30, 40, n=100)
    U = O.inv_hessian_factor(H_lam)
    r = O.gptq_quantize(w, U, 4, 0, 8)
    # recover w/scale at every decision by replaying B=1 with recording
    s = r.scales[:, 0]
    z = r.zeros[:, 0]
    W = w.copy()
    for j in range(40):
        v = W[:, j] / s
        if j == 39:
            dist = np.abs(v - (np.floor(v) + 0.5))
            c_un = np.rint(v) + z
            dist[(c_un < 1) | (c_un > 14)] = np.inf
            i = int(np.argmin(dist))
            c_here = int(r.codes[i, j])
            other = c_here + (1 if v[i] > np.rint(v[i]) else -1)
            best = (float(dist[i]), i, j, other)
        q = s * (r.codes[:, j] - z)
        e = (W[:, j] - q) / U[j, j]
        W[:, j:] -= np.outer(e, U[j, j:])
    dist, i, j, other = best
    flipped = r.codes.copy()
    flipped[i, j] = other
    with pytest.raises(O.ReplayMismatch):
        O.gptq_quantize(w, U, 4, 0, 8, replay_codes=flipped, replay_tol=dist * 0.5)
    rr = O.gptq_quantize(w, U, 4, 0, 8, replay_codes=flipped, replay_tol=dist * 2 + 1e-12,)
    assert rr.adopted_codes >= 1 and rr.codes[i, j] == other


# ---------------------------------------------------------------- forced replay at ties
# Wiki "실무 변형" (group parameters from the latest weights) makes the zero-point an
# integer decision like the codes: round(-min / scale).  Forced replay may adopt a
# supplied value only where that decision sits at a tie.  These cases construct a
# tie exactly, so the adoption branch runs, and a non-tie neighbour, which must be
# rejected.

def zero_tie_case():
    """Per-row grid (4-bit) where row 3 has -min/scale = 7.5 + 2e-4: the oracle's
    zero-point is 8, the other side of the tie is 7 (adoptable), 9 is a neighbour
    of 8 whose tie 8.5 is ~1 away (not adoptable).  Returns
    (W0, U, bits, group, block, row, zeros_adopt, zeros_reject)."""
    w, x = wl.tiny_case(41, 6, 12, 64, 0.8)
    H_lam, _ = O.damp(O.hessian([x]), 0.01)
    U = O.inv_hessian_factor(H_lam)
    r, span, v = 3, 0.06, 7.5 + 2e-4
    a = span * v / 15.0
    w[r] = np.linspace(-a + 1e-3, span - a - 1e-3, w.shape[1])
    w[r, 4], w[r, 9] = -a, span - a          # min and max of the row
    base = O.gptq_quantize(w, U, 4, 0, 4)
    assert base.zeros[r, 0] == 8
    adopt, reject = base.zeros.copy(), base.zeros.copy()
    adopt[r, 0], reject[r, 0] = 7, 9
    return w, U, 4, 0, 4, r, adopt, reject


def code_tie_case():
    """Identity U (no feedback, so every decision is round-to-nearest of W0 / scale
    on the per-row grid): row 2, column 5 holds w / scale = (k + 0.5) + 3e-4 with
    the code k + 1 + zero; supplying k + zero must be adopted.  Row 1, column 6
    (w / scale = k' + 0.3) supplied with its other neighbour must be rejected.
    Returns (W0, U, bits, block, codes_adopt, codes_reject)."""
    rng = np.random.default_rng(43)
    w = 0.02 * rng.standard_normal((4, 10))
    s, z = O.grid_params(w, 4)
    w[2, 5] = s[2] * (2 + 0.5 + 3e-4)
    w[1, 6] = s[1] * (-1 + 0.3)
    s2, z2 = O.grid_params(w, 4)
    assert np.array_equal(s, s2) and np.array_equal(z, z2)   # interior values only
    U = np.eye(10)
    base = O.gptq_quantize(w, U, 4, 0, 4)
    assert base.codes[2, 5] == 3 + z[2] and base.codes[1, 6] == -1 + z[1]
    adopt, reject = base.codes.copy(), base.codes.copy()
    adopt[2, 5] = 2 + z[2]
    reject[1, 6] = 0 + z[1]
    return w, U, 4, 4, adopt, reject


def test_replay_adopts_a_zero_point_at_a_tie():
    w, U, bits, g, B, r, adopt, reject = zero_tie_case()
    res = O.gptq_quantize(w, U, bits, g, B, replay_zeros=adopt)
    assert res.adopted_zeros == 1
    np.testing.assert_array_equal(res.zeros, adopt)
    # the adopted zero-point is the one the row's codes and What use
    np.testing.assert_array_equal(res.w_hat[r], res.scales[r, 0] * (res.codes[r].astype(np.float64) - 7))
    free = O.gptq_quantize(w, U, bits, g, B)
    np.testing.assert_array_equal(res.codes[np.arange(6) != r], free.codes[np.arange(6) != r])
    assert not np.array_equal(res.w_hat[r], free.w_hat[r])


def test_replay_rejects_a_zero_point_off_the_tie():
    w, U, bits, g, B, r, adopt, reject = zero_tie_case()
    with pytest.raises(O.ReplayMismatch):
        O.gptq_quantize(w, U, bits, g, B, replay_zeros=reject)
    far = adopt.copy()
    far[r, 0] = 6                                            # two steps away
    with pytest.raises(O.ReplayMismatch):
        O.gptq_quantize(w, U, bits, g, B, replay_zeros=far)
    with pytest.raises(O.ReplayMismatch):                    # tie farther than the tolerance
        O.gptq_quantize(w, U, bits, g, B, replay_zeros=adopt, replay_tol=1e-4)


def test_replay_adopts_a_group_zero_point_at_a_tie():
    """Groups of 16 inside blocks of 32, identity U (each group's grid comes from
    W0 alone): group 2 of row 1 is built with -min/scale = 4.5 - 3e-4."""
    rng = np.random.default_rng(44)
    w = 0.02 * rng.standard_normal((3, 64))
    span, v = 0.05, 4.5 - 3e-4
    a = span * v / 15.0
    w[1, 32:48] = np.linspace(-a, span - a, 16)
    U = np.eye(64)
    base = O.gptq_quantize(w, U, 4, 16, 32)
    assert base.zeros[1, 2] == 4
    adopt = base.zeros.copy()
    adopt[1, 2] = 5
    res = O.gptq_quantize(w, U, 4, 16, 32, replay_zeros=adopt)
    assert res.adopted_zeros == 1 and res.zeros[1, 2] == 5
    np.testing.assert_array_equal(res.w_hat[1, 32:48],
                                  res.scales[1, 2] * (res.codes[1, 32:48].astype(np.float64) - 5))
    bad = base.zeros.copy()
    bad[1, 2] = 3
    with pytest.raises(O.ReplayMismatch):
        O.gptq_quantize(w, U, 4, 16, 32, replay_zeros=bad)


def test_replay_adopts_a_code_at_a_tie_and_rejects_a_neighbour_off_it():
    w, U, bits, B, adopt, reject = code_tie_case()
    res = O.gptq_quantize(w, U, bits, 0, B, replay_codes=adopt)
    assert res.adopted_codes == 1
    np.testing.assert_array_equal(res.codes, adopt)
    assert res.max_boundary_dist == pytest.approx(3e-4, abs=1e-9)
    with pytest.raises(O.ReplayMismatch):
        O.gptq_quantize(w, U, bits, 0, B, replay_codes=reject)


def test_trailing_block_of_U_is_the_factor_of_the_trailing_block():
    """For upper U with U^T U = H^-1, rows and columns k.. of U form the factor of
    (H[k:, k:])^-1: H = Ut Ut^T with Ut = U^-1 upper gives H[k:, k:] =
    Ut[k:, k:] Ut[k:, k:]^T.  This is what lets a trailing block of a factor too
    wide for the host be checked against the oracle on its own."""
    rng = np.random.default_rng(12)
    a = rng.standard_normal((400, 160))
    Hl, _ = O.damp(a.T @ a, 0.01)
    U = O.inv_hessian_factor(Hl)
    for k in (0, 1, 37, 100, 159):
        np.testing.assert_allclose(U[k:, k:], O.inv_hessian_factor(Hl[k:, k:]), rtol=0, atol=1e-12)
