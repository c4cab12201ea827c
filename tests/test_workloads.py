"""Checks of the seeded synthetic input recipes (not of the solver)."""
import numpy as np
import pytest

import workloads as wl


def test_ar1_closed_form_factor_matches_cholesky():
    d, rho = 40, 0.9
    k = np.arange(d)
    S = rho ** np.abs(k[:, None] - k[None, :])
    np.testing.assert_allclose(wl.ar1_lower_factor(d, rho), np.linalg.cholesky(S),
                               rtol=0, atol=1e-13)


def test_workload1_bytes_are_deterministic_and_correlated():
    s = wl.workload_layers(1)[0]
    w1, w2 = wl.make_weight(s), wl.make_weight(s)
    x1, x2 = wl.make_x(s), wl.make_x(s)
    assert w1.dtype == np.float32 and x1.dtype == np.float32
    assert w1.shape == (512, 512) and x1.shape == (2048, 512)
    np.testing.assert_array_equal(w1, w2)
    np.testing.assert_array_equal(x1, x2)
    # the first draw of default_rng(0) is W
    np.testing.assert_array_equal(
        w1, (0.02 * np.random.default_rng(0).standard_normal((512, 512))).astype(np.float32))
    c = np.corrcoef(x1[:, :8].T.astype(np.float64))
    assert abs(c[0, 1] - 0.9) < 0.05 and abs(c[0, 2] - 0.81) < 0.06


@pytest.mark.parametrize("wk", [2, 3, 4, 5])
def test_layer_specs_and_small_chunks(wk):
    for spec in wl.workload_layers(wk):
        assert spec.n_rows in (163840, 262144)
        w_dt = np.float16 if wk >= 3 else np.float32
        assert spec.np_w_dtype == w_dt
        small = spec.scaled(d_row=8) if spec.x_kind != "powerlaw" else spec.scaled(d_row=8)
        x = wl.make_x_chunk(small, 0, rows=4) if spec.d_col <= 16384 else None
        if x is not None:
            assert x.shape == (4, spec.d_col) and x.dtype == spec.np_x_dtype
            np.testing.assert_array_equal(x, wl.make_x_chunk(small, 0, rows=4))


def test_chunks_are_independent_streams():
    spec = wl.workload_layers(3)[0].scaled(d_col=256)
    a = wl.make_x_chunk(spec, 0, rows=32)
    b = wl.make_x_chunk(spec, 1, rows=32)
    assert not np.array_equal(a, b)
    np.testing.assert_array_equal(a, wl.make_x_chunk(spec, 0, rows=32))


def test_lowrank_inputs_have_rank_64_before_outliers():
    spec = wl.workload_layers(3)[0].scaled(d_col=256)
    x = wl.make_x_chunk(spec, 0, rows=512).astype(np.float64)
    a, ch = wl._lowrank_params(spec)
    keep = np.setdiff1d(np.arange(256), ch)
    sv = np.linalg.svd(x[:, keep], compute_uv=False)
    assert sv[63] > 1e-2 * sv[0] and sv[64] < 1e-2 * sv[0]   # fp16 rounding noise only


def test_powerlaw_mix_is_orthogonal_with_k_inverse_spectrum():
    """X = (Z * s) Q^T with Q orthogonal: push the identity through the mix."""
    spec = wl.LayerSpec(5, 0, "t", 4, 24, 100, "f16", "f16", 0.01, 3, 0, x_kind="powerlaw")
    m, s, signs, q3, perm = wl._powerlaw_params(spec)
    eye = np.eye(24) * signs
    y = np.einsum("ab,rbk->rak", q3, eye.reshape(24, 3, 1 << m))
    y = wl._fwht_rows(y) * 2.0 ** (-m / 2.0)
    Q = np.empty((24, 24))
    Q[:, perm] = y.reshape(24, 24)
    np.testing.assert_allclose(Q @ Q.T, np.eye(24), atol=1e-12)
    k = np.arange(1, 25)
    np.testing.assert_allclose(s ** 2, 24.0 / (k * np.sum(1.0 / k)), rtol=1e-12)


# ---------------------------------------------------------------- device recipes
# The device generator draws other random numbers than the host one; what must
# agree is the law.  Each check inverts the recipe's deterministic part on the
# CPU build of torch and looks at what is left.

def _device_chunk(spec, rows):
    from workloads import device as D
    return D.make_x_chunk_device(spec, 0, rows=rows, device="cpu").float().numpy().astype(np.float64)


def test_device_powerlaw_inverts_to_white_noise():
    spec = wl.workload_layers(5)[0].scaled(d_col=3 * 256)
    x = _device_chunk(spec, 8192)
    m, s, signs, q3, perm = wl._powerlaw_params(spec)
    y = x[:, perm].reshape(-1, 3, 1 << m)                  # undo the permutation
    y = wl._fwht_rows(y) * 2.0 ** (-m / 2.0)               # the normalised transform is its own inverse
    y = np.einsum("ba,rbk->rak", q3, y).reshape(-1, spec.d_col) / (s * signs)
    # fp16 storage rounds x by <= 2^-11 relative; the whitened values stay N(0, 1)
    assert abs(y.mean()) < 0.01
    v = y.var(axis=0)
    assert abs(v.mean() - 1.0) < 0.01 and v.max() < 1.2 and v.min() > 0.8


def test_device_lowrank_lies_in_the_mixing_row_space():
    spec = wl.workload_layers(3)[0].scaled(d_col=512)
    x = _device_chunk(spec, 4096)
    a, ch = wl._lowrank_params(spec)
    x[:, ch] /= 20.0
    z = x @ np.linalg.pinv(a)
    resid = np.linalg.norm(x - z @ a) / np.linalg.norm(x)
    assert resid < 2e-3                                   # fp16 rounding only
    assert abs(z.var() - 1.0) < 0.05


def test_device_silu_moments():
    spec = wl.workload_layers(4)[1].scaled(d_col=256)
    x = _device_chunk(spec, 16384)
    # E[SiLU(a) b] = 0, E[(SiLU(a) b)^2] = E[SiLU(a)^2] (b independent, unit variance)
    t = np.linspace(-12, 12, 200001)
    phi = np.exp(-t * t / 2) / np.sqrt(2 * np.pi)
    m2 = np.trapezoid((t / (1 + np.exp(-t))) ** 2 * phi, t)
    assert abs(x.mean()) < 0.01
    assert abs((x * x).mean() - m2) < 0.01 * m2 * 3
