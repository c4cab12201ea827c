"""GPU parity of act-order (itwiki "GPTQ", section "실무 변형": columns with the
largest Hessian diagonal quantized first, with a column-to-group map) against
the fp64 oracle on the same seeded inputs.

The quantization order is an integer decision taken from the same fp32
diagonal on both sides, so it must match exactly.  The other stages keep the
natural-order tolerances (stage-isolated):
  U      relative Frobenius error <= 1e-4 against the oracle's factor of the
         reordered, damped fp32 H;
  codes  >= 99.9% identical (original column order), mismatches only within
         1e-3 of a rounding tie (forced replay with the oracle's reordered U in
         fp32); scales to 1e-5, zeros and g_idx exact;
  error  within 1% of the oracle's.
"""
import numpy as np
import pytest

import oracle as O
import workloads as wl

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

import post_weight_quantization_02_amd as G  # noqa: E402


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def relf(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    return float(np.linalg.norm(a - b) / np.linalg.norm(b))


def case_x(kind, n, d, dtype, seed):
    spec = wl.LayerSpec(9, seed, "t", 8, d, n, "f32", "f16" if dtype == np.float16 else "f32",
                        0.02, 4, 0, x_kind=kind)
    return wl.make_x_chunk(spec, 0, rows=n)


def case_w(d_row, d_col, dtype, seed, std=0.02):
    spec = wl.LayerSpec(9, seed, "t", d_row, d_col, 1, "f16" if dtype == np.float16 else "f32",
                        "f32", std, 4, 0)
    return wl.make_weight(spec)


def tie_nan_hessian(d, seed):
    """A Hessian-shaped fp32 input whose diagonal repeats few values (many ties)
    and holds two NaNs: the order's tie and NaN rules decide most positions."""
    rng = np.random.default_rng(seed)
    H = np.zeros((d, d), np.float32)
    dg = rng.choice(np.array([1.0, 2.0, 3.0, 0.0, -0.0], np.float32), d)
    dg[[5, d - 3]] = np.nan
    H[np.arange(d), np.arange(d)] = dg
    return H


PERM_CASES = [
    ("lowrank_1024", lambda: O.hessian([case_x("lowrank", 16384, 1024, np.float16, 61)]).astype(np.float32)),
    ("attn4096_recipe", lambda: O.hessian([wl.make_x_chunk(wl.workload_layers(3)[0], 0)]).astype(np.float32)),
    ("ties_and_nan_300", lambda: tie_nan_hessian(300, 62)),
    ("ties_and_nan_1", lambda: tie_nan_hessian(8, 63)[:1, :1].copy()),
]


@pytest.mark.parametrize("name,make", PERM_CASES, ids=[c[0] for c in PERM_CASES])
def test_act_order_perm_parity(name, make):
    H32 = make()
    pg = G.gptq_act_order_perm(dev(H32))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(pg.cpu().numpy(), O.act_order_perm(H32))


def _factor_perm_case(Ho, percdamp=0.01):
    H32 = Ho.astype(np.float32)
    perm = O.act_order_perm(H32)
    Hd, lam = O.damp(H32.astype(np.float64)[np.ix_(perm, perm)], percdamp)
    Uo = O.inv_hessian_factor(Hd)
    U, lamg, info = G.gptq_prepare_hinv_perm(dev(H32), dev(perm.astype(np.int32)), percdamp)
    torch.cuda.synchronize()
    assert int(info.item()) == 0
    assert abs(float(lamg.item()) - lam) <= 1e-6 * abs(lam)
    Ug = U.cpu().numpy()
    assert np.all(np.tril(Ug, -1) == 0)
    return relf(Ug, Uo)


F_CASES = [
    ("lowrank_1024", lambda: O.hessian([case_x("lowrank", 16384, 1024, np.float16, 64)])),
    ("ar1_700_ragged", lambda: O.hessian([case_x("ar1", 3000, 700, np.float32, 65)])),
    ("powerlaw_1536", lambda: O.hessian([case_x("powerlaw", 6144, 1536, np.float16, 66)])),
    ("attn4096_recipe", lambda: O.hessian([wl.make_x_chunk(wl.workload_layers(3)[0], 0)])),
]


@pytest.mark.parametrize("name,make", F_CASES, ids=[c[0] for c in F_CASES])
def test_act_order_factor_parity(name, make):
    assert _factor_perm_case(make()) <= 1e-4


def _quant_perm_case(W0, Ho, bits, group, B):
    H32 = Ho.astype(np.float32)
    perm = O.act_order_perm(H32)
    Hd, lam = O.damp(H32.astype(np.float64)[np.ix_(perm, perm)], 0.01)
    U32 = O.inv_hessian_factor(Hd).astype(np.float32)
    lam32 = np.array([lam], np.float32)
    codes, scales, zeros, g_idx, err = G.gptq_quantize_layer_perm(
        dev(W0), dev(U32), dev(lam32), dev(perm.astype(np.int32)), bits, group, B)
    torch.cuda.synchronize()
    cg, sg, zg, gg = codes.cpu().numpy(), scales.cpu().numpy(), zeros.cpu().numpy(), g_idx.cpu().numpy()
    r = O.gptq_quantize_act_order(W0.astype(np.float64), U32.astype(np.float64), perm, bits, group, B,
                                  replay_codes=cg, replay_zeros=zg)
    n = cg.size
    assert r.in_order.adopted_codes <= 0.001 * n, (r.in_order.adopted_codes, n)
    np.testing.assert_array_equal(r.codes, cg)
    np.testing.assert_allclose(sg, r.scales, rtol=1e-5, atol=0)
    np.testing.assert_array_equal(zg, r.zeros)
    np.testing.assert_array_equal(gg, r.g_idx)
    e_o = O.output_error(W0, r.w_hat, H32.astype(np.float64))
    e_g = float(err.item())
    assert abs(e_g - e_o) <= 0.01 * e_o, (e_g, e_o)


Q_CASES = [
    ("lowrank_fp16_512x1024_g128", lambda: (case_w(512, 1024, np.float16, 71, 0.015),
                                            O.hessian([case_x("lowrank", 16384, 1024, np.float16, 72)])), 4, 128, 128),
    ("ragged_37x300", lambda: (case_w(37, 300, np.float32, 73),
                               O.hessian([case_x("ar1", 2000, 300, np.float32, 74)])), 4, 0, 128),
    ("group32_in_block", lambda: (case_w(100, 384, np.float32, 75),
                                  O.hessian([case_x("powerlaw", 3000, 384, np.float32, 76)])), 3, 32, 128),
    ("group256_over_block", lambda: (case_w(100, 640, np.float16, 77),
                                     O.hessian([case_x("lowrank", 4000, 640, np.float16, 78)])), 4, 256, 128),
    ("B64_8bit", lambda: (case_w(80, 320, np.float32, 79),
                          O.hessian([case_x("lnorm", 1000, 320, np.float32, 80)])), 8, 0, 64),
    ("B16_2bit", lambda: (case_w(64, 200, np.float32, 81),
                          O.hessian([case_x("silu", 1000, 200, np.float32, 82)])), 2, 0, 16),
]


@pytest.mark.parametrize("name,make,bits,group,B", Q_CASES, ids=[c[0] for c in Q_CASES])
def test_act_order_quantize_parity(name, make, bits, group, B):
    W0, Ho = make()
    _quant_perm_case(W0, Ho, bits, group, B)


def test_act_order_end_to_end_and_determinism():
    W = case_w(256, 1024, np.float16, 83, 0.015)
    X = case_x("lowrank", 16384, 1024, np.float16, 84)
    sol = O.solve_layer_act_order(W, [X], 4, 128, 128)
    outs = [G.quantize_layer(dev(W), [dev(X[:9000]), dev(X[9000:])], 4, 128, 128, act_order=True)
            for _ in range(2)]
    for k in ("perm", "U", "codes", "scales", "zeros", "g_idx", "err"):
        assert torch.equal(outs[0][k], outs[1][k]), k
    e_g = float(outs[0]["err"].item())
    assert abs(e_g - sol.err) <= 0.01 * sol.err, (e_g, sol.err)
    # the GPU order comes from the GPU's fp32 H; it agrees with the oracle's
    # order except where two diagonals are within rounding of each other
    pg = outs[0]["perm"].cpu().numpy()
    dg = np.diag(sol.H)
    for i in np.nonzero(pg != sol.result.perm)[0]:
        a, b = dg[pg[i]], dg[sol.result.perm[i]]
        assert abs(a - b) <= 1e-5 * max(abs(a), abs(b)), (i, a, b)


def test_identity_order_matches_natural_order():
    """With perm = 0 .. d-1 the reordered entry points are the natural-order ones."""
    W0 = case_w(96, 384, np.float16, 85)
    Ho = O.hessian([case_x("ar1", 3000, 384, np.float32, 86)]).astype(np.float32)
    ident = dev(np.arange(384, dtype=np.int32))
    U1, l1, _ = G.gptq_prepare_hinv(dev(Ho), 0.01)
    U2, l2, _ = G.gptq_prepare_hinv_perm(dev(Ho), ident, 0.01)
    a = G.gptq_quantize_layer(dev(W0), U1, l1, 4, 128, 128)
    b = G.gptq_quantize_layer_perm(dev(W0), U2, l2, ident, 4, 128, 128)
    torch.cuda.synchronize()
    assert torch.equal(U1, U2) and torch.equal(l1, l2)
    for x, y in zip(a, (b[0], b[1], b[2], b[4])):
        assert torch.equal(x, y)
    np.testing.assert_array_equal(b[3].cpu().numpy(), np.arange(384) // 128)
