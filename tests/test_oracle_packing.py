"""Pins of the oracle's packed codes and dequantizing product (the consumer of the
loop's codes: itwiki "GPTQ", section "결과", reports kernels that unpack the
weights on the fly).  CPU only."""
import numpy as np
import pytest

import oracle as O
import workloads as wl


def _bigint_words(row, bits, words):
    """The same bitstream built as one Python integer: field i at bit bits*i."""
    v = 0
    for i, c in enumerate(row):
        v |= int(c) << (bits * i)
    return [(v >> (32 * k)) & 0xFFFFFFFF for k in range(words)]


@pytest.mark.parametrize("bits", [2, 3, 4, 8])
@pytest.mark.parametrize("d_col", [1, 11, 32, 45, 96])
def test_pack_matches_bigint_bitstream(bits, d_col):
    rng = np.random.default_rng(bits * 100 + d_col)
    codes = rng.integers(0, 1 << bits, (5, d_col)).astype(np.uint8)
    p = O.pack_codes(codes, bits)
    words = -(-d_col // 32) * bits
    assert p.shape == (5, words) and p.dtype == np.uint32
    for r in range(5):
        assert p[r].tolist() == _bigint_words(codes[r], bits, words)
    np.testing.assert_array_equal(O.unpack_codes(p, bits, d_col), codes)


def test_pack_hand_example_3bit():
    # codes 5, 3, 7, 1, 6, 2, 4, 0, 7, 7, 1 at 3 bits: 0b001_111_111_000_100_010_110_001_111_011_101
    row = [5, 3, 7, 1, 6, 2, 4, 0, 7, 7, 1]
    p = O.pack_codes(np.array([row], np.uint8), 3)
    assert p[0, 0] == 0b01_111_111_000_100_010_110_001_111_011_101    # code 10's low bits are 01
    assert p[0, 1] == 0b0                                            # its high bit is 0
    assert p.shape == (1, 3)


def test_pack_with_order_and_overflow():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 16, (4, 40)).astype(np.uint8)
    perm = rng.permutation(40)
    p = O.pack_codes(codes, 4, perm)
    np.testing.assert_array_equal(O.unpack_codes(p, 4, 40), codes[:, perm])
    with pytest.raises(ValueError):
        O.pack_codes(np.array([[8]], np.uint8), 3)


@pytest.mark.parametrize("bits,group,B", [(4, 0, 16), (3, 16, 16), (4, 32, 16), (2, 64, 64)])
def test_dequant_matmul_equals_x_what(bits, group, B):
    """The product from packed codes equals X What^T with the loop's own What."""
    w, x = wl.tiny_case(41 + bits, 24, 64, 400)
    sol = O.solve_layer(w, [x], bits, group, B)
    r = sol.result
    X = np.random.default_rng(5).standard_normal((3, 64))
    Y = O.dequant_matmul(O.pack_codes(r.codes, bits), bits, r.scales, r.zeros, group, X, 64)
    np.testing.assert_allclose(Y, X @ r.w_hat.T, rtol=1e-13, atol=1e-15)


def test_dequant_matmul_act_order():
    """Act-order codes packed in quantization order, with X gathered in that order,
    give X What^T in the original column order."""
    w, x = wl.tiny_case(51, 20, 64, 400)
    x = x * np.random.default_rng(52).uniform(0.3, 3.0, 64)[None, :]
    sol = O.solve_layer_act_order(w, [x], 4, 16, 16)
    r = sol.result
    X = np.random.default_rng(6).standard_normal((2, 64))
    packed = O.pack_codes(r.codes, 4, r.perm)
    Y = O.dequant_matmul(packed, 4, r.scales, r.zeros, 16, X, 64, perm=r.perm)
    np.testing.assert_allclose(Y, X @ r.w_hat.T, rtol=1e-13, atol=1e-15)
