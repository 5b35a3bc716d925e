"""Pins for the oracle's product y = x . dequant(W) (fp64, k ascending).

The product is a plain matrix-vector / matrix-matrix product over the
dequantised weights (exllama bandwidth discussion, GPTQ paper quote; Triton
GPTQ page, "How It Works").  Pins: exact rational brute force on tiny shapes,
numpy's fp64 matmul on mid shapes, a closed form, act-order permutation
invariance, column subsets, and N-concatenation (fused QKV / gate+up, Triton
GPTQ page, "How It Works") equal to separate products.
"""
from fractions import Fraction

import numpy as np
import pytest

import workloads as wl

F16, BF16 = 0, 1


def lin(orc, x, dtype, L, M, cols=None):
    return orc.linear(x, dtype, L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, M, L.N, L.K,
                      L.bits, L.group_size, cols)


def deq(orc, L, dtype):
    return orc.dequant(L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, L.K, L.N, L.bits,
                       L.group_size, dtype)


@pytest.mark.parametrize("mode,bits,dtype", [(wl.SYM, 4, F16), (wl.ZERO_F16, 3, F16),
                                             (wl.ZERO_PACKED, 2, BF16), (wl.LUT, 4, BF16),
                                             (wl.ZERO_F16_G8, 2, F16), (wl.ZERO_F16_G16, 3, BF16)])
def test_brute_force_exact_sum(orc, mode, bits, dtype):
    M, K, N = 3, 64, 16
    L = wl.make_layer(K, N, bits, 32, mode, 7 + mode, lut=wl.nf_table(bits) if mode == wl.LUT else None)
    x = wl.make_x(M, K, dtype, 3)
    y = lin(orc, x, dtype, L, M)
    # exact rationals of the decoded operands, summed exactly
    xf = [[Fraction(v) for v in row] for row in orc.decode(x, dtype).tolist()]
    wf = [[Fraction(v) for v in row] for row in orc.decode(deq(orc, L, dtype), dtype).tolist()]
    for m in range(M):
        for n in range(N):
            exact = sum(xf[m][k] * wf[k][n] for k in range(K))
            scale = sum(abs(xf[m][k] * wf[k][n]) for k in range(K))
            assert abs(Fraction(y[m, n]) - exact) <= Fraction(1, 10 ** 12) * scale


def test_matches_numpy_matmul(orc):
    M, K, N = 7, 512, 96
    L = wl.make_layer(K, N, 4, 128, wl.ZERO_F16, 5, act_order=True)
    x = wl.make_x(M, K, F16, 4)
    y = lin(orc, x, F16, L, M)
    w = orc.decode(deq(orc, L, F16), F16)
    xd = orc.decode(x, F16)
    ref = xd @ w
    bound = 1e-12 * (np.abs(xd) @ np.abs(w))
    assert np.all(np.abs(y - ref) <= bound)


def test_closed_form_constant_weights(orc):
    # every code q = 11, scale 0.5, symmetric zero 8, x = 1: y = K * 0.5 * 3 exactly
    K, N = 256, 16
    codes = np.full((K, N), 11, np.uint8)
    L = wl.make_layer(K, N, 4, 64, wl.SYM, 0)
    L.qweight = orc.pack_codes(codes, 4)
    L.scales = wl.to_f16_bits(np.full((K // 64, N), 0.5))
    x = wl.to_f16_bits(np.ones((2, K)))
    y = lin(orc, x, F16, L, 2)
    assert np.all(y == K * 1.5)
    # and x = -1 on the odd rows only: y = 0
    x2 = wl.to_f16_bits(np.where(np.arange(K) % 2, -1.0, 1.0)[None, :])
    assert np.all(lin(orc, x2, F16, L, 1) == 0.0)


@pytest.mark.parametrize("mode", [wl.ZERO_F16, wl.ZERO_PACKED, wl.LUT])
def test_act_order_permutation_invariance(orc, mode):
    """Reordering the input rows of x, W and g_idx together leaves y unchanged
    (only the fp64 summation order moves)."""
    M, K, N, bits = 4, 256, 24, 4
    L = wl.make_layer(K, N, bits, 32, mode, 30 + mode, act_order=True,
                      lut=wl.nf_table(bits) if mode == wl.LUT else None)
    x = wl.make_x(M, K, BF16, 9)
    y = lin(orc, x, BF16, L, M)
    perm = np.random.default_rng(1).permutation(K)
    codes = orc.unpack_codes(L.qweight, K, N, bits)
    P = wl.Layer(K, N, bits, L.group_size, mode, orc.pack_codes(codes[perm], bits), L.scales,
                 L.zeros, L.lut, L.g_idx[perm].copy())
    yp = lin(orc, x[:, perm].copy(), BF16, P, M)
    assert np.allclose(yp, y, rtol=1e-12, atol=1e-12 * np.max(np.abs(y)))


def test_column_subset_equals_full(orc):
    M, K, N = 2, 256, 64
    L = wl.make_layer(K, N, 3, 64, wl.LUT, 2, lut=wl.nf_table(3))
    x = wl.make_x(M, K, BF16, 1)
    full = lin(orc, x, BF16, L, M)
    cols = np.array([63, 0, 17, 17, 40], np.int32)
    assert np.array_equal(lin(orc, x, BF16, L, M, cols), full[:, cols])


def test_fused_concatenation_equals_separate(orc):
    """Fused QKV / gate+up: one product over N-concatenated weights equals the
    concatenation of the separate products, bit for bit."""
    M, K = 3, 256
    parts = [wl.make_layer(K, n, 4, 128, wl.ZERO_F16, 50 + i) for i, n in enumerate((32, 16, 48))]
    x = wl.make_x(M, K, F16, 2)
    fused = wl.Layer(K, 96, 4, 128, wl.ZERO_F16,
                     np.concatenate([p.qweight for p in parts], axis=1),
                     np.concatenate([p.scales for p in parts], axis=1),
                     np.concatenate([p.zeros for p in parts], axis=1))
    y = lin(orc, x, F16, fused, M)
    sep = np.concatenate([lin(orc, x, F16, p, M) for p in parts], axis=1)
    assert np.array_equal(y, sep)


def test_empty_m(orc):
    L = wl.make_layer(128, 16, 4, 32, wl.SYM, 0)
    y = orc.linear(np.zeros((0, 128), np.uint16), F16, L.qweight, L.scales, None, wl.SYM, None, None,
                   0, 16, 128, 4, 32)
    assert y.shape == (0, 16)
