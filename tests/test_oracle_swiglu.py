"""Pins for the oracle's fused gate+up activation h = SiLU(g) * u.

The Triton GPTQ page ("How It Works") fuses the FFN input layers; the
activation is not named there and SiLU(v) = v * sigmoid(v) is the reading.
Pins: scipy's logistic function (a library routine), the identity
SiLU(v) - SiLU(-v) = v, closed values, and the fused product equal to the
two halves of one ordinary product.
"""
import numpy as np
import pytest
import scipy.special

import workloads as wl

F16, BF16 = 0, 1


def test_silu_matches_library_logistic(orc):
    v = np.concatenate([np.linspace(-40, 40, 4001), np.random.default_rng(0).standard_normal(10000) * 5])
    g = v.copy()
    u = np.ones_like(v)
    h = orc.swiglu(g, u)
    ref = v * scipy.special.expit(v)
    assert np.allclose(h, ref, rtol=1e-14, atol=1e-300)


def test_silu_identities(orc):
    v = np.random.default_rng(1).standard_normal(1000) * 8
    one = np.ones_like(v)
    assert np.allclose(orc.swiglu(v, one) - orc.swiglu(-v, one), v, rtol=1e-13, atol=1e-13)
    assert orc.lib().wqo_silu(0.0) == 0.0
    assert abs(orc.lib().wqo_silu(50.0) - 50.0) < 1e-15 * 50
    assert abs(orc.lib().wqo_silu(-50.0)) < 1e-18


def test_swiglu_scales_with_up(orc):
    g = np.random.default_rng(2).standard_normal(100)
    u = np.random.default_rng(3).standard_normal(100)
    assert np.allclose(orc.swiglu(g, 3.0 * u), 3.0 * orc.swiglu(g, u), rtol=1e-14)


@pytest.mark.parametrize("mode", [wl.SYM, wl.ZERO_F16, wl.LUT])
def test_fused_gate_up_equals_halves_of_one_product(orc, mode):
    M, K, I = 3, 256, 48
    L = wl.make_layer(K, 2 * I, 4, 64, mode, 11 + mode, lut=wl.nf_table(4) if mode == wl.LUT else None)
    x = wl.make_x(M, K, F16, 4)
    y = orc.linear(x, F16, L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, M, 2 * I, K, 4, 64)
    h = orc.linear_gate_up(x, F16, L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, M, 2 * I, K, 4, 64)
    g, u = y[:, :I], y[:, I:]
    assert np.array_equal(h, orc.swiglu(g, u))
    cols = np.array([5, 0, 47], np.int32)
    hc = orc.linear_gate_up(x, F16, L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, M, 2 * I, K, 4, 64, cols)
    assert np.array_equal(hc, h[:, cols])
