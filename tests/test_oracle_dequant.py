"""Pins for the oracle's dequantisation w = RN_dtype(s * (q - z)) or RN_dtype(s * T[q]).

Sources: symmetric = zero-point fixed at the middle of the code range, stored
zero-points in fp16 or quantised, scales per group or per column (Marlin
zero-point issue, efrantar and mobicham); table value times scale (FLUTE page,
"How It Works"); act-order groups via g_idx (Triton GPTQ page, "Limitations &
Caveats").

Pins: the closed form evaluated here in exact rational arithmetic (fractions)
with the library rounding of numpy / torch; the identities the pages imply
(symmetric == fp16 zero 2^(b-1) == packed zero 2^(b-1); the integer-grid table
== symmetric; group = K == column-wise; identity g_idx == no g_idx).
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

import workloads as wl

F16, BF16 = 0, 1


def bigint_codes(qweight, K, N, bits):
    out = np.empty((K, N), np.int64)
    for n in range(N):
        big = 0
        for r in range(qweight.shape[0]):
            big |= int(qweight[r, n]) << (32 * r)
        for k in range(K):
            out[k, n] = (big >> (bits * k)) & ((1 << bits) - 1)
    return out


def bigint_zero_codes(zp, G, N, bits):
    out = np.empty((G, N), np.int64)
    for g in range(G):
        big = 0
        for r in range(zp.shape[1]):
            big |= int(zp[g, r]) << (32 * r)
        for n in range(N):
            out[g, n] = (big >> (bits * n)) & ((1 << bits) - 1)
    return out


def f16val(h):
    return Fraction(float(np.array([h], np.uint16).view(np.float16)[0]))


def round_exact(vals, dtype: int) -> np.ndarray:
    """Library rounding of exact rationals that fit in fp32 (as every value of
    these workloads does): numpy float64 -> float16, torch float32 -> bfloat16."""
    d = np.array([float(e) for e in vals], np.float64)
    assert all(Fraction(float(a)) == e for a, e in zip(d, vals))
    if dtype == F16:
        return d.astype(np.float16).view(np.uint16)
    f = d.astype(np.float32)
    assert np.array_equal(f.astype(np.float64), d)
    return torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def closed_form(L: wl.Layer, dtype: int) -> np.ndarray:
    K, N, b = L.K, L.N, L.bits
    q = bigint_codes(L.qweight, K, N, b)
    zc = bigint_zero_codes(L.zeros, L.G, N, b) if L.mode == wl.ZERO_PACKED else None
    vals = []
    for k in range(K):
        g = int(L.g_idx[k]) if L.g_idx is not None else (0 if L.group_size == -1 else k // L.group_size)
        for n in range(N):
            s = f16val(L.scales[g, n])
            if L.mode == wl.LUT:
                e = s * f16val(L.lut[q[k, n]])
            else:
                if L.mode == wl.SYM:
                    z = Fraction(1 << (b - 1))
                elif L.mode == wl.ZERO_F16:
                    z = f16val(L.zeros[g, n])
                elif L.mode in wl.FINE_ZERO_GROUP:
                    z = f16val(L.zeros[k // wl.FINE_ZERO_GROUP[L.mode], n])
                else:
                    z = Fraction(int(zc[g, n]))
                e = s * (int(q[k, n]) - z)
            vals.append(e)
    return round_exact(vals, dtype).reshape(K, N)


def oracle_dequant(orc, L, dtype):
    return orc.dequant(L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, L.K, L.N, L.bits,
                       L.group_size, dtype)


CASES = [(mode, bits, dtype, gs, ao)
         for mode in (wl.SYM, wl.ZERO_F16, wl.ZERO_PACKED, wl.LUT, wl.ZERO_F16_G8, wl.ZERO_F16_G16,
                      wl.ZERO_F16_G32)
         for bits in (2, 3, 4)
         for dtype in (F16, BF16)
         for gs, ao in ((32, False), (-1, False), (32, True))]


@pytest.mark.parametrize("mode,bits,dtype,gs,ao", CASES)
def test_dequant_closed_form(orc, mode, bits, dtype, gs, ao):
    K, N = 64, 32
    seed = 100 * mode + 10 * bits + dtype + (5 if ao else 0) + (3 if gs == -1 else 0)
    L = wl.make_layer(K, N, bits, gs, mode, seed, act_order=ao,
                      lut=wl.nf_table(bits) if mode == wl.LUT else None)
    assert np.array_equal(oracle_dequant(orc, L, dtype), closed_form(L, dtype))


@pytest.mark.parametrize("fine", [wl.ZERO_F16_G8, wl.ZERO_F16_G16, wl.ZERO_F16_G32])
@pytest.mark.parametrize("gs", [32, 64, -1])
def test_fine_zero_groups_reduce_to_shared_groups(orc, fine, gs):
    """Zero-points with their own group (Marlin zero-point issue, mobicham's
    reply) that repeat the value of the scale group's zero-point give exactly
    the fp16-zero mode with one zero-point per scale group."""
    K, N = 128, 24
    coarse = wl.make_layer(K, N, 4, gs, wl.ZERO_F16, 50 + gs % 7)
    zg = wl.FINE_ZERO_GROUP[fine]
    gsz = K if gs == -1 else gs
    rows = np.arange(0, K, zg) // gsz  # scale group of each zero group
    fine_layer = wl.Layer(K, N, 4, gs, fine, coarse.qweight, coarse.scales, coarse.zeros[rows])
    for dt in (F16, BF16):
        assert np.array_equal(oracle_dequant(orc, fine_layer, dt), oracle_dequant(orc, coarse, dt))


def test_fine_zero_group_changes_within_a_scale_group(orc):
    """One zero-point per 8 rows under a per-column scale: changing one
    zero-point changes exactly its 8 rows of its column."""
    K, N = 64, 8
    L = wl.make_layer(K, N, 2, -1, wl.ZERO_F16_G8, 3)
    base = oracle_dequant(orc, L, F16)
    z2 = L.zeros.copy()
    z2[3, 5] = wl.to_f16_bits(np.array([2.5]))[0]
    L2 = wl.Layer(K, N, 2, -1, wl.ZERO_F16_G8, L.qweight, L.scales, z2)
    diff = oracle_dequant(orc, L2, F16) != base
    assert not diff[:, :5].any() and not diff[:, 6:].any()
    assert not diff[:24, 5].any() and not diff[32:, 5].any()


def test_dequant_subnormal_and_overflow_closed_form(orc):
    # tiny scales give fp16 subnormals (kept, not flushed); huge scales overflow to inf
    K, N = 32, 8
    L = wl.make_layer(K, N, 4, 32, wl.SYM, 7)
    L.scales = wl.to_f16_bits(np.full((1, N), 2.0 ** -20))
    L.scales[0, :4] = wl.to_f16_bits(np.full(4, 60000.0))
    got = oracle_dequant(orc, L, F16)
    assert np.array_equal(got, closed_form(L, F16))
    q = bigint_codes(L.qweight, K, N, 4)
    big = got[:, :4]
    assert np.all((big == 0x7C00) == (q[:, :4] - 8 >= 2))
    assert np.all((big == 0xFC00) == (q[:, :4] - 8 <= -2))
    small = got[:, 4:]
    assert np.any((small & 0x7C00) == 0)  # subnormal exponent field present


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_symmetric_equals_zero_point_at_midpoint(orc, bits, dtype):
    """Marlin zero-point issue (efrantar): symmetric is a zero-point fixed at the middle."""
    K, N = 128, 32
    L = wl.make_layer(K, N, bits, 32, wl.SYM, 40 + bits)
    ref = oracle_dequant(orc, L, dtype)
    zf = wl.make_layer(K, N, bits, 32, wl.SYM, 40 + bits)
    zf.mode = wl.ZERO_F16
    zf.zeros = wl.to_f16_bits(np.full((L.G, N), float(1 << (bits - 1))))
    assert np.array_equal(oracle_dequant(orc, zf, dtype), ref)
    zp = wl.make_layer(K, N, bits, 32, wl.SYM, 40 + bits)
    zp.mode = wl.ZERO_PACKED
    zp.zeros = orc.pack_zeros(np.full((L.G, N), 1 << (bits - 1), np.uint8), bits)
    assert np.array_equal(oracle_dequant(orc, zp, dtype), ref)


@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dtype", [F16, BF16])
def test_integer_grid_table_equals_symmetric(orc, bits, dtype):
    """FLUTE page ("How It Works"): value = table entry times scale; with the table
    T[i] = i - 2^(b-1) this is exactly the symmetric uniform dequant."""
    K, N = 128, 32
    L = wl.make_layer(K, N, bits, 64, wl.SYM, 60 + bits)
    ref = oracle_dequant(orc, L, dtype)
    L.mode = wl.LUT
    L.lut = wl.uniform_table(bits)
    assert np.array_equal(oracle_dequant(orc, L, dtype), ref)


@pytest.mark.parametrize("mode", [wl.SYM, wl.ZERO_F16, wl.ZERO_PACKED, wl.LUT])
def test_group_of_whole_K_equals_column_wise(orc, mode):
    K, N = 256, 16
    L = wl.make_layer(K, N, 4, -1, mode, 80 + mode, lut=wl.nf_table(4) if mode == wl.LUT else None)
    ref = oracle_dequant(orc, L, F16)
    L.group_size = K
    assert np.array_equal(oracle_dequant(orc, L, F16), ref)


@pytest.mark.parametrize("mode", [wl.SYM, wl.ZERO_F16, wl.ZERO_PACKED, wl.LUT])
def test_identity_g_idx_equals_no_g_idx(orc, mode):
    K, N = 256, 16
    L = wl.make_layer(K, N, 4, 64, mode, 90 + mode, lut=wl.nf_table(4) if mode == wl.LUT else None)
    ref = oracle_dequant(orc, L, BF16)
    L.g_idx = (np.arange(K) // 64).astype(np.int32)
    assert np.array_equal(oracle_dequant(orc, L, BF16), ref)


def test_g_idx_selects_the_group(orc):
    # a g_idx that sends every row to group 1 must use only scale row 1
    K, N = 64, 8
    L = wl.make_layer(K, N, 4, 32, wl.SYM, 3)
    L.g_idx = np.ones(K, np.int32)
    got = oracle_dequant(orc, L, F16)
    L2 = wl.make_layer(K, N, 4, 32, wl.SYM, 3)
    L2.scales = np.repeat(L.scales[1:2], 2, axis=0)
    assert np.array_equal(got, oracle_dequant(orc, L2, F16))


def test_rejects_inconsistent_arguments(orc):
    L = wl.make_layer(128, 8, 4, 32, wl.SYM, 1)
    with pytest.raises(orc.OracleError):   # K not a multiple of the group size
        orc.dequant(L.qweight, L.scales, None, wl.SYM, None, None, 128, 8, 4, 48, F16)
    with pytest.raises(orc.OracleError):   # table mode without a table
        orc.dequant(L.qweight, L.scales, None, wl.LUT, None, None, 128, 8, 4, 32, F16)
    with pytest.raises(orc.OracleError):   # g_idx out of range
        orc.dequant(L.qweight, L.scales, None, wl.SYM, None, np.full(128, 4, np.int32), 128, 8, 4, 32, F16)
