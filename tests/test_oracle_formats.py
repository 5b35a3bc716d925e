"""Pins for the oracle's number formats (fp16 / bf16 decode and RNE encode).

The dequantised weight is one round-to-nearest-even of an exact real to the
activation dtype, so the converters decide every dequant bit.  They are checked
against library routines (numpy's direct float64 -> float16, torch's float32 ->
bfloat16) and against closed forms (exhaustive round trips, exact midpoints).
"""
import numpy as np
import pytest
import torch

F16, BF16 = 0, 1


def all_f16_finite():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (h >> 10) & 0x1F
    return h[e != 31]


def all_bf16_finite():
    h = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    e = (h >> 7) & 0xFF
    return h[e != 255]


def test_f16_decode_every_pattern_matches_numpy(orc):
    h = all_f16_finite()
    got = orc.decode(h, F16)
    ref = h.view(np.float16).astype(np.float64)
    assert np.array_equal(got, ref)


def test_f16_decode_inf_nan(orc):
    got = orc.decode(np.array([0x7C00, 0xFC00, 0x7E00], np.uint16), F16)
    assert got[0] == np.inf and got[1] == -np.inf and np.isnan(got[2])


def test_f16_round_trip_every_pattern(orc):
    h = all_f16_finite()
    assert np.array_equal(orc.encode(orc.decode(h, F16), F16), h)


def test_f16_encode_matches_numpy_on_random_doubles(orc):
    rng = np.random.default_rng(11)
    # magnitudes from deep subnormal to overflow, random mantissas
    v = rng.uniform(1, 2, 200000) * np.exp2(rng.integers(-30, 18, 200000)) * rng.choice([-1, 1], 200000)
    got = orc.encode(v, F16)
    with np.errstate(over="ignore"):
        ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)


def test_f16_midpoints_round_to_even(orc):
    # exact midpoint between consecutive finite positive fp16 values -> the even one
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    a = h.view(np.float16).astype(np.float64)
    b = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = (a + b) / 2  # exact in fp64
    got = orc.encode(mid, F16)
    expect = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(got, expect)
    # and just above / below the midpoint go to the nearer neighbour
    assert np.array_equal(orc.encode(np.nextafter(mid, np.inf), F16), (h + 1).astype(np.uint16))
    assert np.array_equal(orc.encode(np.nextafter(mid, -np.inf), F16), h)


def test_f16_overflow_and_subnormal_edges(orc):
    enc = lambda v: int(orc.encode(np.array([v]), F16)[0])
    assert enc(65504.0) == 0x7BFF
    assert enc(65519.999) == 0x7BFF
    assert enc(65520.0) == 0x7C00          # halfway to 2^16 rounds to even -> overflow
    assert enc(-1e9) == 0xFC00
    assert enc(2.0 ** -24) == 0x0001        # smallest subnormal
    assert enc(2.0 ** -25) == 0x0000        # tie with zero -> even (zero)
    assert enc(1.5 * 2.0 ** -25) == 0x0001
    assert enc(-0.0) == 0x8000


def bf16_from_bits(h):
    return torch.from_numpy(h.astype(np.int16)).view(torch.bfloat16).double().numpy()


def test_bf16_decode_every_pattern_matches_torch(orc):
    h = all_bf16_finite()
    assert np.array_equal(orc.decode(h, BF16), bf16_from_bits(h))


def test_bf16_round_trip_every_pattern(orc):
    h = all_bf16_finite()
    assert np.array_equal(orc.encode(orc.decode(h, BF16), BF16), h)


def test_bf16_encode_matches_torch_on_fp32_values(orc):
    # values exactly representable in fp32 (like every exact dequant product), so
    # torch's single float32 -> bfloat16 RNE rounding is the reference
    rng = np.random.default_rng(12)
    v = (rng.uniform(1, 2, 200000) * np.exp2(rng.integers(-140, 127, 200000))).astype(np.float32)
    v = v * rng.choice([-1, 1], 200000).astype(np.float32)
    got = orc.encode(v.astype(np.float64), BF16)
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_bf16_midpoints_round_to_even(orc):
    h = np.arange(0, 0x7F7F, 7, dtype=np.uint16)
    a = bf16_from_bits(h)
    b = bf16_from_bits((h + 1).astype(np.uint16))
    mid = (a + b) / 2
    expect = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)
    assert np.array_equal(orc.encode(mid, BF16), expect)


def test_bf16_overflow_edge(orc):
    enc = lambda v: int(orc.encode(np.array([v]), BF16)[0])
    mx = (2 - 2.0 ** -7) * 2.0 ** 127
    assert enc(mx) == 0x7F7F
    assert enc((2 - 2.0 ** -8) * 2.0 ** 127) == 0x7F80   # tie, rounds to even -> 2^128 -> inf
    assert enc(np.nextafter((2 - 2.0 ** -8) * 2.0 ** 127, 0)) == 0x7F7F
