"""Pins for the oracle's canonical unpacking (codes along K, zero-points along N).

The pages fix no bit layout (Marlin zero-point issue, efrantar's reply: weights
follow the kernel's own format), so the layout is a reading: each column is a
little-endian bit stream along K.  Pinned three ways: literal examples of the
reading (tests/golden/canonical_packing.txt), a second unpacker written here
with Python big integers, and the pack/unpack round trip.
"""
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "canonical_packing.txt")


def golden_cases():
    cases = []
    with open(GOLDEN) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            b, codes, words = [s.strip() for s in line.split("|")]
            cases.append((int(b), [int(c) for c in codes.split()], [int(w, 16) for w in words.split()]))
    return cases


@pytest.mark.parametrize("bits,codes,words", golden_cases())
def test_golden_examples(orc, bits, codes, words):
    qw = np.array(words, np.uint32).reshape(-1, 1)
    got = orc.unpack_codes(qw, len(codes), 1, bits)[:, 0]
    assert got.tolist() == codes
    assert orc.pack_codes(np.array(codes, np.uint8).reshape(-1, 1), bits)[:, 0].tolist() == words


def bigint_unpack(qweight, K, N, bits):
    """Independent reading: concatenate a column's words into one integer, word r
    at bit 32r, and cut it into bits-wide fields."""
    out = np.empty((K, N), np.uint8)
    for n in range(N):
        big = 0
        for r in range(qweight.shape[0]):
            big |= int(qweight[r, n]) << (32 * r)
        for k in range(K):
            out[k, n] = (big >> (bits * k)) & ((1 << bits) - 1)
    return out


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_unpack_matches_bigint_reading(orc, bits):
    rng = np.random.default_rng(bits)
    K, N = 96, 5
    qw = rng.integers(0, 1 << 32, size=(K * bits // 32, N), dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(orc.unpack_codes(qw, K, N, bits), bigint_unpack(qw, K, N, bits))


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_pack_unpack_round_trip(orc, bits):
    rng = np.random.default_rng(10 + bits)
    K, N = 256, 33
    codes = rng.integers(0, 1 << bits, size=(K, N)).astype(np.uint8)
    qw = orc.pack_codes(codes, bits)
    assert qw.shape == (K * bits // 32, N)
    assert np.array_equal(orc.unpack_codes(qw, K, N, bits), codes)
    # and words -> codes -> words is the identity too
    words = rng.integers(0, 1 << 32, size=qw.shape, dtype=np.uint64).astype(np.uint32)
    assert np.array_equal(orc.pack_codes(orc.unpack_codes(words, K, N, bits), bits), words)


@pytest.mark.parametrize("bits", [2, 3, 4])
def test_zero_points_unpack_matches_bigint_reading(orc, bits):
    rng = np.random.default_rng(20 + bits)
    G, N = 3, 64
    zp = rng.integers(0, 1 << 32, size=(G, N * bits // 32), dtype=np.uint64).astype(np.uint32)
    got = orc.unpack_zeros(zp, G, N, bits)
    # row g is a bit stream along N: same big-integer reading, transposed roles
    ref = bigint_unpack(zp.T.copy(), N, G, bits).T
    assert np.array_equal(got, ref)
    assert np.array_equal(orc.pack_zeros(got, bits), zp)


def test_rejects_bad_shapes(orc):
    with pytest.raises(orc.OracleError):
        orc.unpack_codes(np.zeros((1, 1), np.uint32), 12, 1, 4)  # K*bits not a multiple of 32
    with pytest.raises(orc.OracleError):
        orc.unpack_codes(np.zeros((5, 1), np.uint32), 32, 1, 5)  # bits outside {2,3,4}
