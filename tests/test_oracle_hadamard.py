"""Pins for the oracle's online Hadamard rotation of the activations.

The FLUTE page ("Maintenance & Community") lists Hadamard-transform support
without details; the reading is a block-diagonal, orthonormal Walsh-Hadamard
rotation of each activation row, matched by weights rotated offline, so that
(x H)(H W) = x W.  Pins: scipy's Hadamard matrix (a library routine),
hand-derived small cases, H H = I, norm preservation, block independence,
the rotated-product identity, and the one rounding to the activation dtype
against numpy's float16 conversion.
"""
import math

import numpy as np
import pytest
import scipy.linalg

F16, BF16 = 0, 1


def rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("b", [2, 4, 8, 16, 32, 64, 128, 256, 512])
def test_matches_library_hadamard_matrix(orc, b):
    M, K = 3, 2 * b
    x = rng(b).standard_normal((M, K))
    H = scipy.linalg.hadamard(b).astype(np.float64) / math.sqrt(b)
    ref = np.concatenate([x[:, j * b:(j + 1) * b] @ H.T for j in range(K // b)], axis=1)
    assert np.allclose(orc.hadamard(x, b), ref, rtol=1e-13, atol=1e-13)


def test_small_cases_by_hand(orc):
    a, c = 3.0, -1.25
    y = orc.hadamard(np.array([[a, c]]), 2)
    assert np.allclose(y, [[(a + c) / math.sqrt(2), (a - c) / math.sqrt(2)]], rtol=0, atol=1e-15)
    # unit vectors of size 4: column j of H4 / 2, entry i = (-1)^popcount(i & j) / 2
    e0 = orc.hadamard(np.array([[1.0, 0, 0, 0]]), 4)
    e3 = orc.hadamard(np.array([[0, 0, 0, 1.0]]), 4)
    e1 = orc.hadamard(np.array([[0, 1.0, 0, 0]]), 4)
    assert np.array_equal(e0, [[0.5, 0.5, 0.5, 0.5]])
    assert np.array_equal(e3, [[0.5, -0.5, -0.5, 0.5]])
    assert np.array_equal(e1, [[0.5, -0.5, 0.5, -0.5]])
    # a constant block maps to its first entry only
    y = orc.hadamard(np.full((1, 16), 2.0), 16)
    assert np.allclose(y, [[8.0] + [0.0] * 15], rtol=0, atol=1e-14)


@pytest.mark.parametrize("b", [16, 128, 512])
def test_involution_and_norm(orc, b):
    x = rng(7 + b).standard_normal((4, 4 * b))
    y = orc.hadamard(x, b)
    assert np.allclose(orc.hadamard(y, b), x, rtol=1e-12, atol=1e-12)
    for j in range(4):
        blk = slice(j * b, (j + 1) * b)
        assert np.allclose(np.linalg.norm(y[:, blk], axis=1), np.linalg.norm(x[:, blk], axis=1), rtol=1e-13)


def test_blocks_are_independent(orc):
    b, K = 32, 128
    x = rng(3).standard_normal((2, K))
    y = orc.hadamard(x, b)
    x2 = x.copy()
    x2[:, 32:64] = rng(4).standard_normal((2, 32))
    y2 = orc.hadamard(x2, b)
    assert np.array_equal(y[:, :32], y2[:, :32]) and np.array_equal(y[:, 64:], y2[:, 64:])
    assert not np.allclose(y[:, 32:64], y2[:, 32:64])
    # one block the size of the whole row = the full transform
    H = scipy.linalg.hadamard(K).astype(np.float64) / math.sqrt(K)
    assert np.allclose(orc.hadamard(x, K), x @ H.T, rtol=1e-13, atol=1e-13)


def test_rotated_product_identity(orc):
    """(x H)(H W) = x W: rotating the activations undoes weights rotated offline."""
    b, K, N = 64, 256, 24
    x = rng(11).standard_normal((5, K))
    W = rng(12).standard_normal((K, N))
    HW = orc.hadamard(W.T.copy(), b).T  # H W: rotate every column of W along K
    assert np.allclose(orc.hadamard(x, b) @ HW, x @ W, rtol=1e-12, atol=1e-11)


def test_rotate_x_rounds_once(orc):
    b, K = 128, 512
    x = rng(13).standard_normal((3, K)).astype(np.float16)
    bits = x.view(np.uint16)
    got = orc.rotate_x(bits, F16, b)
    ref = orc.hadamard(x.astype(np.float64), b).astype(np.float16).view(np.uint16)
    assert np.array_equal(got, ref)
    # bf16: against torch's float64 -> bfloat16 rounding
    import torch
    xb = torch.from_numpy(rng(14).standard_normal((3, K))).to(torch.bfloat16)
    xbits = xb.view(torch.int16).numpy().view(np.uint16)
    got = orc.rotate_x(xbits, BF16, b)
    yr = orc.hadamard(xb.double().numpy(), b)
    ref = torch.from_numpy(yr).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)


def test_rejects_bad_sizes(orc):
    from oracle import OracleError
    x = np.zeros((1, 96))
    with pytest.raises(OracleError):
        orc.hadamard(x, 64)      # 96 % 64
    with pytest.raises(OracleError):
        orc.hadamard(x, 48)      # not a power of two
