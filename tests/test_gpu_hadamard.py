"""GPU parity of the online Hadamard rotation (wq_hadamard) and of the rotated
product x H -> wq_gemv / wq_gemm.

The rotation runs in fp32 butterflies and rounds once; the oracle sums in fp64
and rounds once.  Element-wise bound (b = block, S = sum of |x| over the
element's block, p = 11 for fp16 and 8 for bf16):
    |y' - y| <= (log2(b) + 2) 2^-24 S / sqrt(b) + 2^-(p-1) max(|y'|, |y|) + 2^-24
(fp32 rounding of each butterfly level and of the scale, then one unit in the
last place of the activation dtype between the two final roundings, plus the
fp16 subnormal quantum).  The product after the rotation meets the product's
own tolerance against the oracle product of the oracle's rotated activations.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from _util import act_dtype, bits_to_tensor, oracle_y, repack_layer, tensor_bits, tensor_f64, within_tolerance

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_w4a16_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def rotation_bound(x64, y_ref, y_gpu, b, dt):
    M, K = x64.shape
    S = np.repeat(np.abs(x64).reshape(M, K // b, b).sum(axis=2), b, axis=1)
    p = 11 if dt == wl.F16 else 8
    mag = np.maximum(np.abs(y_ref), np.abs(y_gpu))
    return (math.log2(b) + 2) * 2.0 ** -24 * S / math.sqrt(b) + 2.0 ** -(p - 1) * mag + 2.0 ** -24


def check_rotation(orc, wq, M, K, b, dt, seed, rows=None):
    x_bits = wl.make_x(M, K, dt, seed)
    x = bits_to_tensor(x_bits, act_dtype(dt), "cuda")
    y = wq.wq_hadamard(x, b)
    torch.cuda.synchronize()
    sel = slice(None) if rows is None else rows
    xs = x_bits[sel]
    ref_bits = orc.rotate_x(xs, dt, b)
    ref = orc.decode(ref_bits, dt)
    got = tensor_f64(y)[sel]
    bound = rotation_bound(orc.decode(xs, dt), ref, got, b, dt)
    err = np.abs(got - ref)
    assert np.all(err <= bound), f"{int((err > bound).sum())} elements outside the bound"
    # the two sides round the same real number; they agree on nearly every element
    same = float(np.mean(tensor_bits(y)[sel] == ref_bits))
    assert same > 0.99, f"only {same:.4f} of the elements are bit-equal"
    return x, y


@pytest.mark.parametrize("b", [2, 4, 8, 16, 32, 64, 128, 256, 512])
@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_rotation_parity(orc, wq, b, dt):
    M, K = 5, 1536  # 960 chunks of 8: four workgroups, the last one partial
    print(f"[hadamard] b={b} dt={dt} M={M} K={K}", flush=True)
    check_rotation(orc, wq, M, K, b, dt, 100 + b + dt)


def test_rotation_ragged_and_empty(orc, wq):
    # 5 x 384 = 240 chunks: one partial workgroup, a partial last wave
    check_rotation(orc, wq, 5, 384, 128, wl.F16, 3)
    x = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    assert wq.wq_hadamard(x, 128).shape == (0, 512)


def test_rotation_in_place_and_involution(wq):
    x_bits = wl.make_x(7, 4096, wl.F16, 9)
    x = bits_to_tensor(x_bits, torch.float16, "cuda")
    y = wq.wq_hadamard(x, 256)
    z = x.clone()
    wq.wq_hadamard(z, 256, out=z)
    torch.cuda.synchronize()
    assert torch.equal(y, z)
    back = wq.wq_hadamard(y, 256)
    torch.cuda.synchronize()
    # H H = I up to the two roundings
    assert torch.allclose(back.float(), x.float(), rtol=4e-3, atol=4e-3)


@pytest.mark.parametrize("M,K,b", [(16, 16384, 512), (1, 11008, 128), (2048, 4096, 128)])
def test_rotation_full_sizes(orc, wq, M, K, b):
    """Activation shapes of the benchmarked layers; large M checks a seeded
    sample of rows (rows are independent)."""
    rows = None if M <= 16 else np.sort(np.random.default_rng(M).choice(M, 64, replace=False))
    print(f"[hadamard full] M={M} K={K} b={b}", flush=True)
    check_rotation(orc, wq, M, K, b, wl.F16, 500 + M, rows)


@pytest.mark.parametrize("fn,M", [("wq_gemv", 1), ("wq_gemv", 16), ("wq_gemm", 130)])
@pytest.mark.parametrize("mode,dt", [(wl.ZERO_F16, wl.F16), (wl.LUT, wl.BF16)])
def test_rotated_product(orc, wq, fn, M, mode, dt):
    """x H through the product: within the product's tolerance of the oracle
    product of the oracle's rotated activations."""
    K, N, b = 1024, 96, 128
    L = wl.make_layer(K, N, 4, 128, mode, 77 + M, lut=wl.nf_table(4) if mode == wl.LUT else None)
    x_bits = wl.make_x(M, K, dt, 5 + M)
    x = bits_to_tensor(x_bits, act_dtype(dt), "cuda")
    layer = repack_layer(wq, L)
    y = getattr(wq, fn)(wq.wq_hadamard(x, b), layer)
    torch.cuda.synchronize()
    ref = oracle_y(orc, orc.rotate_x(x_bits, dt, b), dt, L)
    ok, err, bound = within_tolerance(tensor_f64(y), ref)
    assert ok, f"max error {err:.3e} > bound {bound:.3e}"
