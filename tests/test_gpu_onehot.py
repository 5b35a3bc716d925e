"""Which weights the products multiply: one-hot activations read them back.

With x = e_k (row k of the identity) the product y = x . W returns row k of
the weights the kernel actually multiplies, rounded once to the activation
dtype.  Wherever those weights are the dequantised weights the oracle defines
(RN(s * (q - z)) or RN(s * T[q]), one rounding) and the arithmetic after the
MFMA is exact for one-hot inputs, y must equal the oracle's dequantised
weights bit for bit:

  * the decode-sized product (wq_gemv) with the exact decode -- every bf16
    layer, and fp16 layers with scale groups under 128 rows;
  * the decode-sized product with fp16 activations and one group per 128 rows,
    which applies the scale after the MFMA: the one-hot sum is bias + q, the
    row-sum correction removes bias + z exactly, and s * (q - z) is exact in
    fp32 for the workloads' scales and zero-points (at most 22 significant
    bits), so the single rounding to fp16 gives the oracle's bits;
  * the large-M product (wq_gemm): the exact decode, and the fp16 forms with
    the scale in the epilogue (exact integer q - 8 times s in fp32) and with
    packed zero-points ((1024 + q) - (1024 + z) exact, then one fp16 product).

The documented exceptions form q - z in fp16 first and multiply
RN(s * RN(q - z)): the large-M fp16 product with fp16 zero-points (shared or
fine), and the decode-sized fp16 product with fine zero-points and one scale
group per 128 rows (the scale follows the MFMA; s * RN(q - z) is exact in
fp32).  Their bits are predicted here on the CPU from the canonical arrays, and
the positions where they differ from the oracle's weights can only be those
where q - z needs more than 11 significant bits; zero-points drawn from
U[0.3, 3.9] make that set non-empty for the large-M product.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from _util import act_dtype, repack_layer, tensor_bits

pytestmark = pytest.mark.gpu

K, N = 512, 64


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_w4a16_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def onehot_rows(rows, dtype):
    """x [len(rows)][K] with x[i][rows[i]] = 1."""
    x = torch.zeros((len(rows), K), dtype=dtype, device="cuda")
    x[torch.arange(len(rows)), torch.as_tensor(rows)] = 1
    return x


def product_rows(wq, fn, layer, dt, rows):
    x = onehot_rows(rows, act_dtype(dt))
    y = fn(x, layer)
    torch.cuda.synchronize()
    return tensor_bits(y)


def oracle_bits(orc, L, dt):
    return orc.dequant(L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, L.K, L.N, L.bits, L.group_size, dt)


# (mode, bits, group) with the decode each path takes for fp16 / bf16
CASES = [
    (wl.SYM, 4, -1), (wl.SYM, 4, 128), (wl.SYM, 4, 32), (wl.SYM, 3, 64), (wl.SYM, 2, 128),
    (wl.ZERO_F16, 4, 128), (wl.ZERO_F16, 4, 32), (wl.ZERO_F16, 2, 256),
    (wl.ZERO_PACKED, 4, 128), (wl.ZERO_PACKED, 4, 32), (wl.ZERO_PACKED, 3, 128),
    (wl.LUT, 4, 128), (wl.LUT, 4, 64), (wl.LUT, 2, 128),
    (wl.ZERO_F16_G8, 2, -1), (wl.ZERO_F16_G32, 4, 128), (wl.ZERO_F16_G16, 4, 64),
]


def make(mode, bits, gs, seed, zero_range=(6.0, 10.0)):
    return wl.make_layer(K, N, bits, gs, mode, seed, zero_range=zero_range)


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("mode,bits,gs", CASES)
def test_gemv_multiplies_the_oracle_weights(orc, wq, mode, bits, gs, dt):
    """Every decode-sized scheme (4, 8, 16 and 32 rows) returns the oracle's weight bits."""
    L = make(mode, bits, gs, seed=900 + 7 * mode + bits + max(gs, 0))
    layer = repack_layer(wq, L)
    ref = oracle_bits(orc, L, dt)
    if dt == wl.F16 and mode in wl.FINE_ZERO_GROUP and (gs == -1 or gs >= 128):
        # scale after the MFMA on RN(q - z): the two-step weights
        want, diff = fp16_two_step(orc, L)
        inexact = diff != diff.astype(np.float16).astype(np.float64)
        assert not ((want != ref) & ~inexact).any()
        ref = want
    for M in (4, 8, 16, 32):
        for k0 in range(0, K, M):
            rows = list(range(k0, k0 + M))
            got = product_rows(wq, wq.wq_gemv, layer, dt, rows)
            bad = np.argwhere(got != ref[rows])
            assert bad.size == 0, f"M={M} rows {k0}..: {len(bad)} weights differ, first at {bad[0]}"


def fp16_two_step(orc, L):
    """RN(s * RN(q - z)) in fp16 bits for a layer with fp16 zero-points (shared
    or per zero group), from the canonical arrays (numpy fp16 arithmetic: each
    operation on two fp16 values is exact in fp32 and rounded once)."""
    q = orc.unpack_codes(L.qweight, L.K, L.N, L.bits).astype(np.float16)
    gsz = L.K if L.group_size == -1 else L.group_size
    s = L.scales.view(np.float16)[np.arange(L.K) // gsz]
    zg = wl.FINE_ZERO_GROUP.get(L.mode, gsz)
    z = L.zeros.view(np.float16)[np.arange(L.K) // zg]
    d = (q - z).astype(np.float16)
    return (s * d).astype(np.float16).view(np.uint16), (q.astype(np.float64) - z.astype(np.float64))


@pytest.mark.parametrize("dt", [wl.F16, wl.BF16], ids=["f16", "bf16"])
@pytest.mark.parametrize("mode,bits,gs", CASES)
def test_gemm_multiplies_the_oracle_weights(orc, wq, mode, bits, gs, dt):
    """The large-M product at 64 rows (64 x 256 tiles) and 512 rows (128-row tiles)."""
    two_step = dt == wl.F16 and (mode == wl.ZERO_F16 or mode in wl.FINE_ZERO_GROUP)
    # fine-resolution zero-points make RN(q - z) inexact somewhere
    zr = (0.3, 3.9) if two_step else (6.0, 10.0)
    L = make(mode, bits, gs, seed=1900 + 7 * mode + bits + max(gs, 0), zero_range=zr)
    layer = repack_layer(wq, L)
    ref = oracle_bits(orc, L, dt)
    want = ref
    if two_step:
        want, diff = fp16_two_step(orc, L)
        inexact = diff != diff.astype(np.float16).astype(np.float64)
        moved = want != ref
        assert moved.any(), "the fine zero-points were meant to make some q - z inexact in fp16"
        # only positions whose q - z needs more than 11 significant bits can move
        assert not (moved & ~inexact).any()
    for rows in (list(range(64)), list(range(K))):
        got = product_rows(wq, wq.wq_gemm, layer, dt, rows)
        bad = np.argwhere(got != want[rows])
        assert bad.size == 0, f"M={len(rows)}: {len(bad)} weights differ, first at {bad[0]}"
