"""GPU parity on seeded random problems: code width, mode (all seven, fine
zero-point groups included), activation dtype, group size, act-order, K, N and
M drawn together, so that combinations the structured tests do not list (odd
tile counts, ragged row blocks, K splits at odd slice counts, two row blocks
with a partial second one, tables with tiny N ...) meet the oracle as well.

A second set draws deeper and wider layers.  Each case checks
wq_dequant_debug bit-exactly and the product through the
entry point linear() picks, plus the other entry point when both accept M,
against max|y - y_ref| <= 5e-3 * max|y_ref| + 1e-3.
"""
import math

import numpy as np
import pytest
import torch

import workloads as wl
from _util import act_dtype, bits_to_tensor, oracle_y, repack_layer, tensor_bits, tensor_f64, within_tolerance

pytestmark = pytest.mark.gpu

MODES = [wl.SYM, wl.ZERO_F16, wl.ZERO_PACKED, wl.LUT, wl.ZERO_F16_G8, wl.ZERO_F16_G16, wl.ZERO_F16_G32]
M_CHOICES = [1, 2, 3, 4, 5, 7, 8, 9, 13, 16, 17, 23, 31, 32, 33, 50, 64, 65, 100, 129, 257]


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_w4a16_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def draw(seed, base=90_000, kmax=2560, nmax_tiles=48, work=120_000_000):
    """One valid random problem (re-drawn until the layer is supported)."""
    rng = np.random.Generator(np.random.PCG64(base + seed))
    while True:
        bits = int(rng.choice([2, 3, 4]))
        kt = 256 if bits == 2 else 128
        mode = int(rng.choice(MODES))
        dt = int(rng.choice([wl.F16, wl.BF16]))
        groups = [-1] + [g for g in (32, 64, 128, 256, 512) if g % kt == 0 or kt % g == 0]
        gs = int(rng.choice(groups))
        unit = kt if gs == -1 else kt * gs // math.gcd(kt, gs)
        K = unit * int(rng.integers(1, max(2, kmax // unit) + 1))
        N = 16 * int(rng.integers(1, nmax_tiles + 1))
        if mode == wl.ZERO_PACKED and (N * bits) % 32:
            continue
        fine = mode in wl.FINE_ZERO_GROUP
        act_order = bool(gs != -1 and not fine and rng.random() < 0.3)
        M = int(rng.choice(M_CHOICES))
        if M * N * K > work:
            continue
        return dict(bits=bits, mode=mode, dt=dt, gs=gs, K=K, N=N, M=M, act_order=act_order)


# seed 388 (bf16, 4-bit symmetric, group -1, K = 2048, N = 688, M = 3) exceeded
# the tolerance when the decode-sized product multiplied unrounded bf16 weights
@pytest.mark.parametrize("seed", list(range(150)) + [388])
def test_random_problem(orc, wq, seed):
    check(orc, wq, seed, draw(seed))


@pytest.mark.parametrize("seed", range(100))
def test_random_problem_large(orc, wq, seed):
    """Deeper and wider layers (K up to 16384, N up to 4096): long k-loops,
    K splits of many slices, many column blocks."""
    check(orc, wq, seed, draw(seed, base=70_000, kmax=16384, nmax_tiles=256, work=400_000_000))


def check(orc, wq, seed, p):
    print(f"[random] seed={seed} {p}", flush=True)
    L = wl.make_layer(p["K"], p["N"], p["bits"], p["gs"], p["mode"], 500 + seed, act_order=p["act_order"],
                      lut=wl.nf_table(p["bits"]) if p["mode"] == wl.LUT else None)
    layer = repack_layer(wq, L)
    dt = p["dt"]
    w = wq.wq_dequant_debug(layer, act_dtype(dt))
    torch.cuda.synchronize()
    ref_w = orc.dequant(L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, L.K, L.N, L.bits, L.group_size, dt)
    assert np.array_equal(tensor_bits(w), ref_w)
    M = p["M"]
    x_bits = wl.make_x(M, L.K, dt, 60 + seed)
    x = bits_to_tensor(x_bits, act_dtype(dt), "cuda")
    ref = oracle_y(orc, x_bits, dt, L)
    fns = [wq.wq_gemm] + ([wq.wq_gemv] if M <= 32 else [])
    ys = {"linear": wq.linear(x, layer)}
    for fn in fns:
        ys[fn.__name__] = fn(x, layer)
    torch.cuda.synchronize()
    for name, y in ys.items():
        ok, err, bound = within_tolerance(tensor_f64(y), ref)
        assert ok, f"{name}: max error {err:.3e} > bound {bound:.3e}"
