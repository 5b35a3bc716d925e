"""GPU parity of the activation-fused gate+up layer, h = SiLU(x.gate) * (x.up)
(Triton GPTQ page, "How It Works": fused feed-forward layers; the gated SiLU
is the reading of the activation the page leaves unnamed).

  * the interleaving repack is checked bit-exactly through the debug dequant
    (its columns come out as gate tile j, up tile j, ...);
  * wq_gemv_gate_up / wq_gemm_gate_up are checked element by element against
    the oracle's h with a bound derived from the plain product's bound B
    (5e-3 * max|y| + 1e-3 over the gate and up outputs y = x.W):
        |h' - h| <= (1.1 |u| + |SiLU(g)|) B + 1.1 B^2 + |h| 2^-p + 1e-6
    where 1.1 bounds |SiLU'|, g and u are the oracle's gate and up outputs,
    and 2^-p is the relative rounding of h to the activation dtype
    (p = 11 for fp16, 8 for bf16).  The fused kernels keep g and u in fp32,
    so their error is within B.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from _util import (TOL_ABS, TOL_REL, act_dtype, bits_to_tensor, oracle_y, tensor_bits, tensor_f64)

pytestmark = pytest.mark.gpu

MODES = [wl.SYM, wl.ZERO_F16, wl.ZERO_PACKED, wl.LUT]


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_w4a16_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def make(mode, bits, gs, K, N, seed, act_order=False):
    return wl.make_layer(K, N, bits, gs, mode, seed, act_order=act_order,
                         lut=wl.nf_table(bits) if mode == wl.LUT else None)


def repack_gate_up(wq, L, device="cuda"):
    q = bits_to_tensor(L.qweight, torch.int32, device)
    s = bits_to_tensor(L.scales, torch.float16, device)
    z = None
    if L.mode == wl.ZERO_F16 or L.mode in wl.FINE_ZERO_GROUP:
        z = bits_to_tensor(L.zeros, torch.float16, device)
    elif L.mode == wl.ZERO_PACKED:
        z = bits_to_tensor(L.zeros, torch.int32, device)
    lut = bits_to_tensor(L.lut, torch.float16, device) if L.lut is not None else None
    return wq.wq_repack_gate_up(q, s, z, L.mode, L.g_idx, L.K, L.N, L.bits, L.group_size, lut=lut)


def interleaved_columns(N):
    """Column order of a gate+up repack: gate tile j, then up tile j."""
    I = N // 2
    order = []
    for j in range(I // 16):
        order.extend(range(16 * j, 16 * j + 16))
        order.extend(range(I + 16 * j, I + 16 * j + 16))
    return np.array(order)


def gate_up_bound(y_gu, h_ref, dt):
    """Element-wise bound on |h' - h| (see the module docstring)."""
    I = y_gu.shape[1] // 2
    g, u = y_gu[:, :I], y_gu[:, I:]
    B = TOL_REL * float(np.max(np.abs(y_gu))) + TOL_ABS
    silu = g / (1.0 + np.exp(-g))
    rel = 2.0 ** -(11 if dt == wl.F16 else 8)
    return (1.1 * np.abs(u) + np.abs(silu)) * B + 1.1 * B * B + np.abs(h_ref) * rel + 1e-6


def check_gate_up(orc, wq, fn, L, M, dt, seed, cols=None):
    x_bits = wl.make_x(M, L.K, dt, seed)
    layer = repack_gate_up(wq, L)
    x = bits_to_tensor(x_bits, act_dtype(dt), "cuda")
    h = getattr(wq, fn)(x, layer)
    torch.cuda.synchronize()
    assert h.shape == (M, L.N // 2)
    I = L.N // 2
    if cols is None:
        cols = np.arange(I)
        got = tensor_f64(h)
    else:
        got = tensor_f64(h[:, torch.from_numpy(cols).long().cuda()])
    h_ref = orc.linear_gate_up(x_bits, dt, L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, M, L.N, L.K,
                               L.bits, L.group_size, cols)
    y_gu = oracle_y(orc, x_bits, dt, L, np.concatenate([cols, cols + I]).astype(np.int32))
    bound = gate_up_bound(y_gu, h_ref, dt)
    err = np.abs(got - h_ref)
    assert np.all(np.isfinite(got))
    bad = err > bound
    assert not bad.any(), (f"{fn}: {int(bad.sum())} outputs outside the bound, worst excess "
                           f"{float(np.max(err - bound)):.3e}")


DEQ_CASES = [(mode, bits, dt) for mode in MODES for bits in (2, 3, 4) for dt in (wl.F16, wl.BF16)]


@pytest.mark.parametrize("mode,bits,dt", DEQ_CASES)
def test_gate_up_repack_interleaves_tiles(orc, wq, mode, bits, dt):
    K, N = 512, 96
    print(f"[gate_up dequant] mode={mode} bits={bits} dt={dt}", flush=True)
    L = make(mode, bits, 128, K, N, 5000 + 97 * mode + 13 * bits + dt)
    w = wq.wq_dequant_debug(repack_gate_up(wq, L), act_dtype(dt))
    torch.cuda.synchronize()
    ref = orc.dequant(L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, K, N, bits, 128, dt)
    assert np.array_equal(tensor_bits(w), ref[:, interleaved_columns(N)])


GEMV_CASES = [(mode, bits, dt, gs, M, ao)
              for mode in MODES for bits in (2, 3, 4) for dt in (wl.F16, wl.BF16)
              for gs in (32, 128) for M in (1, 5, 8, 16, 32)
              for ao in ((False, True) if (gs == 32 and M == 1) else (False,))]


@pytest.mark.parametrize("mode,bits,dt,gs,M,ao", GEMV_CASES)
def test_gemv_gate_up_parity(orc, wq, mode, bits, dt, gs, M, ao):
    K, N = 1024, 192  # 4-8 k-tiles, 6 output tiles (12 column tiles)
    print(f"[gemv_gate_up] mode={mode} bits={bits} dt={dt} gs={gs} M={M} act_order={ao}", flush=True)
    L = make(mode, bits, gs, K, N, 6000 + 97 * mode + 13 * bits + 5 * dt + M + ao, act_order=ao)
    check_gate_up(orc, wq, "wq_gemv_gate_up", L, M, dt, 31 + M)


GEMM_CASES = [(mode, bits, dt, gs, M, ao)
              for mode in MODES for bits in (2, 3, 4) for dt in (wl.F16, wl.BF16)
              for gs in (32, -1) for M in (1, 70, 130)
              for ao in ((False, True) if (gs == 32 and M == 70) else (False,))]


@pytest.mark.parametrize("mode,bits,dt,gs,M,ao", GEMM_CASES)
def test_gemm_gate_up_parity(orc, wq, mode, bits, dt, gs, M, ao):
    K, N = 512, 448  # 2-4 k-tiles; 28 column tiles: the second 256-column block is ragged
    print(f"[gemm_gate_up] mode={mode} bits={bits} dt={dt} gs={gs} M={M} act_order={ao}", flush=True)
    L = make(mode, bits, gs, K, N, 7000 + 97 * mode + 13 * bits + 5 * dt + M + ao, act_order=ao)
    check_gate_up(orc, wq, "wq_gemm_gate_up", L, M, dt, 41 + M)


@pytest.mark.parametrize("mode,dt", [(wl.SYM, wl.F16), (wl.ZERO_F16, wl.BF16), (wl.LUT, wl.F16)])
def test_gemm_gate_up_k_split(orc, wq, mode, dt):
    """A narrow fused gate+up layer at small M splits K; the reduction kernel
    applies SiLU(gate) * up to the summed halves."""
    K, N = 2048, 448
    for gs in (128, -1):
        for M in (1, 33, 130):
            L = make(mode, 4, gs, K, N, 7500 + mode + dt + M)
            check_gate_up(orc, wq, "wq_gemm_gate_up", L, M, dt, 77 + M)


def test_gate_up_m_zero_and_layer_kind(wq):
    L = make(wl.SYM, 4, 128, 512, 64, 5)
    fused = repack_gate_up(wq, L)
    x = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    for fn in (wq.wq_gemv_gate_up, wq.wq_gemm_gate_up):
        assert fn(x, fused).shape == (0, 32)
    with pytest.raises(ValueError):
        wq.wq_gemv(x, fused)  # a gate+up buffer is not a plain layer


@pytest.mark.parametrize("fn", ["wq_gemv_gate_up", "wq_gemm_gate_up"])
def test_gate_up_deterministic(wq, fn):
    L = make(wl.ZERO_F16, 4, 128, 2048, 256, 6)
    layer = repack_gate_up(wq, L)
    x = bits_to_tensor(wl.make_x(4, 2048, wl.F16, 1), torch.float16, "cuda")
    h1 = getattr(wq, fn)(x, layer).clone()
    h2 = getattr(wq, fn)(x, layer)
    torch.cuda.synchronize()
    assert torch.equal(h1, h2)


@pytest.mark.parametrize("M", [1, 4, 16, 2048])
def test_gate_up_llama7b_full_size(orc, wq, M):
    """LLaMA-7B gate+up (4096 x 22016, int4, fp16 zero-points, group 128, fp16)
    at full size, through the launch shapes the benchmark times; the oracle
    computes a seeded sample of output columns."""
    cfg = wl.CONFIGS[2]
    L = cfg.layer("gate_up", 4, 128)
    print(f"[gate_up full] M={M}", flush=True)
    cols = wl.sample_cols(L.N // 2, 128 if M <= 16 else 32, seed=700 + M)
    fn = "wq_gemv_gate_up" if M <= 16 else "wq_gemm_gate_up"
    check_gate_up(orc, wq, fn, L, M, cfg.dtype, 900 + M, cols)
