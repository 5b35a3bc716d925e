"""GPU parity of the fp16 zero-points with their own 8/16/32-row groups
(Marlin zero-point issue, mobicham's reply: zero-point and scale group sizes
chosen apart, e.g. per-column scales with a zero-point every 8 rows).

  * wq_dequant_debug is bit-exact with the oracle;
  * wq_gemv / wq_gemm (and the fused gate+up variants) meet
    max|y - y_ref| <= 5e-3 max|y_ref| + 1e-3 against the oracle;
  * act-order is rejected (the zero groups follow the original row order).
"""
import numpy as np
import pytest
import torch

import workloads as wl
from _util import act_dtype, bits_to_tensor, oracle_y, repack_layer, tensor_bits, tensor_f64, within_tolerance

pytestmark = pytest.mark.gpu

FINE = [wl.ZERO_F16_G8, wl.ZERO_F16_G16, wl.ZERO_F16_G32]


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_w4a16_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


def groups_for(bits):
    kt = 256 if bits == 2 else 128
    return [g for g in (32, 128, 256, -1) if g == -1 or g % kt == 0 or kt % g == 0]


@pytest.mark.parametrize("mode", FINE)
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_fine_dequant_bit_exact(orc, wq, mode, bits, dt):
    K, N = 512, 64
    for gs in groups_for(bits):
        print(f"[fine dequant] mode={mode} bits={bits} dt={dt} gs={gs}", flush=True)
        L = wl.make_layer(K, N, bits, gs, mode, 11 * mode + bits + dt + (gs if gs > 0 else 1))
        w = wq.wq_dequant_debug(repack_layer(wq, L), act_dtype(dt))
        torch.cuda.synchronize()
        ref = orc.dequant(L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, K, N, bits, gs, dt)
        got = tensor_bits(w)
        assert np.array_equal(got, ref), f"gs={gs}: {np.count_nonzero(got != ref)} mismatching weights"


def check(orc, wq, fn, L, M, dt, seed):
    x_bits = wl.make_x(M, L.K, dt, seed)
    x = bits_to_tensor(x_bits, act_dtype(dt), "cuda")
    y = getattr(wq, fn)(x, repack_layer(wq, L))
    torch.cuda.synchronize()
    ok, err, bound = within_tolerance(tensor_f64(y), oracle_y(orc, x_bits, dt, L))
    assert ok, f"{fn}: max error {err:.3e} > bound {bound:.3e}"


@pytest.mark.parametrize("mode", FINE)
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
@pytest.mark.parametrize("gs", [128, -1])
def test_fine_gemv_parity(orc, wq, mode, bits, dt, gs):
    K, N = 1024, 96
    for M in (1, 3, 5, 16, 17, 32):
        print(f"[fine gemv] mode={mode} bits={bits} dt={dt} gs={gs} M={M}", flush=True)
        L = wl.make_layer(K, N, bits, gs, mode, 300 + 7 * mode + bits + dt + M)
        check(orc, wq, "wq_gemv", L, M, dt, 5 + M)


@pytest.mark.parametrize("mode", FINE)
@pytest.mark.parametrize("bits", [2, 3, 4])
@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
@pytest.mark.parametrize("gs", [32, -1])
def test_fine_gemm_parity(orc, wq, mode, bits, dt, gs):
    K, N = 512, 224
    for M in (1, 70, 130):
        print(f"[fine gemm] mode={mode} bits={bits} dt={dt} gs={gs} M={M}", flush=True)
        L = wl.make_layer(K, N, bits, gs, mode, 400 + 7 * mode + bits + dt + M)
        check(orc, wq, "wq_gemm", L, M, dt, 9 + M)


@pytest.mark.parametrize("M", [1, 16, 130])
def test_fine_gate_up(orc, wq, M):
    from test_gpu_gate_up import gate_up_bound, repack_gate_up
    K, N = 1024, 192
    L = wl.make_layer(K, N, 2, -1, wl.ZERO_F16_G8, 70 + M)
    x_bits = wl.make_x(M, K, wl.F16, 3 + M)
    x = bits_to_tensor(x_bits, torch.float16, "cuda")
    fn = wq.wq_gemv_gate_up if M <= 16 else wq.wq_gemm_gate_up
    h = tensor_f64(fn(x, repack_gate_up(wq, L)))
    torch.cuda.synchronize()
    h_ref = orc.linear_gate_up(x_bits, wl.F16, L.qweight, L.scales, L.zeros, L.mode, None, None, M, N, K, 2, -1)
    y_gu = oracle_y(orc, x_bits, wl.F16, L)
    assert np.all(np.abs(h - h_ref) <= gate_up_bound(y_gu, h_ref, wl.F16))


def test_fine_rejects_act_order(wq):
    L = wl.make_layer(512, 64, 4, 128, wl.ZERO_F16_G8, 1, act_order=True)
    with pytest.raises(wq.WQError):
        repack_layer(wq, L)


@pytest.mark.parametrize("M", [1, 16, 2048])
def test_fine_full_size_2bit_column_scales(orc, wq, M):
    """The zero-point experiment's shape: 2-bit codes, one scale per column, a
    zero-point every 8 rows, on the LLaMA-7B fused QKV layer (4096 x 12288),
    sampled output columns."""
    K, N = 4096, 12288
    L = wl.make_layer(K, N, 2, -1, wl.ZERO_F16_G8, 12, scale_range=(0.002, 0.01))
    x_bits = wl.make_x(M, K, wl.F16, 77 + M)
    x = bits_to_tensor(x_bits, torch.float16, "cuda")
    y = (wq.wq_gemv if M <= 16 else wq.wq_gemm)(x, repack_layer(wq, L))
    torch.cuda.synchronize()
    cols = wl.sample_cols(N, 256 if M <= 16 else 48, seed=M)
    got = tensor_f64(y[:, torch.from_numpy(cols).long().cuda()])
    ok, err, bound = within_tolerance(got, oracle_y(orc, x_bits, wl.F16, L, cols))
    assert ok, f"max error {err:.3e} > bound {bound:.3e}"
