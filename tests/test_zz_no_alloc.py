"""wq_gemm_noalloc (the entry point for callers that cannot allocate) against
wq_gemm: same kernels and launch shapes, so the outputs must be bit-identical.

Two calls in a row through the C ABI, the second with a smaller problem, so
the second runs on scratch that still holds the first call's partial products
and permuted activations; then a call too large for the scratch array, which
must be refused before anything is launched."""
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


def run_pair(wq, L, M, dt, seed):
    layer = repack_layer(wq, L)
    x_bits = wl.make_x(M, L.K, dt, seed)
    x = bits_to_tensor(x_bits, act_dtype(dt), "cuda")
    ws_need = wq.wq_workspace_bytes(M, L.N, L.K, L.bits, layer.perm is not None)
    assert 0 < ws_need <= wq.NOALLOC_SCRATCH_BYTES
    y_ref = wq.wq_gemm(x, layer)
    y = torch.full((M, L.N), float("nan"), dtype=act_dtype(dt), device="cuda")
    wq.wq_gemm_noalloc(x, layer, y)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(y), tensor_bits(y_ref))
    return x_bits, y


def test_noalloc_matches_gemm_twice(orc, wq):
    # 1) act-order, packed zero-points, bf16, K split: permuted x + 32 MiB of partials
    L1 = wl.make_layer(14336, 4096, 4, 32, wl.ZERO_PACKED, seed=71, act_order=True)
    print("[noalloc] call 1: K=14336 N=4096 M=128 act-order packed zeros bf16", flush=True)
    x1, y1 = run_pair(wq, L1, 128, wl.BF16, 72)
    cols = wl.sample_cols(L1.N, 64, seed=73)
    ok, err, bound = within_tolerance(tensor_f64(y1)[:, cols], oracle_y(orc, x1, wl.BF16, L1, cols))
    assert ok, f"{err} > {bound}"
    # 2) smaller: symmetric fp16 4096 x 4096, M = 64 (K split over less scratch)
    L2 = wl.make_layer(4096, 4096, 4, 128, wl.SYM, seed=74)
    print("[noalloc] call 2: K=4096 N=4096 M=64 symmetric fp16", flush=True)
    x2, y2 = run_pair(wq, L2, 64, wl.F16, 75)
    cols = wl.sample_cols(L2.N, 64, seed=76)
    ok, err, bound = within_tolerance(tensor_f64(y2)[:, cols], oracle_y(orc, x2, wl.F16, L2, cols))
    assert ok, f"{err} > {bound}"


def test_noalloc_refuses_oversized_scratch(wq):
    # act-order with M * K * 2 bytes beyond the array: refused on the host
    L = wl.make_layer(16384, 256, 4, 32, wl.SYM, seed=77, act_order=True)
    layer = repack_layer(wq, L)
    M = 2048
    assert wq.wq_workspace_bytes(M, L.N, L.K, 4, True) > wq.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((M, L.K), dtype=torch.float16, device="cuda")
    y = torch.zeros((M, L.N), dtype=torch.float16, device="cuda")
    with pytest.raises(wq.WQError) as e:
        wq.wq_gemm_noalloc(x, layer, y)
    assert e.value.status == 4  # WQ_ENOSPACE
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0  # nothing was written
