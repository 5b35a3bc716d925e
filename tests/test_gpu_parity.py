"""GPU parity: the HIP path through the C ABI against the oracle.

  * wq_dequant_debug is bit-exact with the oracle's dequantised weights;
  * wq_gemv / wq_gemm meet max|y - y_ref| <= 5e-3 * max|y_ref| + 1e-3 (fp32
    accumulation, one rounding of the output);
on seeded inputs at sizes the oracle finishes quickly that still span several
tiles, for every mode, code width, activation dtype and group size, with and
without act-order, plus ragged M and column counts.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from _util import act_dtype, bits_to_tensor, oracle_y, repack_layer, tensor_bits, tensor_f64, within_tolerance

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


def groups_for(bits):
    kt = 256 if bits == 2 else 128
    return [g for g in (32, 64, 128, 256, -1) if g == -1 or g % kt == 0 or kt % g == 0]


DEQ_CASES = [(mode, bits, dt, gs, ao) for mode in MODES for bits in (2, 3, 4) for dt in (wl.F16, wl.BF16)
             for gs in groups_for(bits) for ao in ((False, True) if gs in (32, 128) else (False,))]


@pytest.mark.parametrize("mode,bits,dt,gs,ao", DEQ_CASES)
def test_dequant_debug_bit_exact(orc, wq, mode, bits, dt, gs, ao):
    K, N = 512, 64
    print(f"[dequant] mode={mode} bits={bits} dt={dt} gs={gs} act_order={ao}", flush=True)
    L = make(mode, bits, gs, K, N, 1000 + 97 * mode + 13 * bits + 5 * dt + (gs if gs > 0 else 1) + ao)
    layer = repack_layer(wq, L)
    w = wq.wq_dequant_debug(layer, act_dtype(dt))
    torch.cuda.synchronize()
    ref = orc.dequant(L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, K, N, bits, gs, dt)
    got = tensor_bits(w)
    assert np.array_equal(got, ref), f"{np.count_nonzero(got != ref)} mismatching weights"


def check_product(orc, wq, fn, L, M, dt, seed):
    x_bits = wl.make_x(M, L.K, dt, seed)
    layer = repack_layer(wq, L)
    x = bits_to_tensor(x_bits, act_dtype(dt), "cuda")
    y = getattr(wq, fn)(x, layer)
    torch.cuda.synchronize()
    ref = oracle_y(orc, x_bits, dt, L)
    ok, err, bound = within_tolerance(tensor_f64(y), ref)
    assert ok, f"{fn}: max error {err:.3e} > bound {bound:.3e}"
    return y


GEMV_CASES = [(mode, bits, dt, gs, M, ao)
              for mode in MODES for bits in (2, 3, 4) for dt in (wl.F16, wl.BF16)
              for gs in (32, 128, -1) for M in ((1, 3, 5, 8, 16, 17, 32) if gs == 128 else (1, 3, 5, 8, 16, 32))
              for ao in ((False, True) if (gs == 32 and M in (1, 5, 32)) else (False,))]


@pytest.mark.parametrize("mode,bits,dt,gs,M,ao", GEMV_CASES)
def test_gemv_parity(orc, wq, mode, bits, dt, gs, M, ao):
    K, N = 1024, 96  # 4-8 k-tiles, 6 column tiles; M > 16 takes two blocks of 16 rows
    print(f"[gemv] mode={mode} bits={bits} dt={dt} gs={gs} M={M} act_order={ao}", flush=True)
    L = make(mode, bits, gs, K, N, 2000 + 97 * mode + 13 * bits + 5 * dt + M + ao, act_order=ao)
    check_product(orc, wq, "wq_gemv", L, M, dt, 77 + M)


GEMM_CASES = [(mode, bits, dt, gs, M, ao)
              for mode in MODES for bits in (2, 3, 4) for dt in (wl.F16, wl.BF16)
              for gs in (32, 128, -1) for M in (1, 70, 130)
              for ao in ((False, True) if (gs == 32 and M == 70) else (False,))]


@pytest.mark.parametrize("mode,bits,dt,gs,M,ao", GEMM_CASES)
def test_gemm_parity(orc, wq, mode, bits, dt, gs, M, ao):
    K, N = 512, 224  # 2-4 k-tiles, two column blocks, the second one ragged (96 of 128 columns)
    print(f"[gemm] mode={mode} bits={bits} dt={dt} gs={gs} M={M} act_order={ao}", flush=True)
    L = make(mode, bits, gs, K, N, 3000 + 97 * mode + 13 * bits + 5 * dt + M + ao, act_order=ao)
    check_product(orc, wq, "wq_gemm", L, M, dt, 99 + M)


@pytest.mark.parametrize("mode", MODES + [wl.ZERO_F16_G16])
@pytest.mark.parametrize("bits", [2, 3, 4])
def test_gemv_wide_two_row_blocks(orc, wq, mode, bits):
    """A layer wide enough (>= 512 column tiles) for waves that own two column
    tiles, at M = 32 (two blocks of 16 activation rows; 2-bit codes take a
    second launch for rows 16..31) and M = 20 (a ragged second block); the
    oracle computes a seeded sample of columns."""
    K, N = 512, 8192 + 32
    L = make(mode, bits, 128 if mode in wl.FINE_ZERO_GROUP else 64, K, N, 4100 + 7 * mode + bits)
    layer = repack_layer(wq, L)
    cols = wl.sample_cols(N, 192, seed=bits + mode)
    cols = np.unique(np.concatenate([cols, np.arange(N - 32, N)])).astype(np.int32)  # the last tiles
    for M in (32, 20):
        dt = wl.BF16 if M == 20 else wl.F16
        print(f"[gemv wide] mode={mode} bits={bits} M={M}", flush=True)
        x_bits = wl.make_x(M, K, dt, 50 + M)
        y = wq.wq_gemv(bits_to_tensor(x_bits, act_dtype(dt), "cuda"), layer)
        torch.cuda.synchronize()
        got = tensor_f64(y)[:, cols]
        ok, err, bound = within_tolerance(got, oracle_y(orc, x_bits, dt, L, cols))
        assert ok, f"max error {err:.3e} > bound {bound:.3e}"


TILE128_CASES = [(wl.SYM, 4, 128), (wl.SYM, 4, 64), (wl.SYM, 3, -1), (wl.ZERO_F16, 4, 128), (wl.ZERO_F16, 3, 256),
                 (wl.ZERO_PACKED, 3, 128), (wl.LUT, 3, 64)]


@pytest.mark.parametrize("mode,bits,gs", TILE128_CASES)
@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_gemm_128_row_tiles(orc, wq, mode, bits, gs, dt):
    """Enough row and column blocks (9 x 61 >= 480) for the 128-row tiles of
    the decodes that have them; the last row tile and the last column block
    are ragged.  The oracle computes a seeded sample of columns."""
    K, N, M = 512, 15520, 1088
    L = make(mode, bits, gs, K, N, 9100 + 7 * mode + bits + dt)
    layer = repack_layer(wq, L)
    x_bits = wl.make_x(M, K, dt, 17 + mode + bits)
    print(f"[gemm 128-row] mode={mode} bits={bits} gs={gs} dt={dt}", flush=True)
    y = wq.wq_gemm(bits_to_tensor(x_bits, act_dtype(dt), "cuda"), layer)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([wl.sample_cols(N, 96, seed=mode + bits), np.arange(N - 16, N)])).astype(np.int32)
    ok, err, bound = within_tolerance(tensor_f64(y)[:, cols], oracle_y(orc, x_bits, dt, L, cols))
    assert ok, f"max error {err:.3e} > bound {bound:.3e}"


NARROW_TILE_CASES = [(wl.SYM, 4, 32), (wl.SYM, 2, 128), (wl.ZERO_F16, 4, 64), (wl.ZERO_F16, 2, 256),
                     (wl.ZERO_PACKED, 4, 128), (wl.ZERO_PACKED, 4, 32), (wl.ZERO_PACKED, 3, 64),
                     (wl.ZERO_PACKED, 2, 256), (wl.ZERO_PACKED, 2, 32), (wl.LUT, 2, 64), (wl.LUT, 4, 64), (wl.LUT, 4, -1),
                     (wl.ZERO_F16_G8, 4, -1), (wl.ZERO_F16_G32, 3, 128)]


@pytest.mark.parametrize("mode,bits,gs,shapes", [c + (((512, 15520, 1088), (4096, 1024, 250)),) for c in NARROW_TILE_CASES]
                         + [c + (((512, 2080, 1088), (4096, 1024, 250)),) for c in TILE128_CASES])
@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_gemm_128x128_tiles(orc, wq, mode, bits, gs, shapes, dt):
    """128 x 128 workgroup tiles above 64 rows: 17 row blocks of 64 (ragged
    last 128-row tile) over a ragged last column block, and 4 row blocks with
    K split (K = 4096, N = 1024: 16 workgroups of 64 x 256).  Decodes that
    fit 128 x 256 tiles take 128 x 128 where 128 x 256 would leave too few
    workgroups (N = 2080) or K is split.  The oracle computes a seeded
    sample of columns / all columns."""
    for K, N, M in shapes:
        L = make(mode, bits, gs, K, N, 9300 + 7 * mode + bits + dt + M)
        layer = repack_layer(wq, L)
        x_bits = wl.make_x(M, K, dt, 23 + mode + bits)
        print(f"[gemm 128x128] mode={mode} bits={bits} gs={gs} dt={dt} K={K} N={N} M={M}", flush=True)
        y = wq.wq_gemm(bits_to_tensor(x_bits, act_dtype(dt), "cuda"), layer)
        torch.cuda.synchronize()
        cols = np.unique(np.concatenate([wl.sample_cols(N, 96, seed=mode + bits), np.arange(N - 16, N)])).astype(np.int32)
        if N <= 1024:
            cols = np.arange(N, dtype=np.int32)
        ok, err, bound = within_tolerance(tensor_f64(y)[:, cols], oracle_y(orc, x_bits, dt, L, cols))
        assert ok, f"K={K} N={N} M={M}: max error {err:.3e} > bound {bound:.3e}"


@pytest.mark.parametrize("M", [1, 17, 40, 64])
@pytest.mark.parametrize("dt", [wl.F16, wl.BF16])
def test_gemm_2bit_packed_group32_small_m(orc, wq, M, dt):
    """2-bit codes with packed zero-points in groups of 32 rows take 128 x 128
    tiles at every M (their 64 x 256 variant would spill): one padded row tile,
    K split, ragged last column block (N = 528)."""
    K, N = 1024, 528
    L = make(wl.ZERO_PACKED, 2, 32, K, N, 9500 + M + dt)
    layer = repack_layer(wq, L)
    x_bits = wl.make_x(M, K, dt, 31 + M)
    print(f"[gemm 2-bit packed g32] M={M} dt={dt}", flush=True)
    y = wq.wq_gemm(bits_to_tensor(x_bits, act_dtype(dt), "cuda"), layer)
    torch.cuda.synchronize()
    ok, err, bound = within_tolerance(tensor_f64(y), oracle_y(orc, x_bits, dt, L))
    assert ok, f"max error {err:.3e} > bound {bound:.3e}"


def test_m_zero_is_a_noop(wq):
    L = make(wl.SYM, 4, 128, 512, 64, 5)
    layer = repack_layer(wq, L)
    x = torch.empty((0, 512), dtype=torch.float16, device="cuda")
    for fn in (wq.wq_gemv, wq.wq_gemm):
        y = fn(x, layer)
        assert y.shape == (0, 64)


@pytest.mark.parametrize("fn", ["wq_gemv", "wq_gemm"])
def test_deterministic(wq, fn):
    L = make(wl.ZERO_F16, 4, 128, 2048, 256, 6)
    layer = repack_layer(wq, L)
    x = bits_to_tensor(wl.make_x(4, 2048, wl.F16, 1), torch.float16, "cuda")
    y1 = getattr(wq, fn)(x, layer).clone()
    y2 = getattr(wq, fn)(x, layer)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)


@pytest.mark.parametrize("mode,dt", [(wl.SYM, wl.F16), (wl.ZERO_PACKED, wl.BF16), (wl.LUT, wl.BF16)])
def test_rows_independent_and_paths_agree(orc, wq, mode, dt):
    """One M=16 call, sixteen M=1 calls and the large-M path all meet the
    tolerance against the oracle, so they agree with each other within twice
    the bound (each output is rounded to the activation dtype separately, so
    two of them can differ by one unit in the last place)."""
    K, N = 1024, 128
    L = make(mode, 4, 64, K, N, 8)
    layer = repack_layer(wq, L)
    x_bits = wl.make_x(16, K, dt, 3)
    x = bits_to_tensor(x_bits, act_dtype(dt), "cuda")
    ref = oracle_y(orc, x_bits, dt, L)
    y16 = tensor_f64(wq.wq_gemv(x, layer))
    rows = np.concatenate([tensor_f64(wq.wq_gemv(x[i:i + 1].contiguous(), layer)) for i in range(16)])
    yg = tensor_f64(wq.wq_gemm(x, layer))
    for y in (y16, rows, yg):
        assert within_tolerance(y, ref)[0]
    _, _, bound = within_tolerance(y16, ref)
    assert np.max(np.abs(rows - y16)) <= 2 * bound and np.max(np.abs(yg - y16)) <= 2 * bound


def test_fused_qkv_equals_separate(orc, wq):
    """Fused QKV: one call on weights concatenated along N gives the column
    ranges of the separate calls."""
    K = 1024
    parts = [make(wl.ZERO_F16, 4, 128, K, n, 40 + i) for i, n in enumerate((128, 64, 64))]
    fused = wl.Layer(K, 256, 4, 128, wl.ZERO_F16, np.concatenate([p.qweight for p in parts], 1),
                     np.concatenate([p.scales for p in parts], 1), np.concatenate([p.zeros for p in parts], 1))
    x_bits = wl.make_x(4, K, wl.F16, 5)
    x = bits_to_tensor(x_bits, torch.float16, "cuda")
    for fn in ("wq_gemv", "wq_gemm"):
        yf = tensor_f64(getattr(wq, fn)(x, repack_layer(wq, fused)))
        off = 0
        for p in parts:
            ys = tensor_f64(getattr(wq, fn)(x, repack_layer(wq, p)))
            assert np.array_equal(yf[:, off:off + p.N], ys)
            off += p.N
        assert within_tolerance(yf, oracle_y(orc, x_bits, wl.F16, fused))[0]


def test_group256_bf16_regression(orc, wq):
    """4-bit, group 256, bf16 (flagged as unstable for another kernel on the
    FLUTE page, "Limitations & Caveats"), uniform with fp16 zeros and table."""
    for mode in (wl.ZERO_F16, wl.LUT):
        L = make(mode, 4, 256, 4096, 256, 9)
        for fn, M in (("wq_gemv", 1), ("wq_gemv", 16), ("wq_gemm", 256)):
            check_product(orc, wq, fn, L, M, wl.BF16, 11 + M)


KSPLIT_CASES = [(mode, bits, dt, gs) for mode in MODES for bits in (2, 4) for dt in (wl.F16, wl.BF16)
                for gs in (128, -1)]


@pytest.mark.parametrize("mode,bits,dt,gs", KSPLIT_CASES)
def test_gemm_k_split_parity(orc, wq, mode, bits, dt, gs):
    """Narrow products split K over several workgroups (fp32 partial sums in
    the workspace, summed by a second kernel): 224 columns and K = 2048 give 4
    slices, for M = 1, 17, 64, 130 and 300 (ragged row and column tiles)."""
    K, N = 2048, 224
    assert wq.wq_workspace_bytes(64, N, K, bits, False) > 0
    assert wq.wq_workspace_bytes(300, N, K, bits, False) > 0
    for M in (1, 17, 64, 130, 300):
        print(f"[gemm k-split] mode={mode} bits={bits} dt={dt} gs={gs} M={M}", flush=True)
        L = make(mode, bits, gs, K, N, 8000 + 97 * mode + 13 * bits + 5 * dt + M)
        check_product(orc, wq, "wq_gemm", L, M, dt, 123 + M)


@pytest.mark.parametrize("M", [40, 64, 200])
def test_gemm_k_split_reduction_rows(orc, wq, M):
    """A 4096-column layer split into 4 slices, at row counts where the
    reduction gives each group of 4 outputs 4 (M = 40, 64) or 2 (M = 200)
    threads; the oracle computes a seeded sample of columns."""
    K, N = 2048, 4096
    assert wq.wq_workspace_bytes(M, N, K, 4, False) == 4 * M * N * 4
    L = make(wl.ZERO_F16, 4, 128, K, N, 8800 + M)
    layer = repack_layer(wq, L)
    x_bits = wl.make_x(M, K, wl.F16, 5 + M)
    y = wq.wq_gemm(bits_to_tensor(x_bits, torch.float16, "cuda"), layer)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([wl.sample_cols(N, 160, seed=M), np.arange(N - 16, N)])).astype(np.int32)
    ok, err, bound = within_tolerance(tensor_f64(y)[:, cols], oracle_y(orc, x_bits, wl.F16, L, cols))
    assert ok, f"max error {err:.3e} > bound {bound:.3e}"


def test_gemm_k_split_uneven_and_act_order(orc, wq):
    """K = 1664 (13 k-tiles) splits into slices of 4, 4, 4 and 1 tiles; with
    act-order the workspace holds the permuted activations and the partial
    sums side by side."""
    L = make(wl.ZERO_PACKED, 4, 128, 1664, 96, 77, act_order=True)
    for M in (3, 40):
        check_product(orc, wq, "wq_gemm", L, M, wl.BF16, 9 + M)


@pytest.mark.parametrize("fn,M", [("wq_gemv", 1), ("wq_gemv", 16), ("wq_gemm", 1), ("wq_gemm", 17)])
def test_smallest_layer(orc, wq, fn, M):
    """One tile: K = 128 rows, N = 16 columns (one workgroup, one k-tile)."""
    for mode in MODES:
        L = make(mode, 4, 32, 128, 16, 60 + mode)
        check_product(orc, wq, fn, L, M, wl.F16, 7 + M)


@pytest.mark.parametrize("fn,M", [("wq_gemv", 3), ("wq_gemm", 40), ("wq_gemm", 300)])
def test_degenerate_values(orc, wq, fn, M):
    """Zero scales give zero output; zero activations give zero output; equal
    activation rows give equal output rows; group = K matches group -1 bit for bit."""
    K, N = 1024, 64
    L = make(wl.ZERO_F16, 4, 128, K, N, 3)
    L0 = wl.Layer(K, N, 4, 128, wl.ZERO_F16, L.qweight, np.zeros_like(L.scales), L.zeros)
    x_bits = wl.make_x(M, K, wl.F16, 4)
    x = bits_to_tensor(x_bits, torch.float16, "cuda")
    assert torch.count_nonzero(getattr(wq, fn)(x, repack_layer(wq, L0))) == 0
    assert torch.count_nonzero(getattr(wq, fn)(torch.zeros_like(x), repack_layer(wq, L))) == 0
    xr = x[:1].repeat(M, 1).contiguous()
    y = getattr(wq, fn)(xr, repack_layer(wq, L))
    assert torch.equal(y, y[:1].expand(M, N))
    Lg = wl.make_layer(K, N, 4, -1, wl.SYM, 8)
    LK = wl.Layer(K, N, 4, K, wl.SYM, Lg.qweight, Lg.scales)
    assert torch.equal(getattr(wq, fn)(x, repack_layer(wq, Lg)), getattr(wq, fn)(x, repack_layer(wq, LK)))
    torch.cuda.synchronize()


@pytest.mark.parametrize("fn,M", [("wq_gemv", 1), ("wq_gemv", 7), ("wq_gemm", 40)])
def test_act_order_gather_forms_agree(orc, wq, fn, M):
    """The act-order gather runs eight elements per thread when perm is
    16-byte aligned and one per thread otherwise; both give the same output
    bit for bit, and it meets the oracle."""
    import dataclasses
    L = make(wl.ZERO_PACKED, 4, 32, 1024, 96, 91, act_order=True)
    layer = repack_layer(wq, L)
    assert layer.perm.data_ptr() % 16 == 0
    buf = torch.empty(layer.K + 1, dtype=torch.int32, device=layer.perm.device)
    buf[1:] = layer.perm
    odd = dataclasses.replace(layer, perm=buf[1:])
    assert odd.perm.data_ptr() % 16 == 4
    x_bits = wl.make_x(M, L.K, wl.BF16, 31 + M)
    x = bits_to_tensor(x_bits, torch.bfloat16, "cuda")
    y8, y1 = getattr(wq, fn)(x, layer), getattr(wq, fn)(x, odd)
    torch.cuda.synchronize()
    assert torch.equal(y8.view(torch.int16), y1.view(torch.int16))
    cols = np.arange(L.N, dtype=np.int32)
    ok, err, bound = within_tolerance(tensor_f64(y8), oracle_y(orc, x_bits, wl.BF16, L, cols))
    assert ok, f"max error {err:.3e} > bound {bound:.3e}"
