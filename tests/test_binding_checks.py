"""The Python binding checks every buffer before the library sees a pointer.

The product kernels read and write through raw pointers, so a short `out`, a
workspace on another device or a mis-shaped scale tensor would be an access
out of bounds on the GPU.  These CPU tests show that each such argument raises
ValueError before anything is launched (all tensors here live on the CPU, so a
launch could not even start; the checks on shapes, dtypes and layout come
before the device check)."""
import pytest
import torch

import weight_only_quantized_w4a16_amd as wq


@pytest.fixture(scope="module")
def layer():
    if not __import__("os").path.exists(wq.LIB_PATH):
        from weight_only_quantized_w4a16_amd import build
        build.build()
    wq.lib()
    K, N = 256, 64
    nbytes = wq.wq_packed_bytes(K, N, 4, 128, wq.SYM)
    return wq.PackedLayer(torch.zeros(nbytes, dtype=torch.uint8), K, N, 4, 128, wq.SYM)


def x_of(M, layer, dtype=torch.float16):
    return torch.zeros((M, layer.K), dtype=dtype)


def test_out_shape(layer):
    with pytest.raises(ValueError, match="out must have shape"):
        wq.wq_gemv(x_of(2, layer), layer, out=torch.empty((2, layer.N - 16), dtype=torch.float16))
    with pytest.raises(ValueError, match="out must have shape"):
        wq.wq_gemm(x_of(2, layer), layer, out=torch.empty((1, layer.N), dtype=torch.float16))


def test_out_dtype_and_layout(layer):
    with pytest.raises(ValueError, match="out must have dtype"):
        wq.wq_gemv(x_of(1, layer), layer, out=torch.empty((1, layer.N), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="out must be contiguous"):
        wq.wq_gemv(x_of(2, layer), layer, out=torch.empty((layer.N, 2), dtype=torch.float16).t())


def test_fused_out_is_half_width(layer):
    fused = wq.PackedLayer(layer.packed, layer.K, layer.N, 4, 128, wq.SYM, gate_up=True)
    with pytest.raises(ValueError, match="out must have shape"):
        wq.wq_gemv_gate_up(x_of(1, fused), fused, out=torch.empty((1, layer.N), dtype=torch.float16))
    with pytest.raises(ValueError, match="repacked by"):
        wq.wq_gemv_gate_up(x_of(1, layer), layer)


def test_workspace_too_small(layer):
    # act-order needs M*K*2 bytes of workspace for the permuted activations
    perm_layer = wq.PackedLayer(layer.packed, layer.K, layer.N, 4, 128, wq.SYM,
                                perm=torch.arange(layer.K, dtype=torch.int32))
    need = wq.wq_workspace_bytes(3, layer.N, layer.K, 4, True)
    assert need > 0
    with pytest.raises(ValueError, match="ws holds fewer"):
        wq.wq_gemv(x_of(3, perm_layer), perm_layer, ws=torch.empty(need - 1, dtype=torch.uint8))


def test_x_checks(layer):
    with pytest.raises(ValueError, match="x must be"):
        wq.wq_gemv(torch.zeros((1, layer.K + 128), dtype=torch.float16), layer)
    with pytest.raises(ValueError, match="activation dtype"):
        wq.wq_gemv(torch.zeros((1, layer.K), dtype=torch.float32), layer)
    # well-formed but on the CPU: refused before the library is called
    with pytest.raises(ValueError, match="GPU tensor"):
        wq.wq_gemv(x_of(1, layer), layer)


def canonical(K=256, N=64, bits=4, G=2):
    return (torch.zeros((K * bits // 32, N), dtype=torch.int32), torch.ones((G, N), dtype=torch.float16))


def test_repack_checks():
    q, s = canonical()
    with pytest.raises(ValueError, match="qweight must have shape"):
        wq.wq_repack(q[:-1], s, None, wq.SYM, None, 256, 64, 4, 128)
    with pytest.raises(ValueError, match="scales must have shape"):
        wq.wq_repack(q, s[:1], None, wq.SYM, None, 256, 64, 4, 128)
    with pytest.raises(ValueError, match="scales must have dtype"):
        wq.wq_repack(q, s.float(), None, wq.SYM, None, 256, 64, 4, 128)
    with pytest.raises(ValueError, match="zeros must have dtype"):
        wq.wq_repack(q, s, torch.zeros((2, 64), dtype=torch.int32), wq.ZERO_F16, None, 256, 64, 4, 128)
    with pytest.raises(ValueError, match="zeros must have shape"):
        wq.wq_repack(q, s, torch.zeros((2, 7), dtype=torch.int32), wq.ZERO_PACKED, None, 256, 64, 4, 128)
    with pytest.raises(ValueError, match="zeros must be None"):
        wq.wq_repack(q, s, torch.zeros((2, 64), dtype=torch.float16), wq.SYM, None, 256, 64, 4, 128)
    with pytest.raises(ValueError, match="lut must have shape"):
        wq.wq_repack(q, s, None, wq.LUT, None, 256, 64, 4, 128, lut=torch.zeros(8, dtype=torch.float16))
    with pytest.raises(ValueError, match="lut is only used"):
        wq.wq_repack(q, s, None, wq.SYM, None, 256, 64, 4, 128, lut=torch.zeros(16, dtype=torch.float16))
    with pytest.raises(ValueError, match="zeros must have shape"):
        wq.wq_repack(q, s, torch.zeros((256 // 16, 64), dtype=torch.float16), wq.ZERO_F16_G8, None,
                     256, 64, 4, 128)
    with pytest.raises(ValueError, match="g_idx must have"):
        wq.wq_repack(q, s, None, wq.SYM, [0] * 255, 256, 64, 4, 128)
    with pytest.raises(ValueError, match="must be contiguous"):
        wq.wq_repack(torch.zeros((64, 32), dtype=torch.int32).t(), s, None, wq.SYM, None, 256, 64, 4, 128)
    # well-formed but on the CPU
    with pytest.raises(ValueError, match="GPU tensor"):
        wq.wq_repack(q, s, None, wq.SYM, None, 256, 64, 4, 128)


def test_hadamard_checks():
    x = torch.zeros((2, 256), dtype=torch.float16)
    with pytest.raises(ValueError, match="out must be"):
        wq.wq_hadamard(x, 128, out=torch.zeros((2, 256), dtype=torch.bfloat16))
    with pytest.raises(ValueError, match="GPU tensor"):
        wq.wq_hadamard(x, 128)


def test_layer_checks(layer):
    x = x_of(1, layer)
    short = wq.PackedLayer(layer.packed[:-256], layer.K, layer.N, 4, 128, wq.SYM)
    with pytest.raises(ValueError, match="shorter than the packed size"):
        wq.wq_gemv(x, short)
    with pytest.raises(ValueError, match="shorter than the packed size"):
        wq.wq_dequant_debug(short, torch.float16)
    wide = wq.PackedLayer(layer.packed, layer.K, layer.N + 16, 4, 128, wq.SYM)
    with pytest.raises(ValueError, match="shorter than the packed size"):
        wq.wq_gemm(x_of(1, wide), wide)
    bad_perm = wq.PackedLayer(layer.packed, layer.K, layer.N, 4, 128, wq.SYM,
                              perm=torch.arange(layer.K, dtype=torch.int64))
    with pytest.raises(ValueError, match="layer.perm must have dtype"):
        wq.wq_gemv(x, bad_perm)
    short_perm = wq.PackedLayer(layer.packed, layer.K, layer.N, 4, 128, wq.SYM,
                                perm=torch.arange(layer.K - 1, dtype=torch.int32))
    with pytest.raises(ValueError, match="layer.perm must have shape"):
        wq.wq_gemm(x, short_perm)
    no_lut = wq.PackedLayer(torch.zeros(wq.wq_packed_bytes(layer.K, layer.N, 4, 128, wq.LUT), dtype=torch.uint8),
                            layer.K, layer.N, 4, 128, wq.LUT)
    with pytest.raises(ValueError, match="table is needed"):
        wq.wq_gemv(x, no_lut)
    with pytest.raises(ValueError, match="layer.packed must be"):
        wq.wq_gemv(x, wq.PackedLayer(layer.packed.view(torch.int8), layer.K, layer.N, 4, 128, wq.SYM))
    out = torch.empty((1, layer.N), dtype=torch.float16)
    with pytest.raises(ValueError, match="shorter than the packed size"):
        wq.wq_gemm_noalloc(x, short, out)


def test_linear_dispatch():
    """linear() sends decode-sized M to the GEMV, except where the large-M
    product was measured faster: table codes above 16 rows at 2 bits, and at
    4 bits on layers wider than 16384 columns."""
    def lay(bits, N, mode=wq.LUT):
        return wq.PackedLayer(None, 8192, N, bits, 64, mode)
    assert wq.use_gemv(1, lay(4, 28672)) and wq.use_gemv(16, lay(4, 28672))
    assert not wq.use_gemv(17, lay(4, 28672)) and not wq.use_gemv(32, lay(4, 28672))
    assert wq.use_gemv(32, lay(4, 8192)) and wq.use_gemv(32, lay(3, 28672))
    assert wq.use_gemv(16, lay(2, 8192)) and not wq.use_gemv(17, lay(2, 8192))
    assert wq.use_gemv(32, lay(4, 53248, wq.ZERO_PACKED)) and not wq.use_gemv(33, lay(4, 4096, wq.SYM))
