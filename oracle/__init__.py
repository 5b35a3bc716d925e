"""CPU oracle for y = x . dequant(W) -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  The product path (the HIP library and its binding) never does.

Thin numpy wrappers over liboracle.so (plain C, fp64, naive loops), built from
wq_oracle.c by oracle/build.py.  Every function mirrors a C entry point:

  unpack_codes / pack_codes   canonical packing (per column, a little-endian bit
                              stream along K; GPTQ's 8 int4 codes per uint32 for
                              4 bits)
  unpack_zeros / pack_zeros   packed zero-points (per group row, a bit stream along N)
  dequant                     w = RN_dtype(s*(q-z)) or RN_dtype(s*T[q]), one rounding
  linear                      y = x . w in fp64, k ascending, optional column subset
  swiglu / linear_gate_up     h = SiLU(x . W_gate) * (x . W_up) for fused gate+up weights
  decode / encode             exact fp16/bf16 -> fp64 and RNE fp64 -> fp16/bf16
"""
import ctypes
import os

import numpy as np

from . import build as _build

SYM, ZERO_F16, ZERO_PACKED, LUT = 0, 1, 2, 3
ZERO_F16_G8, ZERO_F16_G16, ZERO_F16_G32 = 4, 5, 6  # fp16 zero-points per 8 / 16 / 32 rows
F16, BF16 = 0, 1

_lib = None


def lib():
    """The oracle library.  WQ_ORACLE_LIB may name another build of the same
    source (the mutation tests load deliberately broken copies this way)."""
    global _lib
    if _lib is None:
        path = os.environ.get("WQ_ORACLE_LIB", _build.LIB)
        if path == _build.LIB and not os.path.exists(path):
            _build.build()
        L = ctypes.CDLL(path)
        P = ctypes.c_void_p
        i = ctypes.c_int
        L.wqo_unpack_codes.argtypes = [P, i, i, i, P]
        L.wqo_pack_codes.argtypes = [P, i, i, i, P]
        L.wqo_unpack_zeros.argtypes = [P, i, i, i, P]
        L.wqo_pack_zeros.argtypes = [P, i, i, i, P]
        L.wqo_dequant.argtypes = [P, P, P, i, P, P, i, i, i, i, i, P]
        L.wqo_linear.argtypes = [P, i, P, P, P, i, P, P, i, i, i, i, i, P, i, P]
        L.wqo_decode_array.argtypes = [P, ctypes.c_size_t, i, P]
        L.wqo_decode_array.restype = None
        L.wqo_encode_array.argtypes = [P, ctypes.c_size_t, i, P]
        L.wqo_encode_array.restype = None
        L.wqo_f64_to_f16.argtypes = [ctypes.c_double]
        L.wqo_f64_to_f16.restype = ctypes.c_uint16
        L.wqo_f64_to_bf16.argtypes = [ctypes.c_double]
        L.wqo_f64_to_bf16.restype = ctypes.c_uint16
        L.wqo_num_threads.argtypes = []
        L.wqo_silu.argtypes = [ctypes.c_double]
        L.wqo_silu.restype = ctypes.c_double
        L.wqo_swiglu.argtypes = [P, P, ctypes.c_size_t, P]
        L.wqo_swiglu.restype = None
        L.wqo_hadamard.argtypes = [P, i, i, i, P]
        _lib = L
    return _lib


class OracleError(RuntimeError):
    pass


def _p(a):
    return None if a is None else ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    return None if a is None else np.ascontiguousarray(a, dtype=dtype)


def _check(rc):
    if rc != 0:
        raise OracleError(f"oracle rejected the arguments (status {rc})")


def num_threads() -> int:
    return int(lib().wqo_num_threads())


def decode(bits, dtype):
    bits = _c(bits, np.uint16)
    out = np.empty(bits.shape, np.float64)
    lib().wqo_decode_array(_p(bits), bits.size, dtype, _p(out))
    return out


def encode(values, dtype):
    values = _c(values, np.float64)
    out = np.empty(values.shape, np.uint16)
    lib().wqo_encode_array(_p(values), values.size, dtype, _p(out))
    return out


def unpack_codes(qweight, K, N, bits):
    qweight = _c(qweight, np.uint32)
    assert qweight.size == K * bits // 32 * N
    out = np.empty((K, N), np.uint8)
    _check(lib().wqo_unpack_codes(_p(qweight), K, N, bits, _p(out)))
    return out


def pack_codes(codes, bits):
    codes = _c(codes, np.uint8)
    K, N = codes.shape
    out = np.empty((K * bits // 32, N), np.uint32)
    _check(lib().wqo_pack_codes(_p(codes), K, N, bits, _p(out)))
    return out


def unpack_zeros(zp, G, N, bits):
    zp = _c(zp, np.uint32)
    assert zp.size == G * (N * bits // 32)
    out = np.empty((G, N), np.uint8)
    _check(lib().wqo_unpack_zeros(_p(zp), G, N, bits, _p(out)))
    return out


def pack_zeros(z, bits):
    z = _c(z, np.uint8)
    G, N = z.shape
    out = np.empty((G, N * bits // 32), np.uint32)
    _check(lib().wqo_pack_zeros(_p(z), G, N, bits, _p(out)))
    return out


def _zeros_arr(mode, zeros):
    if mode in (ZERO_F16, ZERO_F16_G8, ZERO_F16_G16, ZERO_F16_G32):
        return _c(zeros, np.uint16)
    if mode == ZERO_PACKED:
        return _c(zeros, np.uint32)
    return None


def dequant(qweight, scales, zeros, mode, lut, g_idx, K, N, bits, group_size, dtype):
    """Dequantised weight bits [K][N] (fp16 or bf16 bit patterns), original row order."""
    qweight = _c(qweight, np.uint32)
    scales = _c(scales, np.uint16)
    z = _zeros_arr(mode, zeros)
    lut = _c(lut, np.uint16)
    g_idx = _c(g_idx, np.int32)
    out = np.empty((K, N), np.uint16)
    _check(lib().wqo_dequant(_p(qweight), _p(scales), _p(z), mode, _p(lut), _p(g_idx),
                             K, N, bits, group_size, dtype, _p(out)))
    return out


def swiglu(g, u):
    """h = SiLU(g) * u elementwise (fp64)."""
    g = _c(g, np.float64)
    u = _c(u, np.float64)
    assert g.shape == u.shape
    h = np.empty(g.shape, np.float64)
    lib().wqo_swiglu(_p(g), _p(u), g.size, _p(h))
    return h


def hadamard(x, block):
    """Rows of x (fp64 [M][K]) rotated by the orthonormal block-diagonal
    Walsh-Hadamard matrix of block size `block` (fp64)."""
    x = _c(x, np.float64)
    M, K = x.shape
    y = np.empty((M, K), np.float64)
    _check(lib().wqo_hadamard(_p(x), M, K, block, _p(y)))
    return y


def rotate_x(x_bits, dtype, block):
    """Activation bit patterns -> rotated activations rounded once (RNE) to the
    activation dtype, as bit patterns."""
    return encode(hadamard(decode(x_bits, dtype), block), dtype)


def linear_gate_up(x, dtype, qweight, scales, zeros, mode, lut, g_idx, M, N, K, bits, group_size, cols=None):
    """Fused gate+up: W holds [gate | up] along N (N = 2I); returns h [M][len(cols) or I]
    with h[:, j] = SiLU(x.W[:, j]) * (x.W[:, I + j])."""
    I = N // 2
    cols = np.arange(I, dtype=np.int32) if cols is None else np.asarray(cols, np.int32)
    both = np.concatenate([cols, cols + I]).astype(np.int32)
    y = linear(x, dtype, qweight, scales, zeros, mode, lut, g_idx, M, N, K, bits, group_size, both)
    return swiglu(y[:, :cols.size], y[:, cols.size:])


def linear(x, dtype, qweight, scales, zeros, mode, lut, g_idx, M, N, K, bits, group_size, cols=None):
    """y[M][len(cols)] in fp64 (all N columns when cols is None)."""
    x = _c(x, np.uint16)
    qweight = _c(qweight, np.uint32)
    scales = _c(scales, np.uint16)
    z = _zeros_arr(mode, zeros)
    lut = _c(lut, np.uint16)
    g_idx = _c(g_idx, np.int32)
    cols = _c(cols, np.int32)
    ncols = N if cols is None else cols.size
    y = np.empty((M, ncols), np.float64)
    _check(lib().wqo_linear(_p(x), dtype, _p(qweight), _p(scales), _p(z), mode, _p(lut), _p(g_idx),
                            M, N, K, bits, group_size, _p(cols), ncols, _p(y)))
    return y
