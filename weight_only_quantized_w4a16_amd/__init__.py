"""Weight-only quantized mixed-input matmul y = x . dequant(W) on MI355X (gfx950).

Thin ctypes binding over libwq.so (the C ABI in include/wq.h).  Every function
here only marshals arguments -- torch tensors supply device memory and the
current HIP stream -- and calls the library; every step of the product runs in
the library's HIP kernels.  There is no CPU fallback: if libwq.so is missing or
cannot be loaded, every call raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

SYM, ZERO_F16, ZERO_PACKED, LUT = 0, 1, 2, 3
ZERO_F16_G8, ZERO_F16_G16, ZERO_F16_G32 = 4, 5, 6  # fp16 zero-points per 8 / 16 / 32 rows
F16, BF16 = 0, 1
LAYOUT_VERSION = 3

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libwq.so")

_STATUS = {0: "ok", 1: "invalid argument", 2: "unsupported", 3: "HIP error", 4: "workspace too small"}

_lib = None


class WQError(RuntimeError):
    def __init__(self, fn: str, status: int):
        super().__init__(f"{fn} failed: {_STATUS.get(status, status)} (status {status})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libwq.so (built by weight_only_quantized_w4a16_amd/build.py)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run weight_only_quantized_w4a16_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, I, Z = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
        L.wq_layout_version.restype = I
        L.wq_status_str.argtypes = [I]
        L.wq_status_str.restype = ctypes.c_char_p
        L.wq_packed_bytes.argtypes = [I, I, I, I, I]
        L.wq_packed_bytes.restype = Z
        L.wq_workspace_bytes.argtypes = [I, I, I, I, I]
        L.wq_workspace_bytes.restype = Z
        for name in ("wq_repack", "wq_repack_gate_up"):
            f = getattr(L, name)
            f.argtypes = [P, P, P, I, P, I, I, I, I, P, P, P]
            f.restype = I
        L.wq_dequant_debug.argtypes = [P, I, P, P, I, I, I, I, I, P, P]
        L.wq_dequant_debug.restype = I
        for name in ("wq_gemv", "wq_gemm", "wq_gemv_gate_up", "wq_gemm_gate_up"):
            f = getattr(L, name)
            f.argtypes = [P, I, P, I, P, P, P, I, I, I, I, I, P, Z, P]
            f.restype = I
        L.wq_gemm_noalloc.argtypes = [P, I, P, I, P, P, P, I, I, I, I, I, P]
        L.wq_gemm_noalloc.restype = I
        L.wq_hadamard.argtypes = [P, I, P, I, I, I, P]
        L.wq_hadamard.restype = I
        if L.wq_layout_version() != LAYOUT_VERSION:
            raise RuntimeError("libwq.so layout version does not match this binding")
        _lib = L
    return _lib


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream, dev: torch.device) -> ctypes.c_void_p:
    """The stream to launch on: `stream`, or the current stream of `dev`.  The
    library works on the current HIP device (its scratch array is per device),
    so that must be the device of the tensors."""
    cur = torch.cuda.current_device()
    if dev.index != cur:
        raise ValueError(f"the tensors are on {dev} but the current device is cuda:{cur}; "
                         f"call under torch.cuda.device({dev})")
    if stream is None:
        stream = torch.cuda.current_stream(dev)
    elif stream.device != dev:
        raise ValueError(f"stream belongs to {stream.device}, the tensors to {dev}")
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn: str, rc: int):
    if rc != 0:
        raise WQError(fn, rc)


def _dt(dtype: torch.dtype) -> int:
    if dtype == torch.float16:
        return F16
    if dtype == torch.bfloat16:
        return BF16
    raise ValueError(f"activation dtype must be float16 or bfloat16, got {dtype}")


def _torch_dt(dt: int) -> torch.dtype:
    return torch.float16 if dt == F16 else torch.bfloat16


def wq_packed_bytes(K: int, N: int, bits: int, group_size: int, mode: int) -> int:
    return int(lib().wq_packed_bytes(K, N, bits, group_size, mode))


def wq_workspace_bytes(M: int, N: int, K: int, bits: int, has_perm: bool) -> int:
    return int(lib().wq_workspace_bytes(M, N, K, bits, int(bool(has_perm))))


@dataclasses.dataclass
class PackedLayer:
    """A repacked layer: the library's tile-layout buffer plus its description."""
    packed: torch.Tensor                 # uint8 device buffer (codes + scales + zero-points)
    K: int
    N: int
    bits: int
    group_size: int
    mode: int
    lut: Optional[torch.Tensor] = None   # fp16 [2^bits] (table mode)
    perm: Optional[torch.Tensor] = None  # int32 [K] (act-order)
    gate_up: bool = False                # repacked by wq_repack_gate_up (interleaved halves)


def _need(cond: bool, what):
    """Raise ValueError(what) unless cond; `what` may be a callable that builds
    the message (so a passing check costs no string formatting)."""
    if not cond:
        raise ValueError(what() if callable(what) else what)


def _check_tensor(t, name: str, dtypes, shape, device=None):
    """t must be a contiguous tensor of one of `dtypes` with `shape` (and on `device`)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a tensor")
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if t.shape != shape:
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if device is not None and t.device != device:
        raise ValueError(f"{name} must be on {device}, got {t.device}")


def _check_cuda(t, name: str):
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor, got {t.device}")


_FINE_ZG = {ZERO_F16_G8: 8, ZERO_F16_G16: 16, ZERO_F16_G32: 32}


def _repack(fn: str, qweight, scales, zeros, mode, g_idx, K, N, bits, group_size, lut, stream) -> PackedLayer:
    # Every buffer is read by kernels through raw pointers: check shapes, dtypes,
    # layout and device before anything is launched.
    _need(bits in (2, 3, 4), lambda: f"bits must be 2, 3 or 4, got {bits}")
    _need(K > 0 and N > 0 and (K * bits) % 32 == 0, lambda: f"bad shape K={K} N={N} bits={bits}")
    _need(group_size == -1 or (group_size > 0 and K % group_size == 0), lambda: f"bad group_size {group_size}")
    _need(mode in (SYM, ZERO_F16, ZERO_PACKED, LUT, ZERO_F16_G8, ZERO_F16_G16, ZERO_F16_G32),
          lambda: f"bad mode {mode}")
    G = 1 if group_size == -1 else K // group_size
    dev = qweight.device if isinstance(qweight, torch.Tensor) else None
    _check_tensor(qweight, "qweight", (torch.int32,), (K * bits // 32, N), dev)
    _check_tensor(scales, "scales", (torch.float16,), (G, N), dev)
    if mode == ZERO_F16:
        _check_tensor(zeros, "zeros", (torch.float16,), (G, N), dev)
    elif mode == ZERO_PACKED:
        _need((N * bits) % 32 == 0, "packed zero-points need N*bits % 32 == 0")
        _check_tensor(zeros, "zeros", (torch.int32,), (G, N * bits // 32), dev)
    elif mode in _FINE_ZG:
        _need(K % _FINE_ZG[mode] == 0, "K must be a multiple of the zero-point group")
        _check_tensor(zeros, "zeros", (torch.float16,), (K // _FINE_ZG[mode], N), dev)
    else:
        _need(zeros is None, "zeros must be None for this mode")
    if mode == LUT:
        _check_tensor(lut, "lut", (torch.float16,), (1 << bits,), dev)
    else:
        _need(lut is None, "lut is only used in table mode")
    if g_idx is not None:
        _need(len(g_idx) == K, lambda: f"g_idx must have K={K} entries")
    _check_cuda(qweight, "qweight")
    nbytes = wq_packed_bytes(K, N, bits, group_size, mode)
    if nbytes == 0:
        raise WQError("wq_packed_bytes", 2)
    packed = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    perm = None
    g_host = None
    if g_idx is not None:
        import numpy as np
        g_host = np.ascontiguousarray(torch.as_tensor(g_idx).cpu().numpy(), dtype=np.int32)
        perm = torch.empty(K, dtype=torch.int32, device=dev)
    rc = getattr(lib(), fn)(_ptr(qweight), _ptr(scales), _ptr(zeros), mode,
                            None if g_host is None else ctypes.c_void_p(g_host.ctypes.data),
                            K, N, bits, group_size, _ptr(packed), _ptr(perm), _stream(stream, dev))
    _check(fn, rc)
    return PackedLayer(packed, K, N, bits, group_size, mode, lut, perm, fn == "wq_repack_gate_up")


def wq_repack(qweight: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor], mode: int,
              g_idx, K: int, N: int, bits: int, group_size: int, lut: Optional[torch.Tensor] = None,
              stream=None) -> PackedLayer:
    """Canonical GPTQ-style tensors (device: qweight int32 [K*bits/32][N], scales fp16
    [G][N], zeros fp16 [G][N], int32 [G][N*bits/32] or fp16 [K/zg][N] for the fine
    zero-point modes) -> PackedLayer.  g_idx: host int32 array-like [K] or None."""
    return _repack("wq_repack", qweight, scales, zeros, mode, g_idx, K, N, bits, group_size, lut, stream)


def wq_repack_gate_up(qweight: torch.Tensor, scales: torch.Tensor, zeros: Optional[torch.Tensor], mode: int,
                      g_idx, K: int, N: int, bits: int, group_size: int, lut: Optional[torch.Tensor] = None,
                      stream=None) -> PackedLayer:
    """Like wq_repack for a [gate | up] layer (N = 2I, N % 32 == 0); the result feeds
    wq_gemv_gate_up / wq_gemm_gate_up."""
    return _repack("wq_repack_gate_up", qweight, scales, zeros, mode, g_idx, K, N, bits, group_size, lut,
                   stream)


def _check_layer(layer: PackedLayer, dev):
    """The layer's buffers as the kernels read them: the packed buffer at least
    wq_packed_bytes long, the table fp16 [2^bits], the permutation int32 [K],
    all contiguous and on `dev`."""
    p = layer.packed
    _need(isinstance(p, torch.Tensor) and p.dtype == torch.uint8 and p.dim() == 1 and p.is_contiguous(),
          "layer.packed must be a contiguous 1-D uint8 tensor")
    _need(p.device == dev, "x and the layer must be on the same device")
    _need(p.numel() >= wq_packed_bytes(layer.K, layer.N, layer.bits, layer.group_size, layer.mode),
          "layer.packed is shorter than the packed size of the layer it describes")
    _need((layer.lut is not None) == (layer.mode == LUT), "a table is needed exactly in table mode")
    if layer.lut is not None:
        _check_tensor(layer.lut, "layer.lut", (torch.float16,), (1 << layer.bits,), dev)
    if layer.perm is not None:
        _check_tensor(layer.perm, "layer.perm", (torch.int32,), (layer.K,), dev)


def wq_dequant_debug(layer: PackedLayer, dtype: torch.dtype, stream=None) -> torch.Tensor:
    _dt(dtype)
    _check_layer(layer, layer.packed.device)
    _check_cuda(layer.packed, "layer.packed")
    w = torch.empty((layer.K, layer.N), dtype=dtype, device=layer.packed.device)
    rc = lib().wq_dequant_debug(_ptr(layer.packed), layer.mode, _ptr(layer.lut), _ptr(layer.perm),
                                layer.K, layer.N, layer.bits, layer.group_size, _dt(dtype), _ptr(w),
                                _stream(stream, w.device))
    _check("wq_dequant_debug", rc)
    return w


def _product(fn: str, x: torch.Tensor, layer: PackedLayer, out: Optional[torch.Tensor],
             ws: Optional[torch.Tensor], stream) -> torch.Tensor:
    # The kernels take raw pointers: a short or misplaced buffer would be read
    # or written out of bounds on the device, so everything is checked here,
    # before the library is called.
    _need(isinstance(x, torch.Tensor) and x.dim() == 2 and x.shape[1] == layer.K and x.is_contiguous(),
          "x must be a contiguous [M][K] tensor")
    _dt(x.dtype)
    M = x.shape[0]
    fused = "_gate_up" in fn
    if fused != layer.gate_up:
        raise ValueError(f"{fn} needs a layer repacked by "
                         f"{'wq_repack_gate_up' if fused else 'wq_repack'}")
    ncols = layer.N // 2 if fused else layer.N
    if out is not None:
        _check_tensor(out, "out", (x.dtype,), (M, ncols), x.device)
    need = wq_workspace_bytes(M, layer.N, layer.K, layer.bits, layer.perm is not None)
    if ws is not None and need:
        _need(isinstance(ws, torch.Tensor) and ws.is_contiguous() and ws.device == x.device,
              "ws must be a contiguous tensor on the device of x")
        _need(ws.numel() * ws.element_size() >= need, lambda: f"ws holds fewer than the {need} bytes this call needs")
    _check_layer(layer, x.device)
    _check_cuda(x, "x")
    if out is None:
        out = torch.empty((M, ncols), dtype=x.dtype, device=x.device)
    if need and ws is None:
        ws = torch.empty(need, dtype=torch.uint8, device=x.device)
    rc = getattr(lib(), fn)(_ptr(x), _dt(x.dtype), _ptr(layer.packed), layer.mode, _ptr(layer.lut),
                            _ptr(layer.perm), _ptr(out), M, layer.N, layer.K, layer.bits, layer.group_size,
                            _ptr(ws) if need else None, need if need else 0, _stream(stream, x.device))
    _check(fn, rc)
    return out


def wq_gemv(x: torch.Tensor, layer: PackedLayer, out=None, ws=None, stream=None) -> torch.Tensor:
    """y = x . dequant(W) for 1 <= M <= 32 (decode)."""
    return _product("wq_gemv", x, layer, out, ws, stream)


def wq_gemm(x: torch.Tensor, layer: PackedLayer, out=None, ws=None, stream=None) -> torch.Tensor:
    """y = x . dequant(W) for any M (prefill)."""
    return _product("wq_gemm", x, layer, out, ws, stream)


NOALLOC_SCRATCH_BYTES = 64 << 20  # WQ_NOALLOC_SCRATCH_BYTES


def wq_gemm_noalloc(x: torch.Tensor, layer: PackedLayer, out: torch.Tensor, stream=None) -> torch.Tensor:
    """wq_gemm with the library's static scratch array instead of a workspace:
    neither this call nor the library allocates (the caller passes `out`).
    Calls that overlap in time on one GPU race on that array."""
    _need(not layer.gate_up, "wq_gemm_noalloc takes a layer repacked by wq_repack")
    _need(isinstance(x, torch.Tensor) and x.dim() == 2 and x.shape[1] == layer.K and x.is_contiguous(),
          "x must be a contiguous [M][K] tensor")
    _dt(x.dtype)
    _check_tensor(out, "out", (x.dtype,), (x.shape[0], layer.N), x.device)
    _check_layer(layer, x.device)
    _check_cuda(x, "x")
    rc = lib().wq_gemm_noalloc(_ptr(x), _dt(x.dtype), _ptr(layer.packed), layer.mode, _ptr(layer.lut),
                               _ptr(layer.perm), _ptr(out), x.shape[0], layer.N, layer.K, layer.bits,
                               layer.group_size, _stream(stream, x.device))
    _check("wq_gemm_noalloc", rc)
    return out


def wq_gemv_gate_up(x: torch.Tensor, layer: PackedLayer, out=None, ws=None, stream=None) -> torch.Tensor:
    """h [M][N/2] = SiLU(x . gate) * (x . up) for 1 <= M <= 32."""
    return _product("wq_gemv_gate_up", x, layer, out, ws, stream)


def wq_gemm_gate_up(x: torch.Tensor, layer: PackedLayer, out=None, ws=None, stream=None) -> torch.Tensor:
    """h [M][N/2] = SiLU(x . gate) * (x . up) for any M."""
    return _product("wq_gemm_gate_up", x, layer, out, ws, stream)


def wq_hadamard(x: torch.Tensor, block: int, out: Optional[torch.Tensor] = None, stream=None) -> torch.Tensor:
    """Rows of x [M][K] rotated by the orthonormal block-diagonal Walsh-Hadamard
    matrix of size `block` (out may be x itself: in place)."""
    if x.dim() != 2 or not x.is_contiguous():
        raise ValueError("x must be a contiguous [M][K] tensor")
    M, K = x.shape
    _dt(x.dtype)
    if out is None:
        out = torch.empty_like(x)
    elif out.shape != x.shape or out.dtype != x.dtype or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous tensor like x, on its device")
    _check_cuda(x, "x")
    rc = lib().wq_hadamard(_ptr(x), _dt(x.dtype), _ptr(out), M, K, block, _stream(stream, x.device))
    _check("wq_hadamard", rc)
    return out


# Largest M that linear() sends to wq_gemv (which takes M <= 32).  Measured on
# MI355X over the LLaMA-7B/70B/405B layer shapes (graph-replayed, rotated
# copies): the GEMV beats the tiled GEMM at M = 17-32 on every shape and code
# width but two.  2-bit table layers take a second pass over the weights for
# rows 16-31.  4-bit table layers hold 64 KiB of LDS per workgroup above 16
# rows (the pair table and the activation stages), so two workgroups fit per
# CU, and with more than 1024 column tiles the grid needs a second round: on
# the 8192 x 28672 layer the GEMM is 13-17 % faster at M = 17-32, while on
# 28672 x 8192 the GEMV stays 5-6 % ahead.
GEMV_MAX_M = 32
_LUT4_GEMV_MAX_N = 16384  # 1024 column tiles


def use_gemv(M: int, layer: PackedLayer) -> bool:
    """Whether linear() sends an M-row product with this layer to the GEMV."""
    if layer.mode == LUT and M > 16:
        if layer.bits == 2 or (layer.bits == 4 and layer.N > _LUT4_GEMV_MAX_N):
            return False
    return M <= GEMV_MAX_M


def linear(x: torch.Tensor, layer: PackedLayer, out=None, ws=None, stream=None) -> torch.Tensor:
    """Decode-sized M (use_gemv) goes to wq_gemv, larger M to wq_gemm (the
    *_gate_up pair for a layer from wq_repack_gate_up)."""
    small = use_gemv(x.shape[0], layer)
    if layer.gate_up:
        return (wq_gemv_gate_up if small else wq_gemm_gate_up)(x, layer, out, ws, stream)
    return (wq_gemv if small else wq_gemm)(x, layer, out, ws, stream)
