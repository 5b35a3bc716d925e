"""The C ABI: the library loads, exports every function include/wq.h declares,
and rejects malformed or unsupported arguments before touching the GPU.
Runs on the CPU (no compute calls)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wq.h")


@pytest.fixture(scope="module")
def L():
    import weight_only_quantized_w4a16_amd as wq
    if not os.path.exists(wq.LIB_PATH):
        from weight_only_quantized_w4a16_amd import build
        build.build()
    return wq.lib()


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(wq_[a-z_]+)\s*\(", src)))


def test_header_declares_the_entry_points():
    names = declared_functions()
    for required in ("wq_repack", "wq_dequant_debug", "wq_gemv", "wq_gemm", "wq_packed_bytes",
                     "wq_workspace_bytes", "wq_status_str", "wq_layout_version",
                     "wq_repack_gate_up", "wq_gemv_gate_up", "wq_gemm_gate_up", "wq_hadamard"):
        assert required in names


def test_library_exports_every_declared_function(L):
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings_and_version(L):
    assert L.wq_layout_version() == 3
    for s in range(5):
        assert L.wq_status_str(s)


def test_packed_bytes_matches_layout(L):
    # codes K*N*bits/8, scales G*N*2, zero-points, each section 256-byte aligned
    al = lambda v: (v + 255) // 256 * 256
    K, N = 4096, 4096
    codes = K * N // 2
    assert L.wq_packed_bytes(K, N, 4, 128, 0) == al(al(codes) + 32 * N * 2)
    assert L.wq_packed_bytes(K, N, 4, 128, 1) == al(al(codes) + 32 * N * 4)  # (scale, zero) pairs
    assert L.wq_packed_bytes(K, N, 4, 32, 2) == al(al(al(codes) + 128 * N * 2) + 128 * (N // 16) * 8)
    assert L.wq_packed_bytes(K, N, 3, -1, 3) == al(al(K * N * 3 // 8) + N * 2)
    # fine zero-points: 8 * (32 / zg) bytes per column per 128 rows
    for mode, zg in ((4, 8), (5, 16), (6, 32)):
        assert L.wq_packed_bytes(K, N, 2, -1, mode) == al(al(al(K * N // 4) + N * 2) + K * N * 2 // zg)
    assert L.wq_packed_bytes(K, N, 4, 128, 7) == 0   # no such mode
    # unsupported / invalid -> 0
    assert L.wq_packed_bytes(4096, 4104, 4, 128, 0) == 0   # N % 16
    assert L.wq_packed_bytes(4000, 4096, 4, 128, 0) == 0   # K % 128
    assert L.wq_packed_bytes(4096, 4096, 5, 128, 0) == 0   # bits
    assert L.wq_packed_bytes(4096, 4096, 4, 100, 0) == 0   # group does not divide K


def test_workspace_bytes(L):
    al = lambda v: (v + 255) // 256 * 256
    # 2 x 16 workgroups of 64 x 256 -> 16 slices allowed, capped at 4 k-tiles per slice
    assert L.wq_workspace_bytes(128, 4096, 4096, 4, 0) == 8 * 128 * 4096 * 4
    assert L.wq_workspace_bytes(128, 4096, 4096, 4, 1) == al(128 * 4096 * 2) + 8 * 128 * 4096 * 4
    # 8 x 16 workgroups -> 4 slices of 22 (last 20) k-tiles
    assert L.wq_workspace_bytes(512, 4096, 11008, 4, 0) == 4 * 512 * 4096 * 4
    assert L.wq_workspace_bytes(65, 53248, 16384, 4, 0) == 0         # 416 workgroups: no split
    assert L.wq_workspace_bytes(4096, 4096, 4096, 4, 0) == 0
    assert L.wq_workspace_bytes(128, 4096, 4096, 4, 1) > L.wq_workspace_bytes(128, 4096, 4096, 4, 0)
    # narrow problems split K: 16 workgroups of 256 columns -> 32 slices allowed,
    # capped at 4 k-tiles per slice (32 k-tiles -> 8 slices)
    assert L.wq_workspace_bytes(16, 4096, 4096, 4, 0) == 8 * 16 * 4096 * 4
    assert L.wq_workspace_bytes(16, 4096, 4096, 4, 1) == al(16 * 4096 * 2) + 8 * 16 * 4096 * 4
    # 208 workgroups -> 2 slices of 64 k-tiles (a third would exceed 512 workgroups)
    assert L.wq_workspace_bytes(32, 53248, 16384, 4, 0) == 2 * 32 * 53248 * 4
    # wide enough: no split
    assert L.wq_workspace_bytes(64, 131072, 4096, 4, 0) == 0


def call_product(L, fn, M=1, N=4096, K=4096, bits=4, gs=128, mode=0, dt=0, x=16, w=16, y=16, lut=None,
                 perm=None, ws=None, ws_bytes=0):
    P = ctypes.c_void_p
    return getattr(L, fn)(P(x), dt, P(w), mode, P(lut) if lut else None, P(perm) if perm else None, P(y),
                          M, N, K, bits, gs, P(ws) if ws else None, ws_bytes, None)


@pytest.mark.parametrize("fn", ["wq_gemv", "wq_gemm", "wq_gemv_gate_up", "wq_gemm_gate_up"])
def test_product_rejects_before_launch(L, fn):
    # fake, never-dereferenced pointers: validation must return before any launch
    assert call_product(L, fn, bits=5) == 1                      # WQ_EINVAL
    assert call_product(L, fn, dt=2) == 1
    assert call_product(L, fn, mode=7) == 1
    assert call_product(L, fn, gs=100) == 1                      # group does not divide K
    assert call_product(L, fn, K=4000) == 1                      # K not a multiple of group
    assert call_product(L, fn, K=4000, gs=-1) == 2               # K % 128: unsupported
    assert call_product(L, fn, N=4104) == 2                      # N % 16: unsupported
    assert call_product(L, fn, M=-1) == 1
    assert call_product(L, fn, mode=3) == 1                      # table mode without a table
    assert call_product(L, fn, x=0) == 1                         # NULL activations
    assert call_product(L, fn, x=8) == 2                         # misaligned
    assert call_product(L, fn, perm=64) == 4                     # act-order without workspace
    assert call_product(L, fn, perm=64, ws=64, ws_bytes=10) == 4
    assert call_product(L, fn, M=0) == 0                         # empty: no-op


def test_gemv_rejects_large_m(L):
    assert call_product(L, "wq_gemv", M=33) == 2
    assert call_product(L, "wq_gemv_gate_up", M=33) == 2


@pytest.mark.parametrize("fn", ["wq_gemv_gate_up", "wq_gemm_gate_up"])
def test_gate_up_needs_whole_tile_pairs(L, fn):
    # the gate and up halves must each be a whole number of 16-column tiles
    assert call_product(L, fn, N=4112) == 2
    assert call_product(L, fn, N=4112, M=0) == 2


@pytest.mark.parametrize("fn", ["wq_repack", "wq_repack_gate_up"])
def test_repack_rejects_before_launch(L, fn):
    P = ctypes.c_void_p
    f = getattr(L, fn)
    ok = dict(q=P(16), s=P(16), z=None, mode=0, g=None, K=4096, N=4096, bits=4, gs=128, out=P(16), perm=None)

    def call(**kw):
        a = dict(ok, **kw)
        return f(a["q"], a["s"], a["z"], a["mode"], a["g"], a["K"], a["N"], a["bits"], a["gs"], a["out"],
                 a["perm"], None)

    assert call(q=None) == 1
    assert call(mode=1) == 1                # fp16 zero-points missing
    # packed 3-bit zeros need N*3 % 32 == 0 (the gate+up repack rejects N % 32 first)
    assert call(mode=2, bits=3, N=4112, z=P(16)) == (1 if fn == "wq_repack" else 2)
    assert call(bits=3, K=4000) == 1
    g = (ctypes.c_int32 * 4096)(*([0] * 4096))
    assert call(g=ctypes.cast(g, P)) == 1   # g_idx without a perm buffer
    assert call(g=ctypes.cast(g, P), perm=P(16)) == 2  # unbalanced groups: unsupported
    bad = (ctypes.c_int32 * 4096)(*([99] * 4096))
    assert call(g=ctypes.cast(bad, P), perm=P(16)) == 1  # group index out of range
    if fn == "wq_repack_gate_up":
        assert call(N=4112) == 2            # halves must be whole 16-column tiles


def test_dequant_debug_rejects_before_launch(L):
    P = ctypes.c_void_p
    f = L.wq_dequant_debug
    assert f(P(16), 0, None, None, 4096, 4096, 4, 128, 3, P(16), None) == 1   # bad out dtype
    assert f(P(16), 3, None, None, 4096, 4096, 4, 128, 0, P(16), None) == 1   # table missing
    assert f(None, 0, None, None, 4096, 4096, 4, 128, 0, P(16), None) == 1


def test_hadamard_rejects_before_launch(L):
    P = ctypes.c_void_p

    def call(x=16, dt=0, y=4096, M=1, K=512, b=128):
        return L.wq_hadamard(P(x) if x else None, dt, P(y) if y else None, M, K, b, None)

    assert call(b=96) == 1            # not a power of two
    assert call(b=1) == 1
    assert call(b=1024) == 1          # larger than one wave holds
    assert call(K=384, b=256) == 1    # K % block
    assert call(dt=2) == 1
    assert call(M=-1) == 1
    assert call(x=0) == 1
    assert call(y=0) == 1
    assert call(x=8) == 2             # misaligned
    assert call(K=4, b=2) == 2        # K % 8
    assert call(y=16 + 256) == 1      # partial overlap
    assert call(M=0) == 0             # empty: no-op


def test_size_limits(L):
    """Every section of a repacked layer stays below 2 GiB (32-bit buffer
    offsets) and K, N below 2^24: larger layers are rejected up front."""
    assert L.wq_packed_bytes(65536, 65536, 4, 128, 0) == 0        # 2 GiB of codes
    assert L.wq_packed_bytes(65536, 65520, 4, 128, 0) > 0         # just below
    assert L.wq_packed_bytes(1 << 25, 16, 4, 128, 0) == 0         # K past 2^24
    assert call_product(L, "wq_gemv", K=65536, N=65536) == 2
    # activations: M*K*2 bytes must stay below 2 GiB
    assert call_product(L, "wq_gemm", M=1 << 18, K=4096) == 2


def test_bench_refuses_more_than_one_gpu():
    """The benchmark measures one GPU and says so for any other count (it
    exits before touching a GPU)."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_probe_library_exports_its_header():
    """libwq_probe.so (measurement probe, include/wq_probe.h) exports what it declares."""
    import ctypes

    from weight_only_quantized_w4a16_amd import build
    if not os.path.exists(build.PROBE_LIB):
        build.build()
    src = re.sub(r"/\*.*?\*/", "", open(os.path.join(ROOT, "include", "wq_probe.h")).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(wq_[a-z_]+)\s*\(", src)))
    assert names == ["wq_probe_stream_read"]
    P = ctypes.CDLL(build.PROBE_LIB)
    for n in names:
        assert hasattr(P, n), n
    f = P.wq_probe_stream_read
    f.argtypes = [ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    # malformed arguments are refused before any launch
    assert f(None, 4096, 64, 4, None, None) == 1
    assert f(ctypes.c_void_p(4096), 4095, 64, 4, ctypes.c_void_p(64), None) == 1  # not a multiple of 16
    assert f(ctypes.c_void_p(4096), 4096, 64, 3, ctypes.c_void_p(64), None) == 1  # loads in flight
    assert f(ctypes.c_void_p(4096), 1 << 31, 1, 4, ctypes.c_void_p(64), None) == 2  # 2 GiB chunk
