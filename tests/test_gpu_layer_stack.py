"""GPU parity of the token-by-token decode stack (weight_only_quantized_w4a16_amd.stack).

Two LLaMA-7B-shaped decoder layers at full size.  Every product of the chain is
checked against the oracle on the very input the GPU used (teacher forcing):
the plain products within max|y - y_ref| <= 5e-3 max|y_ref| + 1e-3, the fused
gate+up with the bound of tests/test_gpu_gate_up.py, on a seeded sample of
output columns.  The stack is also replayed from a HIP graph several times,
with eager work in between, and every replay must equal the eager step.
"""
import numpy as np
import pytest
import torch

import workloads as wl
from _util import bits_to_tensor, repack_layer, tensor_bits, tensor_f64, within_tolerance
from test_gpu_gate_up import gate_up_bound, repack_gate_up

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_w4a16_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


@pytest.fixture(scope="module")
def stack2(wq):
    from weight_only_quantized_w4a16_amd.stack import DecoderWeights
    layers, raw = [], []
    for li in range(2):
        Ls = {n: wl.stack_layer(li, n) for (n, _, _) in wl.LLAMA7B}
        layers.append(DecoderWeights(repack_layer(wq, Ls["qkv"]), repack_layer(wq, Ls["o_proj"]),
                                     repack_gate_up(wq, Ls["gate_up"]), repack_layer(wq, Ls["down"])))
        raw.append(Ls)
    return layers, raw


def lin_ref(orc, x_bits, L, cols):
    return orc.linear(x_bits, wl.F16, L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, x_bits.shape[0], L.N,
                      L.K, L.bits, L.group_size, cols)


def check_plain(orc, x, y, L, seed):
    cols = wl.sample_cols(L.N, 96, seed)
    ref = lin_ref(orc, tensor_bits(x), L, cols)
    ok, err, bound = within_tolerance(tensor_f64(y)[:, cols], ref)
    assert ok, f"{L.name}: max error {err:.3e} > bound {bound:.3e}"


@pytest.mark.parametrize("M", [1, 4])
def test_stack_teacher_forced_parity(orc, wq, stack2, M):
    from weight_only_quantized_w4a16_amd.stack import DecodeStack
    layers, raw = stack2
    st = DecodeStack(layers, M, torch.float16, "cuda")
    x = bits_to_tensor(wl.make_x(M, st.dim, wl.F16, 70 + M), torch.float16, "cuda")
    rec = []
    y = st.step(x, record=rec)
    torch.cuda.synchronize()
    assert len(rec) == 2 and torch.equal(rec[-1]["y"], y)
    for r, Ls in zip(rec, raw):
        li = r["layer"]
        print(f"[stack] M={M} layer={li}", flush=True)
        assert torch.equal(r["attn"], r["qkv"][:, :st.dim])
        check_plain(orc, r["x"], r["qkv"], Ls["qkv"], 10 * li + 1)
        check_plain(orc, r["attn"], r["o"], Ls["o_proj"], 10 * li + 2)
        check_plain(orc, r["h"], r["y"], Ls["down"], 10 * li + 3)
        # fused gate+up on the o_proj output
        L = Ls["gate_up"]
        I = L.N // 2
        cols = wl.sample_cols(I, 96, 10 * li + 4)
        ob = tensor_bits(r["o"])
        h_ref = orc.linear_gate_up(ob, wl.F16, L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, M, L.N, L.K,
                                   L.bits, L.group_size, cols)
        y_gu = lin_ref(orc, ob, L, np.concatenate([cols, cols + I]).astype(np.int32))
        got = tensor_f64(r["h"])[:, cols]
        assert np.all(np.abs(got - h_ref) <= gate_up_bound(y_gu, h_ref, wl.F16))
    if M > 1:
        # layer 1 consumes layer 0's output
        assert torch.equal(rec[1]["x"], rec[0]["y"])


def test_stack_graph_replays_equal_eager(wq, stack2):
    from weight_only_quantized_w4a16_amd.stack import DecodeStack
    layers, _ = stack2
    st = DecodeStack(layers, 1, torch.float16, "cuda")
    x = bits_to_tensor(wl.make_x(1, st.dim, wl.F16, 99), torch.float16, "cuda")
    eager = st.step(x).clone()
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(cap):
        with torch.cuda.graph(g, stream=cap):
            out = st.step(x, stream=cap)
    torch.cuda.current_stream().wait_stream(cap)
    torch.cuda.synchronize()
    for i in range(3):
        st.qkv_out.zero_()  # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager), f"replay {i} differs from the eager step"
