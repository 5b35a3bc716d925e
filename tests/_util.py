"""Helpers shared by the tests: move seeded workload arrays to the GPU and
compare GPU results with the oracle."""
import numpy as np
import torch

import workloads as wl

TOL_REL = 5e-3
TOL_ABS = 1e-3


def act_dtype(dt: int) -> torch.dtype:
    return torch.float16 if dt == wl.F16 else torch.bfloat16


def bits_to_tensor(a: np.ndarray, dtype: torch.dtype, device) -> torch.Tensor:
    """uint16 / uint32 bit patterns -> a device tensor of `dtype` with the same bits."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        t = torch.from_numpy(a.view(np.int16)).view(dtype)
    elif a.dtype == np.uint32:
        t = torch.from_numpy(a.view(np.int32))
    else:
        t = torch.from_numpy(a)
    return t.to(device)


def tensor_bits(t: torch.Tensor) -> np.ndarray:
    """16-bit float tensor -> uint16 bit patterns (host)."""
    return t.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def tensor_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().double().numpy()


def repack_layer(wq, L: wl.Layer, device="cuda"):
    q = bits_to_tensor(L.qweight, torch.int32, device)
    s = bits_to_tensor(L.scales, torch.float16, device)
    z = None
    if L.mode == wl.ZERO_F16 or L.mode in wl.FINE_ZERO_GROUP:
        z = bits_to_tensor(L.zeros, torch.float16, device)
    elif L.mode == wl.ZERO_PACKED:
        z = bits_to_tensor(L.zeros, torch.int32, device)
    lut = bits_to_tensor(L.lut, torch.float16, device) if L.lut is not None else None
    return wq.wq_repack(q, s, z, L.mode, L.g_idx, L.K, L.N, L.bits, L.group_size, lut=lut)


def oracle_y(orc, x_bits, dt, L: wl.Layer, cols=None):
    M = x_bits.shape[0]
    return orc.linear(x_bits, dt, L.qweight, L.scales, L.zeros, L.mode, L.lut, L.g_idx, M, L.N, L.K,
                      L.bits, L.group_size, cols)


def within_tolerance(y_gpu: np.ndarray, y_ref: np.ndarray):
    """max|y_gpu - y_ref| <= 5e-3 * max|y_ref| + 1e-3 over the whole output."""
    err = float(np.max(np.abs(y_gpu - y_ref))) if y_ref.size else 0.0
    bound = TOL_REL * (float(np.max(np.abs(y_ref))) if y_ref.size else 0.0) + TOL_ABS
    return err <= bound, err, bound
