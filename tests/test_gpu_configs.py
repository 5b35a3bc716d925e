"""GPU parity at the full workload sizes, through the same entry points and
launch shapes the benchmark times.

Two checks per case:
  * the oracle computes every output row for a seeded set of output columns:
    one column of every 256-column block (the column blocks of the large-M
    product's workgroups and of the decode product's grids), all 16 columns of
    the last column tile, and seeded random columns up to about 2 GMAC of
    oracle work (all columns for small outputs); the tolerance is applied over
    that set;
  * every output: the whole y against a float32 product of x with the
    dequantised weights wq_dequant_debug writes (those bits equal the oracle's
    dequantisation, tests/test_gpu_parity.py), same tolerance, and all of y
    finite.
Workloads (layer shapes of the models the pages measure on, with seeded
synthetic values, see workloads.py):
  c1  one 4096 x 4096 layer, int4 symmetric, group 128, fp16, M = 1
  c2  LLaMA-7B decode layer set, int4 with fp16 zero-points, group 128, M = 1, 4, 16
  c3  the same shapes at prefill M = 512, 2048, 4096, symmetric, group -1 and 128
  c4  LLaMA-70B-shaped table-quantised layers, 4/3/2-bit normal-float tables,
      group 64, bf16, M = 1, 16, 64
  c5  405B-width act-order layers with packed 4-bit zero-points, group 32,
      bf16, M = 1, 2, 8, 32, 128, 256
  g256 4-bit group 256 bf16 regression shape, M = 1, 16, 2048
"""
import numpy as np
import pytest
import torch

import workloads as wl
from _util import act_dtype, bits_to_tensor, oracle_y, repack_layer, tensor_f64, within_tolerance

pytestmark = pytest.mark.gpu

ORACLE_MACS = 1e9  # oracle work per case (beyond the per-block columns, always checked)


def check_cols(N, M, K, seed):
    """One seeded column per 256-column block, the last 16-column tile, then
    seeded random columns while the oracle stays within ORACLE_MACS."""
    rng = np.random.Generator(np.random.PCG64(seed))
    blocks = [b * 256 + int(rng.integers(0, min(256, N - b * 256))) for b in range((N + 255) // 256)]
    cols = set(blocks) | set(range(N - 16, N))
    budget = int(ORACLE_MACS // (M * K))
    if budget > len(cols):
        extra = wl.sample_cols(N, min(N, budget), seed=seed + 1)
        cols |= set(int(c) for c in extra[:max(0, budget - len(cols))])
    return np.array(sorted(cols), np.int32)


@pytest.fixture(scope="module")
def wq():
    import weight_only_quantized_w4a16_amd as m
    m.lib()
    assert torch.cuda.is_available()
    return m


_layers = {}


def get_layer(wq, cfg, lname, bits, gs):
    key = (cfg.cid, lname, bits, gs)
    if key not in _layers:
        _layers.clear()  # keep at most one full-size layer alive
        L = cfg.layer(lname, bits, gs)
        _layers[key] = (L, repack_layer(wq, L))
    return _layers[key]


def cases():
    out = []
    for cid, cfg in wl.CONFIGS.items():
        for (lname, K, N) in cfg.layers:
            for bits in cfg.bits:
                for gs in cfg.groups:
                    for M in cfg.Ms:
                        out.append(pytest.param(cid, lname, bits, gs, M, id=f"{cfg.name}-{lname}-b{bits}-g{gs}-M{M}"))
    return out


@pytest.mark.parametrize("cid,lname,bits,gs,M", cases())
def test_config_parity(orc, wq, cid, lname, bits, gs, M):
    cfg = wl.CONFIGS[cid]
    print(f"[config] {cfg.name} {lname} bits={bits} group={gs} M={M}", flush=True)
    L, layer = get_layer(wq, cfg, lname, bits, gs)
    x_bits = cfg.x(M, L.K)
    x = bits_to_tensor(x_bits, act_dtype(cfg.dtype), "cuda")
    fn = wq.wq_gemv if wq.use_gemv(M, layer) else wq.wq_gemm
    y = fn(x, layer)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(y).all())
    # every output against x . dequant(W) in float32 (the debug weights are the oracle's)
    w = wq.wq_dequant_debug(layer, act_dtype(cfg.dtype)).float()
    ref_full = tensor_f64(x.float() @ w)
    del w
    ok, err, bound = within_tolerance(tensor_f64(y), ref_full)
    assert ok, f"whole output: max error {err:.3e} > bound {bound:.3e}"
    # the oracle on the column set
    if L.N * M <= 4096 * 16:
        cols = None
        got = tensor_f64(y)
    else:
        cols = check_cols(L.N, M, L.K, seed=cid * 100 + M)
        got = tensor_f64(y[:, torch.from_numpy(cols).long().cuda()])
    ref = oracle_y(orc, x_bits, cfg.dtype, L, cols)
    ok, err, bound = within_tolerance(got, ref)
    assert ok, f"oracle columns: max error {err:.3e} > bound {bound:.3e}"
