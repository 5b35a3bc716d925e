"""Seeded synthetic workloads for y = x . dequant(W).

This module only draws inputs.  It holds none of the method's arithmetic: no
packing, no dequantisation, no product.  Packed codes are drawn as uniformly
random 32-bit words, which makes every code of every width uniform over
[0, 2^bits) whatever the packing convention; packed zero-points likewise.

The pages measure on real LLaMA / OPT checkpoints (Triton GPTQ page,
"Highlighted Details"; exllama bandwidth discussion, GPTQ paper quote).  No
weights or datasets are available, so seeded tensors with those models' layer
shapes and the stated value ranges stand in for them.

Value recipe (same for every consumer):
  codes    random uint32 words                 -> uniform codes
  scales   fp16 of U[lo, hi] drawn in fp64       (one per (group, column))
  zeros    fp16 of U[6, 10], or random uint32 words (packed, uniform codes)
  lut      fp16 table (normal-float quantiles, or the uniform integer grid)
  g_idx    pi = permutation(K); g_idx[pi[i]] = i // group_size  (balanced)
  x        fp16 / bf16 of N(0, 1) drawn in fp64
Weights draw from Generator(PCG64(seed)) in the order codes, scales, zeros,
g_idx; activations draw from their own Generator(PCG64(1000 * cfg + M)).
"""
from __future__ import annotations

import dataclasses
import statistics
from typing import Optional

import numpy as np

SYM, ZERO_F16, ZERO_PACKED, LUT = 0, 1, 2, 3
# fp16 zero-points in groups of 8 / 16 / 32 rows, independent of the scale group
ZERO_F16_G8, ZERO_F16_G16, ZERO_F16_G32 = 4, 5, 6
FINE_ZERO_GROUP = {ZERO_F16_G8: 8, ZERO_F16_G16: 16, ZERO_F16_G32: 32}
F16, BF16 = 0, 1
MODE_NAMES = {SYM: "sym", ZERO_F16: "zero_f16", ZERO_PACKED: "zero_packed", LUT: "lut",
              ZERO_F16_G8: "zero_f16_g8", ZERO_F16_G16: "zero_f16_g16", ZERO_F16_G32: "zero_f16_g32"}
DTYPE_NAMES = {F16: "f16", BF16: "bf16"}


# ----------------------------------------------------------------------------
# Number formats used to *store* drawn values (input preparation only).
# ----------------------------------------------------------------------------
def to_f16_bits(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, np.float64).astype(np.float16).view(np.uint16)


def to_bf16_bits(v: np.ndarray) -> np.ndarray:
    f = np.asarray(v, np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def to_act_bits(v: np.ndarray, dtype: int) -> np.ndarray:
    return to_bf16_bits(v) if dtype == BF16 else to_f16_bits(v)


# ----------------------------------------------------------------------------
# Lookup tables (FLUTE page, "Highlighted Details": int4 / nf4 / nf3 / nf2).
# ----------------------------------------------------------------------------
def nf_table(bits: int) -> np.ndarray:
    """Normal-float table: quantiles of N(0,1) at (i + 1/2) / 2^bits, scaled so
    the largest magnitude is 1, stored as fp16 bits.  (The pages only name the
    family; this is the plainest construction matching that name.)"""
    n = 1 << bits
    nd = statistics.NormalDist()
    q = np.array([nd.inv_cdf((i + 0.5) / n) for i in range(n)], np.float64)
    return to_f16_bits(q / np.max(np.abs(q)))


def uniform_table(bits: int) -> np.ndarray:
    """T[i] = i - 2^(bits-1): the table under which LUT mode equals symmetric mode."""
    n = 1 << bits
    return to_f16_bits(np.arange(n, dtype=np.float64) - n // 2)


# ----------------------------------------------------------------------------
# Layer and activation generation.
# ----------------------------------------------------------------------------
@dataclasses.dataclass
class Layer:
    K: int
    N: int
    bits: int
    group_size: int
    mode: int
    qweight: np.ndarray                 # uint32 [K*bits/32][N]
    scales: np.ndarray                  # uint16 fp16 bits [G][N]
    zeros: Optional[np.ndarray] = None  # uint16 [G][N] (fp16), uint32 [G][N*bits/32], or
                                        # uint16 [K/zg][N] (fp16, zero groups of zg rows)
    lut: Optional[np.ndarray] = None    # uint16 fp16 bits [2^bits]
    g_idx: Optional[np.ndarray] = None  # int32 [K]
    name: str = ""

    @property
    def G(self) -> int:
        return 1 if self.group_size == -1 else self.K // self.group_size

    def weight_bytes(self) -> int:
        """Codes + scales + zeros + table + g_idx-derived permutation: the bytes
        the method itself has to read for the weight."""
        b = self.qweight.nbytes + self.scales.nbytes
        if self.zeros is not None:
            b += self.zeros.nbytes
        if self.lut is not None:
            b += self.lut.nbytes
        if self.g_idx is not None:
            b += 4 * self.K
        return b


def make_layer(K: int, N: int, bits: int, group_size: int, mode: int, seed: int,
               scale_range=(0.005, 0.02), zero_range=(6.0, 10.0), lut: Optional[np.ndarray] = None,
               act_order: bool = False, name: str = "") -> Layer:
    if (K * bits) % 32:
        raise ValueError("K*bits must be a multiple of 32")
    G = 1 if group_size == -1 else K // group_size
    rng = np.random.Generator(np.random.PCG64(seed))
    qweight = rng.integers(0, 1 << 32, size=(K * bits // 32, N), dtype=np.uint64).astype(np.uint32)
    scales = to_f16_bits(rng.uniform(scale_range[0], scale_range[1], size=(G, N)))
    zeros = None
    if mode == ZERO_F16:
        zeros = to_f16_bits(rng.uniform(zero_range[0], zero_range[1], size=(G, N)))
    elif mode in FINE_ZERO_GROUP:
        zg = FINE_ZERO_GROUP[mode]
        if K % zg:
            raise ValueError("K must be a multiple of the zero group")
        zeros = to_f16_bits(rng.uniform(zero_range[0], zero_range[1], size=(K // zg, N)))
    elif mode == ZERO_PACKED:
        if (N * bits) % 32:
            raise ValueError("N*bits must be a multiple of 32 for packed zero-points")
        zeros = rng.integers(0, 1 << 32, size=(G, N * bits // 32), dtype=np.uint64).astype(np.uint32)
    g_idx = None
    if act_order:
        gs = K if group_size == -1 else group_size
        pi = rng.permutation(K)
        g_idx = np.empty(K, np.int32)
        g_idx[pi] = (np.arange(K) // gs).astype(np.int32)
    if mode == LUT and lut is None:
        lut = nf_table(bits)
    return Layer(K, N, bits, group_size, mode, qweight, scales, zeros,
                 lut if mode == LUT else None, g_idx, name)


def make_x(M: int, K: int, dtype: int, seed: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return to_act_bits(rng.standard_normal(size=(M, K)), dtype)


def sample_cols(N: int, count: int, seed: int) -> np.ndarray:
    """A seeded, sorted subset of output columns (for outputs checked one by one)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if count >= N:
        return np.arange(N, dtype=np.int32)
    return np.sort(rng.choice(N, size=count, replace=False)).astype(np.int32)


# ----------------------------------------------------------------------------
# The workload configurations.
# ----------------------------------------------------------------------------
LLAMA7B = [("qkv", 4096, 12288), ("o_proj", 4096, 4096), ("gate_up", 4096, 22016), ("down", 11008, 4096)]
LLAMA70B = [("up", 8192, 28672), ("down", 28672, 8192)]
LLAMA405B = [("wide", 16384, 53248), ("narrow", 14336, 4096)]


@dataclasses.dataclass
class Config:
    cid: int
    name: str
    layers: list                  # [(name, K, N)]
    Ms: list
    bits: list
    groups: list
    mode: int
    dtype: int
    seed: int
    scale_range: tuple = (0.005, 0.02)
    act_order: bool = False
    lut: str = ""                 # "nf" for normal-float tables

    def layer(self, lname: str, bits: Optional[int] = None, group_size: Optional[int] = None) -> Layer:
        K, N = next((k, n) for (nm, k, n) in self.layers if nm == lname)
        b = self.bits[0] if bits is None else bits
        g = self.groups[0] if group_size is None else group_size
        sr = self.scale_range
        if self.cid == 3 and g == -1:
            sr = (0.002, 0.01)
        # one weight seed per (config, layer, bits, group) so every layer is distinct
        li = [nm for (nm, _, _) in self.layers].index(lname)
        seed = self.seed * 1_000_003 + li * 101 + b * 7 + (0 if g == -1 else g)
        return make_layer(K, N, b, g, self.mode, seed, scale_range=sr,
                          lut=nf_table(b) if self.mode == LUT else None,
                          act_order=self.act_order, name=f"{self.name}/{lname}")

    def x(self, M: int, K: int) -> np.ndarray:
        return make_x(M, K, self.dtype, 1000 * self.cid + M + K)


CONFIGS = {
    1: Config(1, "c1_single_4096", [("layer", 4096, 4096)], [1], [4], [128], SYM, F16, 0),
    2: Config(2, "c2_llama7b_decode", LLAMA7B, [1, 4, 16], [4], [128], ZERO_F16, F16, 1),
    3: Config(3, "c3_llama7b_prefill", LLAMA7B, [512, 2048, 4096], [4], [-1, 128], SYM, F16, 2,
              scale_range=(0.005, 0.02)),
    4: Config(4, "c4_llama70b_lut", LLAMA70B, [1, 16, 64], [4, 3, 2], [64], LUT, BF16, 3,
              scale_range=(0.01, 0.05), lut="nf"),
    5: Config(5, "c5_act_order_packed_zeros", LLAMA405B, [1, 2, 8, 32, 128, 256], [4], [32],
              ZERO_PACKED, BF16, 4, act_order=True),
    # FLUTE page, "Limitations & Caveats": 4-bit, group 256, bf16 flagged unstable there.
    6: Config(6, "g256_regression", [("layer", 4096, 4096)], [1, 16, 2048], [4], [256], ZERO_F16, BF16, 5),
}


# ----------------------------------------------------------------------------
# Decode layer stack: LLaMA-7B-shaped decoder layers chained token by token.
# ----------------------------------------------------------------------------
STACK_SEED = 11


def stack_layer(li: int, lname: str) -> Layer:
    """Linear layer `lname` of decoder layer `li` of the LLaMA-7B-shaped stack:
    int4 codes, fp16 zero-points, group 128 (the decode configuration's
    quantisation), fp16 activations.  Zero-points are U[5.5, 9.5], centred on
    the mean code 7.5, so the weights have zero mean and no common-mode
    component builds up from layer to layer.  Scales are U[0.5, 1.5] * c with
    c = 1 / sqrt(E[U^2] * E[(q - z)^2] * K) (E[U^2] = 13/12,
    E[(q - z)^2] = 21.25 + 4/3 for uniform codes and zero-points), so a
    unit-variance input gives a unit-variance output; the down projection's c
    is raised by 1 / sqrt(0.36), the mean square of SiLU(g) * u for unit normal
    g and u, so activations keep their scale through any number of layers."""
    K, N = next((k, n) for (nm, k, n) in LLAMA7B if nm == lname)
    c = 1.0 / np.sqrt(13.0 / 12.0 * (21.25 + 4.0 / 3.0) * K)
    if lname == "down":
        c /= np.sqrt(0.36)
    li_name = [nm for (nm, _, _) in LLAMA7B].index(lname)
    seed = STACK_SEED * 1_000_003 + 1009 * li + li_name
    return make_layer(K, N, 4, 128, ZERO_F16, seed, scale_range=(0.5 * c, 1.5 * c), zero_range=(5.5, 9.5),
                      name=f"stack/{li}/{lname}")
