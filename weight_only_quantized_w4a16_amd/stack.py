"""Token-by-token decode through a stack of LLaMA-style quantised linear layers.

The pages measure generation speed in iterations per second of a whole model
(Triton GPTQ page, "Highlighted Details": LLaMA-7B, 4-bit against GPTQ CUDA
and FP16) and observe that decode is matrix-vector work bound by memory
bandwidth (exllama bandwidth discussion, GPTQ quote and turboderp's reply).
This module chains the library's entry points the way one decoder layer uses
its linear layers -- fused QKV, output projection, activation-fused gate+up,
down projection -- over many layers, so a step is one token through every
layer's weights.  Attention, normalisation and the residual path are not
weight-only-quantised products and are not modelled: the first `dim` columns
of the QKV output stand in for the attention output that feeds the output
projection.

Only argument marshalling and sequencing live here; every product runs in the
library's kernels.  All buffers are allocated once, so a step launches exactly
four kernels per layer (plus one copy per layer when M > 1, where the QKV
slice is not contiguous) and can be captured in a HIP graph.
"""
from __future__ import annotations

import dataclasses
from typing import List, Optional

import torch

from . import PackedLayer, use_gemv, wq_gemv, wq_gemv_gate_up, wq_gemm, wq_gemm_gate_up


@dataclasses.dataclass
class DecoderWeights:
    """The four repacked linear layers of one decoder layer."""
    qkv: PackedLayer       # [dim] -> [3 * dim] (fused Q, K, V)
    o: PackedLayer         # [dim] -> [dim]
    gate_up: PackedLayer   # [dim] -> [2 * inter], repacked by wq_repack_gate_up
    down: PackedLayer      # [inter] -> [dim]


class DecodeStack:
    """y = layer_L-1( ... layer_0(x)) with layer(x) = down(SiLU(gate(o(qkv(x)[:, :dim]))) * up(...))."""

    def __init__(self, layers: List[DecoderWeights], M: int, dtype: torch.dtype, device):
        if not layers:
            raise ValueError("empty stack")
        l0 = layers[0]
        self.dim, self.inter = l0.o.K, l0.down.K
        for L in layers:
            if not L.gate_up.gate_up:
                raise ValueError("gate_up must be repacked by wq_repack_gate_up")
            if (L.qkv.K, L.o.K, L.o.N, L.gate_up.K, L.gate_up.N, L.down.K, L.down.N) != \
                    (self.dim, self.dim, self.dim, self.dim, 2 * self.inter, self.inter, self.dim):
                raise ValueError("layer shapes do not chain")
            if L.qkv.N < self.dim:
                raise ValueError("the QKV output must hold at least dim columns")
        self.layers = layers
        self.M = M
        small = all(use_gemv(M, lay) for L in layers for lay in (L.qkv, L.o, L.gate_up, L.down))
        self._lin = wq_gemv if small else wq_gemm
        self._lin_gu = wq_gemv_gate_up if small else wq_gemm_gate_up
        e = dict(dtype=dtype, device=device)
        self.qkv_out = torch.empty((M, l0.qkv.N), **e)
        self.attn = torch.empty((M, self.dim), **e)
        self.o_out = torch.empty((M, self.dim), **e)
        self.h = torch.empty((M, self.inter), **e)
        self.x = [torch.empty((M, self.dim), **e), torch.empty((M, self.dim), **e)]

    def step(self, x: torch.Tensor, stream=None, record: Optional[list] = None) -> torch.Tensor:
        """One token (M rows) through every layer on `stream` (a torch stream; the
        current one by default); returns the last layer's output (a buffer of the
        stack, overwritten by the next step).  With `record`, the input and output
        of every product are appended as tensors (clones)."""
        if x.shape != (self.M, self.dim) or not x.is_contiguous():
            raise ValueError("x must be a contiguous [M][dim] tensor")
        cur = x
        for i, L in enumerate(self.layers):
            self._lin(cur, L.qkv, out=self.qkv_out, stream=stream)
            if self.M == 1:
                attn = self.qkv_out[:, :self.dim]  # a contiguous prefix of the single row
            else:
                attn = self.attn
                with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
                    attn.copy_(self.qkv_out[:, :self.dim])
            self._lin(attn, L.o, out=self.o_out, stream=stream)
            self._lin_gu(self.o_out, L.gate_up, out=self.h, stream=stream)
            nxt = self.x[i % 2]
            self._lin(self.h, L.down, out=nxt, stream=stream)
            if record is not None:
                record.append(dict(layer=i, x=cur.clone(), qkv=self.qkv_out.clone(), attn=attn.clone(),
                                   o=self.o_out.clone(), h=self.h.clone(), y=nxt.clone()))
            cur = nxt
        return cur
