"""W4A16 linear layers on top of the C ABI: QLinear and fused projections.

QLinear holds one weight in the library's device layout and applies
Y = X . dequant(W)^T (+ bias) with w4a16_gemm.  fuse() concatenates several
layers that read the same input along the output dimension -- the q, k and v
projections of an attention block, or gate and up of an MLP, the fusion
AutoAWQ's test plan checks ("fusing qkv") -- into one weight, so the group
runs as one launch; the outputs come back as column views of one Y.

Argument marshalling only: quantization, packing, layout conversion and the
product all run in the library's kernels.
"""
from __future__ import annotations

from typing import Optional, Sequence

import torch

from . import PackedWeight, gemm, pack, quantize, repack


class QLinear(torch.nn.Module):
    """y = x . dequant(W)^T (+ bias) for an int4 group-quantized W [N, K].

    The canonical quantized tensors (qpacked [N, K/8], scales [N, G],
    zpacked [N, ceil(G/8)] or None) are kept alongside the device layout so
    that layers can be fused later; pass keep_canonical=False to drop them."""

    def __init__(self, qpacked: torch.Tensor, scales: torch.Tensor,
                 zpacked: Optional[torch.Tensor], K: int, g: int,
                 bias: Optional[torch.Tensor] = None, keep_canonical: bool = True):
        super().__init__()
        self.K, self.g = K, g
        self.N = qpacked.shape[0]
        self.symmetric = zpacked is None
        self.packed: PackedWeight = repack(qpacked, scales, zpacked, K, g,
                                           symmetric=self.symmetric, partial=K % g != 0)
        self.canonical = (qpacked, scales, zpacked) if keep_canonical else None
        self.bias = bias

    @classmethod
    def from_float(cls, W: torch.Tensor, g: int = 128, symmetric: bool = False,
                   bias: Optional[torch.Tensor] = None, keep_canonical: bool = True):
        """Round-to-nearest group quantization of an fp16 weight W [N, K] on
        the device (w4a16_quantize), then the device layout (w4a16_repack)."""
        N, K = W.shape
        qp, sc, zp = quantize(W.to(torch.float16).contiguous(), g, symmetric=symmetric,
                              partial=K % g != 0)
        return cls(qp, sc, zp, K, g, bias=bias, keep_canonical=keep_canonical)

    @classmethod
    def from_codes(cls, codes: torch.Tensor, scales: torch.Tensor,
                   zeros: Optional[torch.Tensor], g: int,
                   bias: Optional[torch.Tensor] = None, keep_canonical: bool = True):
        """codes uint8 [N, K] (0..15), scales fp16/bf16 [N, G], zeros uint8
        [N, G] or None (symmetric), all on the device."""
        K = codes.shape[1]
        return cls(pack(codes), scales, None if zeros is None else pack(zeros), K, g,
                   bias=bias, keep_canonical=keep_canonical)

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None) -> torch.Tensor:
        shape = x.shape
        y = gemm(x.reshape(-1, self.K), self.packed, out=out)
        if self.bias is not None:
            y.add_(self.bias)   # in place: a caller's `out` holds the result
        return y.reshape(*shape[:-1], self.N)


class FusedQLinear(torch.nn.Module):
    """Several QLinear layers over the same input as one weight [sum N, K]:
    one w4a16_gemm per call; forward returns one view per part."""

    def __init__(self, fused: QLinear, sizes: Sequence[int]):
        super().__init__()
        self.fused = fused
        self.sizes = list(sizes)

    def forward(self, x: torch.Tensor, out: Optional[torch.Tensor] = None):
        y = self.fused(x, out=out)
        return torch.split(y, self.sizes, dim=-1)


def fuse(layers: Sequence[QLinear]) -> FusedQLinear:
    """Concatenate layers with the same K, group size, symmetry and 16-bit
    format along N (canonical tensors required)."""
    if not layers:
        raise ValueError("nothing to fuse")
    first = layers[0]
    for lay in layers:
        if lay.canonical is None:
            raise ValueError("fusing needs the canonical tensors (keep_canonical=True)")
        if (lay.K, lay.g, lay.symmetric) != (first.K, first.g, first.symmetric):
            raise ValueError("fused layers need the same K, group size and symmetry")
        if lay.canonical[1].dtype != first.canonical[1].dtype:
            raise ValueError("fused layers need the same scale format")
        if lay.bias is not None:
            raise ValueError("fusing layers with a bias is not supported")
    qp = torch.cat([lay.canonical[0] for lay in layers], 0)
    sc = torch.cat([lay.canonical[1] for lay in layers], 0)
    zp = None if first.symmetric else torch.cat([lay.canonical[2] for lay in layers], 0)
    return FusedQLinear(QLinear(qp, sc, zp, first.K, first.g), [lay.N for lay in layers])
