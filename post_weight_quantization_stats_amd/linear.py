"""Deployment linear layer over the packed weights the search writes.

A thin torch.nn.Module: it holds the packed codes, steps and zeros as
buffers and routes each call to a HIP contraction by token count, so
nothing of the product runs in PyTorch.

  * M <= 64 tokens: the decode contraction on decode tiles (made once per
    device on first use; weights streamed once from HBM; dequantized weight
    (q - z) * step exactly).
  * M > 64: the general W4A16 contraction (dequantized weight rounded to
    bf16 in LDS, the search's operand contract).

Both agree with the unrounded product to the contraction tolerance; they are
not bit-identical to each other.

The module takes either metadata format: fp32 steps with u8 zeros (what the
search writes), or the compact format of ``quantize_pack16`` (binary16 steps,
two 4-bit zeros per byte: 2.5 bytes per group instead of 5).  In the compact
format the decode contraction reads the compact metadata directly; the
contraction for many tokens reads an fp32/u8 copy expanded once per device.  The activation must already be divided by
the search's scale s: fold 1/s into the preceding op once, at load time
(``fold_inverse_scale``), as the method does ([RA How it works]: the
activation is divided by the same per-channel factor that multiplies the
weight).
"""

from __future__ import annotations

import torch

from . import (LAYOUT_NIBBLE, OP_DECODE_GEMM, decode_gemm_tiled, decode_gemm_tiled16,
               decode_tiles, expand_meta16, quantize_pack16, w4a16_gemm, workspace_size)

DECODE_MAX_M = 64


class W4A16Linear(torch.nn.Module):
    """y = x . dequant(Q)^T for bf16 x [..., K] -> fp32 y [..., N].

    scales float16 selects the compact format (zeros then uint8
    [N][ceil(G/2)], two per byte); otherwise scales are fp32 and zeros u8
    [N][G]."""

    def __init__(self, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                 bits: int = 4, group: int = 128):
        super().__init__()
        if qweight.dtype != torch.int32 or qweight.dim() != 2:
            raise ValueError("qweight must be int32 [N][K/8]")
        N, K = qweight.shape[0], qweight.shape[1] * 8
        G = K // group
        self.compact = scales.dtype == torch.float16
        zshape = (N, (G + 1) // 2) if self.compact else (N, G)
        if tuple(scales.shape) != (N, G) or tuple(zeros.shape) != zshape:
            raise ValueError(f"scales must be [N][K/group] and zeros {list(zshape)}")
        self.in_features, self.out_features = K, N
        self.bits, self.group = bits, group
        self.register_buffer("qweight", qweight.contiguous())
        self.register_buffer("scales", (scales if self.compact else scales.to(torch.float32)).contiguous())
        self.register_buffer("zeros", zeros.to(torch.uint8).contiguous())
        self._ws = None
        self._tiles = None
        self._meta32 = None

    @classmethod
    def compact_from_weight(cls, w: torch.Tensor, s: torch.Tensor | None, bits: int = 4,
                            group: int = 128) -> "W4A16Linear":
        """The layer W . diag(s) packed in the compact format (the search's
        chosen s; binary16 steps, 4-bit zeros)."""
        qw, st, ze = quantize_pack16(w, s, bits, group)
        return cls(qw, st, ze, bits, group)

    @classmethod
    def from_search(cls, result: dict, bits: int = 4, group: int = 128) -> "W4A16Linear":
        """The layer written by ``search_scale`` / ``search_scale_gram``."""
        return cls(result["qweight"], result["scales"], result["zeros"], bits, group)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected {self.in_features} input features, got {x.shape[-1]}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        M = x2.shape[0]
        if M == 0:
            return torch.empty((*lead, self.out_features), dtype=torch.float32, device=x.device)
        if M <= DECODE_MAX_M:
            need = workspace_size(OP_DECODE_GEMM, M, self.out_features, self.in_features,
                                  self.bits, self.group)
            ws = None
            if need > 0:
                if self._ws is None or self._ws.numel() < need or self._ws.device != x.device:
                    self._ws = torch.empty(need, dtype=torch.uint8, device=x.device)
                ws = self._ws
            if self._tiles is None or self._tiles.device != self.qweight.device:
                self._tiles = decode_tiles(self.qweight, self.in_features, LAYOUT_NIBBLE, self.group)
            decode = decode_gemm_tiled16 if self.compact else decode_gemm_tiled
            y = decode(x2, self._tiles, self.scales, self.zeros, LAYOUT_NIBBLE, self.group,
                       workspace=ws)
        else:
            scales, zeros = self.scales, self.zeros
            if self.compact:
                if self._meta32 is None or self._meta32[0].device != self.scales.device:
                    self._meta32 = expand_meta16(self.scales, self.zeros, self.group)
                scales, zeros = self._meta32
            y = w4a16_gemm(x2, self.qweight, scales, zeros, self.bits, self.group)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bits={self.bits}, group={self.group}, compact={self.compact}")


def fold_inverse_scale(weight: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    """The preceding op's per-channel output weight (a norm's gain, or the
    rows of a previous linear layer) divided by s, so that its output is
    X / s and feeds W4A16Linear directly.  A load-time transform of
    parameters, in fp32."""
    s = s.to(torch.float32)
    if weight.dim() == 1:
        return (weight.to(torch.float32) / s).to(weight.dtype)
    return (weight.to(torch.float32) / s[:, None]).to(weight.dtype)
