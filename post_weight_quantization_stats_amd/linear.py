"""Deployment linear layer over the packed weights the search writes.

A thin torch.nn.Module: it holds the packed codes, steps and zeros as
buffers and routes each call to a HIP contraction by token count, so
nothing of the product runs in PyTorch.

  * M <= 64 tokens: the decode contraction on decode tiles (made once per
    device on first use; weights streamed once from HBM; dequantized weight
    (q - z) * step exactly).
  * M > 64: the staged W4A16 product (the operand bf16(f32((q - z) * step))
    written once per call into a cached workspace, then the bf16
    matrix-core contraction; the same operand as the fused kernel that
    dequantizes in LDS, and faster once many tokens reuse each weight).

Both agree with the unrounded product to the contraction tolerance; they are
not bit-identical to each other.

Codes come in either packed layout: 4-bit containers (``quantize_pack``,
bits 3 or 4) or dense INT3 (``quantize_pack3``, 3 bits per weight), and at
any token count.  The module takes either metadata format: fp32 steps with u8
zeros (what the search writes), or the compact format of ``quantize_pack16``
(binary16 steps, two 4-bit zeros per byte: 2.5 bytes per group instead of 5).
In the compact format the decode contraction reads the compact metadata as
metadata tiles (one u32 per row and group beside the code tiles, made once
per device; 7-23% faster at one token than the per-workgroup table); the
many-token product reads an fp32/u8 copy expanded once per device.  The activation must already be divided by the search's scale s:
fold 1/s into the preceding op once, at load time (``fold_inverse_scale``),
as the method does ([RA How it works]: the activation is divided by the same
per-channel factor that multiplies the weight).
"""

from __future__ import annotations

import torch

from . import (LAYOUT_INT3_DENSE, LAYOUT_NIBBLE, OP_DECODE_GEMM, OP_W4A16_GEMM_STAGED,
               decode_gemm_tiled, decode_gemm_tiled_meta, decode_meta, decode_tiles, divide_rows,
               expand_meta16, quantize_pack16, w4a16_gemm, workspace_size)

DECODE_MAX_M = 64


class W4A16Linear(torch.nn.Module):
    """y = x . dequant(Q)^T for bf16 x [..., K] -> fp32 y [..., N].

    layout LAYOUT_NIBBLE: qweight int32 [N][K/8] (bits 3 or 4);
    LAYOUT_INT3_DENSE: qweight int32 [N][3K/32] (bits 3).  scales float16
    selects the compact format (zeros then uint8 [N][ceil(G/2)], two per
    byte); otherwise scales are fp32 and zeros u8 [N][G]."""

    def __init__(self, qweight: torch.Tensor, scales: torch.Tensor, zeros: torch.Tensor,
                 bits: int = 4, group: int = 128, layout: int = LAYOUT_NIBBLE):
        super().__init__()
        if layout not in (LAYOUT_NIBBLE, LAYOUT_INT3_DENSE):
            raise ValueError(f"unknown layout {layout}")
        if layout == LAYOUT_INT3_DENSE and bits != 3:
            raise ValueError("the dense INT3 layout holds 3-bit codes")
        if qweight.dtype != torch.int32 or qweight.dim() != 2:
            raise ValueError("qweight must be a 2-D int32 tensor")
        N = qweight.shape[0]
        if layout == LAYOUT_INT3_DENSE:
            if (qweight.shape[1] * 32) % 3:
                raise ValueError("dense INT3 qweight must be [N][3K/32]")
            K = qweight.shape[1] * 32 // 3
        else:
            K = qweight.shape[1] * 8
        G = K // group
        self.compact = scales.dtype == torch.float16
        zshape = (N, (G + 1) // 2) if self.compact else (N, G)
        if tuple(scales.shape) != (N, G) or tuple(zeros.shape) != zshape:
            raise ValueError(f"scales must be [N][K/group] and zeros {list(zshape)}")
        self.in_features, self.out_features = K, N
        self.bits, self.group, self.layout = bits, group, layout
        self.register_buffer("qweight", qweight.contiguous())
        self.register_buffer("scales", (scales if self.compact else scales.to(torch.float32)).contiguous())
        self.register_buffer("zeros", zeros.to(torch.uint8).contiguous())
        self._ws = None
        self._tiles = None
        self._meta_tiles = None
        self._meta32 = None

    @classmethod
    def compact_from_weight(cls, w: torch.Tensor, s: torch.Tensor | None, bits: int = 4,
                            group: int = 128, layout: int = LAYOUT_NIBBLE) -> "W4A16Linear":
        """The layer W . diag(s) packed in the compact format (the search's
        chosen s; binary16 steps, 4-bit zeros)."""
        qw, st, ze = quantize_pack16(w, s, bits, group, layout)
        return cls(qw, st, ze, bits, group, layout)

    @classmethod
    def from_search(cls, result: dict, bits: int = 4, group: int = 128) -> "W4A16Linear":
        """The layer written by ``search_scale`` / ``search_scale_gram``."""
        return cls(result["qweight"], result["scales"], result["zeros"], bits, group)

    def _workspace(self, need: int, device) -> torch.Tensor | None:
        if need <= 0:
            return None
        if self._ws is None or self._ws.numel() < need or self._ws.device != device:
            self._ws = torch.empty(need, dtype=torch.uint8, device=device)
        return self._ws

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        if x.shape[-1] != self.in_features:
            raise ValueError(f"expected {self.in_features} input features, got {x.shape[-1]}")
        lead = x.shape[:-1]
        x2 = x.reshape(-1, self.in_features)
        M = x2.shape[0]
        if M == 0:
            return torch.empty((*lead, self.out_features), dtype=torch.float32, device=x.device)
        N, K = self.out_features, self.in_features
        if M <= DECODE_MAX_M:
            ws = self._workspace(workspace_size(OP_DECODE_GEMM, M, N, K, self.bits, self.group),
                                 x.device)
            if self._tiles is None or self._tiles.device != self.qweight.device:
                self._tiles = decode_tiles(self.qweight, K, self.layout, self.group)
            if self.compact:
                if self._meta_tiles is None or self._meta_tiles.device != self.scales.device:
                    self._meta_tiles = decode_meta(self.scales, self.zeros, self.group)
                y = decode_gemm_tiled_meta(x2, self._tiles, self._meta_tiles, N, self.layout,
                                           self.group, workspace=ws)
            else:
                y = decode_gemm_tiled(x2, self._tiles, self.scales, self.zeros, self.layout,
                                      self.group, workspace=ws)
        else:
            scales, zeros = self.scales, self.zeros
            if self.compact:
                if self._meta32 is None or self._meta32[0].device != self.scales.device:
                    self._meta32 = expand_meta16(self.scales, self.zeros, self.group)
                scales, zeros = self._meta32
            ws = self._workspace(workspace_size(OP_W4A16_GEMM_STAGED, M, N, K, self.bits,
                                                self.group), x.device)
            y = w4a16_gemm(x2, self.qweight, scales, zeros, self.bits, self.group,
                           layout=self.layout, staged=True, workspace=ws)
        return y.reshape(*lead, self.out_features)

    def extra_repr(self) -> str:
        return (f"in_features={self.in_features}, out_features={self.out_features}, "
                f"bits={self.bits}, group={self.group}, layout={self.layout}, "
                f"compact={self.compact}")


def fold_inverse_scale(weight: torch.Tensor, s: torch.Tensor) -> torch.Tensor:
    """The preceding op's per-channel output weight (a norm's gain [C], or
    the rows [C][...] of a previous linear layer) divided by s [C], so that
    its output is X / s and feeds W4A16Linear directly.  A load-time
    transform, computed by the library's awq_divide_rows (one IEEE fp32
    division per element); returns float32 (a weight held in another dtype
    is widened first, exactly)."""
    return divide_rows(weight.to(torch.float32).contiguous(), s.to(torch.float32).contiguous())
