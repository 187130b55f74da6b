"""The search run layer after layer through Llama-shaped feed-forward blocks.

Each block is x -> x + down(silu(gate(u)) * up(u)) with u = RMSNorm(x).  The
search quantizes the fused gate/up layer on the block's own normalised
activations, folds 1/s1 into the RMSNorm gain, runs the quantized gate/up as
deployed, searches the down layer on the resulting H, folds 1/s2 into the up
rows' steps, and hands the block's deployed output to the next block
(robotsatlas AWQ page, "How it works": the activation is divided by the
same per-channel factor that multiplies the weight, and a deployment folds
it into the preceding operation; "Computational complexity": one search per
layer, over the layers in order).

Only sequencing lives here: every step is one call into the HIP library,
and the tensors stay on the GPU.
"""

from __future__ import annotations

import torch

from . import (divide_rows, residual_add, rmsnorm, search_scale, search_scale_gram, silu_mul,
               w4a16_gemm)


def quantize_mlp_block(x: torch.Tensor, gamma: torch.Tensor, w_gu: torch.Tensor,
                       w_down: torch.Tensor, eps: float = 1e-5, bits: int = 4, group: int = 128,
                       n_grid: int = 20, keep_intermediates: bool = False,
                       gram: bool = False) -> dict:
    """One block.  x bf16 [M][d]; gamma f32 [d]; w_gu bf16 [2F][d] (gate rows,
    then up rows); w_down bf16 [d][F].  Returns the two searches' results, the
    folded gain and gate/up steps, and x_next (bf16 [M][d]).  gram: both
    searches take their losses in the Gram form (same losses to ~1e-6)."""
    F = w_gu.shape[0] // 2
    if w_gu.shape[0] != 2 * F or w_down.shape[1] != F or w_down.shape[0] != x.shape[1]:
        raise ValueError("w_gu must be [2F][d] and w_down [d][F]")
    out = {}
    search = search_scale_gram if gram else search_scale
    u = rmsnorm(x, gamma, eps)
    gu = search(u, w_gu, bits, group, n_grid)
    gamma_f = divide_rows(gamma, gu["best_s"])
    u_f = rmsnorm(x, gamma_f, eps)
    y_gu = w4a16_gemm(u_f, gu["qweight"], gu["scales"], gu["zeros"], bits, group, staged=True)
    h = silu_mul(y_gu)
    dn = search(h, w_down, bits, group, n_grid)
    scales_f = gu["scales"].clone()
    divide_rows(gu["scales"][F:], dn["best_s"], out=scales_f[F:])
    y_gu2 = w4a16_gemm(u_f, gu["qweight"], scales_f, gu["zeros"], bits, group, staged=True)
    h2 = silu_mul(y_gu2)
    y_down = w4a16_gemm(h2, dn["qweight"], dn["scales"], dn["zeros"], bits, group, staged=True)
    out.update(gate_up=gu, down=dn, gamma_folded=gamma_f, scales_gu_folded=scales_f,
               x_next=residual_add(x, y_down))
    if keep_intermediates:
        out.update(u=u, u_f=u_f, y_gu=y_gu, h=h, y_gu2=y_gu2, h2=h2, y_down=y_down)
    return out


def quantize_mlp_blocks(x: torch.Tensor, blocks, eps: float = 1e-5, bits: int = 4,
                        group: int = 128, n_grid: int = 20, gram: bool = False) -> list:
    """Blocks in order, each fed the previous block's deployed output.
    `blocks` holds (gamma, w_gu, w_down) per block."""
    results = []
    for gamma, w_gu, w_down in blocks:
        r = quantize_mlp_block(x, gamma, w_gu, w_down, eps, bits, group, n_grid, gram=gram)
        results.append(r)
        x = r["x_next"]
    return results
