"""Seeded synthetic layers for the AWQ scale search (inputs only).

This module draws the calibration activations X and weights W that both the
HIP library and the CPU oracle consume.  It holds none of the method's
arithmetic: it only draws random numbers, scales some columns, and rounds
fp32 draws to bf16 with torch's own conversion.

The pages' workloads are real calibration text run through real LLMs
("How it works" and "Implementation pitfalls" on robotsatlas.com's AWQ page:
128-512 representative samples).  No model weights or calibration dataset are
available here, so seeded layers with the same shapes stand in for them:
Gaussian weights, Gaussian (or Student-t) activations, and about 1% of the
input channels scaled up as outliers (the ~1% salient channels of
builderai.tools' "About" and aquanode.io's "The core idea").

Streams: numpy Generator(PCG64(SeedSequence([seed, workload_id, layer_id,
tensor_id]))).  Rows are drawn in order, so a token prefix of M' rows equals
the first M' rows of the full draw.
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

TENSOR_W, TENSOR_X, TENSOR_COLS, TENSOR_FACTORS, TENSOR_DECODE, TENSOR_GAIN = 0, 1, 2, 3, 4, 5
BLOCK_STREAM = 7          # workload id of the synthetic feed-forward blocks


@dataclass(frozen=True)
class LayerSpec:
    workload: str          # workload name
    workload_id: int
    name: str              # layer name inside the workload
    layer_id: int
    M: int                 # calibration tokens
    K: int                 # input channels
    N: int                 # output channels
    w_std: float
    x_kind: str            # "normal" | "student_t4" | "silu_gate_up"
    outlier_frac: float    # fraction of input channels scaled up
    outlier: tuple         # ("const", f) or ("loguniform", lo, hi) or ("none",)
    bits: tuple = (4,)
    group: int = 128
    n_grid: int = 20
    source: str | None = None   # for "silu_gate_up": the gate/up layer feeding it

    @property
    def n_outlier(self) -> int:
        return int(round(self.outlier_frac * self.K))

    def flops_per_gemm(self, M: int | None = None) -> float:
        return 2.0 * (self.M if M is None else M) * self.N * self.K


def _workloads():
    W = {}

    def add(workload, wid, layers):
        W[workload] = [LayerSpec(workload=workload, workload_id=wid, layer_id=i, **l)
                       for i, l in enumerate(layers)]

    # One 512x512 linear layer, 256 tokens, 5 outlier channels x20.
    add("single_linear_512", 0, [
        dict(name="linear", M=256, K=512, N=512, w_std=0.02, x_kind="normal",
             outlier_frac=5 / 512, outlier=("const", 20.0)),
    ])
    # Llama-2-7B-shaped fused QKV, 128 samples x 512 tokens.
    add("llama2_7b_qkv", 1, [
        dict(name="qkv", M=65536, K=4096, N=12288, w_std=0.02, x_kind="normal",
             outlier_frac=0.01, outlier=("loguniform", 10.0, 50.0)),
    ])
    # Llama-2-7B-shaped MLP; down_proj is fed SiLU(gate) * up.
    add("llama2_7b_mlp", 2, [
        dict(name="gate_up", M=65536, K=4096, N=2 * 11008, w_std=0.02,
             x_kind="student_t4", outlier_frac=0.0, outlier=("none",)),
        dict(name="down", M=65536, K=11008, N=4096, w_std=0.02, x_kind="silu_gate_up",
             outlier_frac=0.0, outlier=("none",), source="gate_up"),
    ])
    # Llama-3-8B-shaped decoder block (GQA qkv), 32768 tokens.
    add("llama3_8b_block", 3, [
        dict(name="qkv", M=32768, K=4096, N=6144, w_std=0.02, x_kind="normal",
             outlier_frac=0.01, outlier=("const", 30.0)),
        dict(name="o_proj", M=32768, K=4096, N=4096, w_std=0.02, x_kind="normal",
             outlier_frac=0.01, outlier=("const", 30.0)),
        dict(name="gate_up", M=32768, K=4096, N=2 * 14336, w_std=0.02, x_kind="normal",
             outlier_frac=0.01, outlier=("const", 30.0)),
        dict(name="down", M=32768, K=14336, N=4096, w_std=0.02, x_kind="silu_gate_up",
             outlier_frac=0.0, outlier=("none",), source="gate_up"),
    ])
    # Llama-2-70B-shaped MLP, 16384 tokens, INT3 and INT4.
    add("llama2_70b_mlp", 4, [
        dict(name="down", M=16384, K=28672, N=8192, w_std=0.015, x_kind="normal",
             outlier_frac=0.01, outlier=("const", 50.0), bits=(3, 4)),
        dict(name="gate_up", M=16384, K=8192, N=2 * 28672, w_std=0.015, x_kind="normal",
             outlier_frac=0.01, outlier=("const", 50.0), bits=(3, 4)),
    ])
    return W


WORKLOADS = _workloads()

# Token counts of the decode-shaped contraction run on the Llama-3-8B block.
DECODE_M = (1, 2, 4, 8, 16)


def layer_spec(workload: str, name: str | None = None) -> LayerSpec:
    layers = WORKLOADS[workload]
    if name is None:
        return layers[0]
    for l in layers:
        if l.name == name:
            return l
    raise KeyError(f"{workload} has no layer {name!r}")


def _rng(seed: int, *ids: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, *ids])))


def to_bf16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16) by torch's round-to-nearest-even cast."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x32, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32)


def make_weight(spec: LayerSpec, seed: int = 0, rows: int | None = None) -> np.ndarray:
    """W (bf16 bit patterns [N][K]); `rows` draws only the first rows, which
    equal the first rows of the full draw (the stream is row-major)."""
    rng = _rng(seed, spec.workload_id, spec.layer_id, TENSOR_W)
    n = spec.N if rows is None else min(rows, spec.N)
    w = rng.standard_normal((n, spec.K), dtype=np.float32)
    w *= np.float32(spec.w_std)
    return to_bf16_bits(w)


def outlier_columns(spec: LayerSpec, seed: int = 0):
    """(column indices, per-column factors) of the outlier channels."""
    n = spec.n_outlier
    if n == 0 or spec.outlier[0] == "none":
        return np.zeros(0, np.int64), np.zeros(0, np.float32)
    cols = np.sort(_rng(seed, spec.workload_id, spec.layer_id, TENSOR_COLS)
                   .choice(spec.K, size=n, replace=False))
    if spec.outlier[0] == "const":
        f = np.full(n, spec.outlier[1], dtype=np.float32)
    else:
        _, lo, hi = spec.outlier
        u = _rng(seed, spec.workload_id, spec.layer_id, TENSOR_FACTORS).uniform(
            np.log(lo), np.log(hi), size=n)
        f = np.exp(u).astype(np.float32)
    return cols, f


def _draw_x(spec: LayerSpec, M: int, seed: int) -> np.ndarray:
    rng = _rng(seed, spec.workload_id, spec.layer_id, TENSOR_X)
    if spec.x_kind == "normal":
        x = rng.standard_normal((M, spec.K), dtype=np.float32)
    elif spec.x_kind == "student_t4":
        x = rng.standard_t(4.0, size=(M, spec.K)).astype(np.float32)
    else:
        raise ValueError(spec.x_kind)
    cols, f = outlier_columns(spec, seed)
    if cols.size:
        x[:, cols] *= f[None, :]
    return x


def make_activations(spec: LayerSpec, M: int | None = None, seed: int = 0,
                     chunk_rows: int = 4096) -> np.ndarray:
    """Calibration activations X (bf16 bit patterns [M][K]); M defaults to the spec's."""
    M = spec.M if M is None else M
    if spec.x_kind != "silu_gate_up":
        return to_bf16_bits(_draw_x(spec, M, seed))
    # A down projection sees SiLU(gate) * up of the unquantized gate/up layer.
    import torch
    src = layer_spec(spec.workload, spec.source)
    xs = bf16_bits_to_f32(make_activations(src, M, seed))
    ws = bf16_bits_to_f32(make_weight(src, seed))
    F = src.N // 2
    assert F == spec.K, "gate/up width must equal the down projection's input"
    wg = torch.from_numpy(ws[:F]).double()
    wu = torch.from_numpy(ws[F:]).double()
    out = np.empty((M, F), dtype=np.uint16)
    for r0 in range(0, M, chunk_rows):
        xc = torch.from_numpy(xs[r0:r0 + chunk_rows]).double()
        g = xc @ wg.T
        u = xc @ wu.T
        h = (g * torch.sigmoid(g) * u).float().numpy()
        out[r0:r0 + chunk_rows] = to_bf16_bits(h)
    return out


def make_layer(workload: str, name: str | None = None, M: int | None = None, seed: int = 0,
               rows: int | None = None):
    spec = layer_spec(workload, name)
    return make_activations(spec, M, seed), make_weight(spec, seed, rows), spec


def decode_activations(K: int, M: int, seed: int = 0) -> np.ndarray:
    """Decode-shaped activations A [M][K] ~ N(0,1) in bf16."""
    rng = _rng(seed, 3, 100 + M, TENSOR_DECODE)
    return to_bf16_bits(rng.standard_normal((M, K), dtype=np.float32))


def random_layer(M: int, K: int, N: int, seed: int, w_std: float = 0.02,
                 n_outlier: int = 0, outlier_factor: float = 20.0):
    """Small arbitrary-shape layer for tests: (x_bits [M][K], w_bits [N][K])."""
    rng = _rng(seed, 99, M * 1_000_003 + K * 1009 + N, 0)
    w = rng.standard_normal((N, K), dtype=np.float32) * np.float32(w_std)
    x = rng.standard_normal((M, K), dtype=np.float32)
    if n_outlier:
        cols = rng.choice(K, size=n_outlier, replace=False)
        x[:, cols] *= np.float32(outlier_factor)
    return to_bf16_bits(x), to_bf16_bits(w)


def make_mlp_blocks(M: int, d: int, F: int, n_blocks: int, seed: int = 0, w_std: float = 0.02):
    """Synthetic Llama-shaped feed-forward blocks for the layer-by-layer
    pipeline: the first block's input x0 (bf16 [M][d], Student-t with nu = 4:
    heavy-tailed hidden states) and per block (gamma f32 [d] ~ U(0.5, 1.5),
    w_gu bf16 [2F][d] (gate rows, then up rows), w_down bf16 [d][F]),
    weights ~ N(0, w_std^2)."""
    x = _rng(seed, BLOCK_STREAM, 0, TENSOR_X).standard_t(4.0, size=(M, d)).astype(np.float32)
    blocks = []
    for b in range(n_blocks):
        gamma = _rng(seed, BLOCK_STREAM, 100 + b, TENSOR_GAIN).uniform(0.5, 1.5, d).astype(np.float32)
        wgu = _rng(seed, BLOCK_STREAM, 100 + b, TENSOR_W).standard_normal((2 * F, d), dtype=np.float32)
        wd = _rng(seed, BLOCK_STREAM, 200 + b, TENSOR_W).standard_normal((d, F), dtype=np.float32)
        blocks.append((gamma, to_bf16_bits(wgu * np.float32(w_std)), to_bf16_bits(wd * np.float32(w_std))))
    return to_bf16_bits(x), blocks
