"""The deployment contractions captured in a HIP graph (torch.cuda.CUDAGraph)
and replayed, as a serving loop runs them: every replay must equal the eager
call on the same inputs bit for bit, with the program's own eager work and
host synchronisations between replays, and with new activations copied into
the captured input between replays.  Covered: the decode contraction on
metadata tiles with a caller-owned workspace, the one that allocates nothing
(static scratch), both with and without a K split (the split adds a second
kernel that sums the partials), and the deployment module's many-token path
(the staged W4A16 product with its cached workspace)."""

import numpy as np
import pytest
import torch

import post_weight_quantization_stats_amd as awq
import synth
from gpu_util import announce, require_gpu, to_dev_bf16

pytestmark = pytest.mark.gpu

# (M, N, K): no split (K = 4096, 32 groups); K split in 2 (M = 8, 128
# groups); 8 waves per workgroup, no split (M = 1, 128 groups, 4096 columns).
SHAPES = [(1, 6144, 4096), (8, 1000, 16384), (1, 4096, 16384),
          # above 8 tokens with K splits; above 32 tokens on a large layer
          # (the column-split kernel, two K splits)
          (40, 4104, 14336), (48, 12296, 8320)]


def _compact_layer(N, K, seed, dev):
    rng = np.random.default_rng(seed)
    w = synth.to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    s = np.exp(rng.uniform(-0.3, 0.3, K)).astype(np.float32)
    qw, st16, z4 = awq.quantize_pack16(to_dev_bf16(w, dev), torch.from_numpy(s).to(dev), 4)
    qw32, sc, ze = awq.quantize_pack(to_dev_bf16(w, dev), torch.from_numpy(s).to(dev), 4)
    return awq.decode_tiles(qw, K), awq.decode_meta(st16, z4), awq.decode_tiles(qw32, K), sc, ze


def _activations(K, M, seed, dev):
    return to_dev_bf16(synth.decode_activations(K, M, seed=seed), dev)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: f"M{s[0]}_N{s[1]}_K{s[2]}")
def test_decode_replays_equal_eager(shape):
    dev = require_gpu()
    M, N, K = shape
    announce("decode graph replay", shape)
    tiles, meta, tiles32, sc, ze = _compact_layer(N, K, seed=N + K, dev=dev)
    need = awq.workspace_size(awq.OP_DECODE_GEMM, M, N, K)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    a_in = _activations(K, M, 1, dev)                 # the captured input buffer
    y_meta = torch.empty((M, N), dtype=torch.float32, device=dev)
    y_free = torch.empty((M, N), dtype=torch.float32, device=dev)

    def calls():
        awq.decode_gemm_tiled_meta(a_in, tiles, meta, N, out=y_meta, workspace=ws)
        awq.decode_gemm_tiled_noalloc(a_in, tiles32, sc, ze, out=y_free)

    calls()                                            # warm up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        calls()
    for rep in range(4):
        a_new = _activations(K, M, 10 + rep, dev)
        a_in.copy_(a_new)
        g.replay()
        torch.cuda.synchronize()
        got_meta, got_free = y_meta.clone(), y_free.clone()
        # eager work between replays, then the eager reference on the same input
        scratch = torch.randn((257, 263), device=dev) @ torch.randn((263, 129), device=dev)
        del scratch
        want_meta = awq.decode_gemm_tiled_meta(a_new, tiles, meta, N)
        want_free = awq.decode_gemm_tiled(a_new, tiles32, sc, ze)
        torch.cuda.synchronize()
        assert torch.equal(got_meta, want_meta), (shape, rep)
        assert torch.equal(got_free, want_free), (shape, rep)


def test_module_many_tokens_replays_equal_eager():
    dev = require_gpu()
    M, N, K = 300, 520, 1024
    announce("W4A16Linear graph replay", M, N, K)
    rng = np.random.default_rng(3)
    w = synth.to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    lin = awq.W4A16Linear.compact_from_weight(to_dev_bf16(w, dev), None)
    x_in = _activations(K, M, 2, dev)
    y = lin(x_in)                                      # warm up: caches the workspace
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        y_out = lin(x_in)
    for rep in range(3):
        x_new = _activations(K, M, 20 + rep, dev)
        x_in.copy_(x_new)
        g.replay()
        torch.cuda.synchronize()
        got = y_out.clone()
        want = lin(x_new)
        torch.cuda.synchronize()
        assert torch.equal(got, want), rep
    del y
