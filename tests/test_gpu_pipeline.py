"""The synthetic block pipeline on the GPU against the oracle: each op on its
own, then every step of two feed-forward blocks checked on the GPU's own
upstream tensors (so a step is judged on identical inputs), then the chained
blocks end to end.

Tolerances: bit-exact for the folds and the residual; RMSNorm and SiLU-multiply
bit-exact up to a rare last-bit flip (the fp64 sum's order, fp64 exp's last
ulp) checked as at most one bf16 step; products within the GEMM contract
(1e-3); losses within 1e-4 relative; the chosen candidate equal or tied within
1e-4."""

import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_stats_amd as awq
import synth
from gpu_util import announce, gemm_close, require_gpu, to_dev_bf16, to_dev_f32, u32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def bits(t):
    return t.cpu().view(torch.int16).numpy().view(np.uint16)


def close_bf16(got, ref, max_frac=1e-3):
    """Bit patterns equal except a rare flip of one bf16 step."""
    g, r = got.astype(np.int32), ref.astype(np.int32)
    diff = g != r
    assert diff.mean() <= max_frac, diff.mean()
    assert np.all(np.abs(g[diff] - r[diff]) <= 1)


def test_rmsnorm(dev):
    announce("rmsnorm")
    x, _ = synth.random_layer(77, 520, 8, seed=5, n_outlier=6, outlier_factor=50.0)
    gamma = np.random.default_rng(5).uniform(0.5, 1.5, 520).astype(np.float32)
    for eps in (1e-5, 0.0):
        u, r = awq.rmsnorm(to_dev_bf16(x, dev), to_dev_f32(gamma, dev), eps, return_r=True)
        ru, rr = O.rmsnorm(x, gamma, eps)
        assert np.array_equal(r.cpu().numpy(), rr)
        assert np.array_equal(bits(u), ru)


@pytest.mark.parametrize("K", [2048, 2056, 6152, 8192, 8200, 14336, 16384, 16392])
def test_rmsnorm_row_lengths(dev, K):
    # one to eight register pieces per thread, ragged last pieces, and rows past
    # the register-resident length (read twice)
    announce(f"rmsnorm K={K}")
    x, _ = synth.random_layer(5, K, 8, seed=K, n_outlier=4, outlier_factor=30.0)
    gamma = np.random.default_rng(K).uniform(0.5, 1.5, K).astype(np.float32)
    u, r = awq.rmsnorm(to_dev_bf16(x, dev), to_dev_f32(gamma, dev), 1e-6, return_r=True)
    ru, rr = O.rmsnorm(x, gamma, 1e-6)
    assert np.array_equal(r.cpu().numpy(), rr)
    assert np.array_equal(bits(u), ru)


def test_silu_mul_divide_residual(dev):
    announce("silu_mul, divide_rows, residual_add")
    rng = np.random.default_rng(6)
    y = (rng.standard_normal((300, 2 * 132)) * 5).astype(np.float32)
    y[0, :3] = [0.0, 90.0, -800.0]
    h = awq.silu_mul(to_dev_f32(y, dev))
    close_bf16(bits(h), O.silu_mul(y, 132))
    v = rng.uniform(1e-4, 1e-2, (40, 7)).astype(np.float32)
    s = rng.uniform(0.2, 5.0, 40).astype(np.float32)
    assert np.array_equal(awq.divide_rows(to_dev_f32(v, dev), to_dev_f32(s, dev)).cpu().numpy(),
                          O.divide_rows(v, s))
    x, _ = synth.random_layer(33, 264, 8, seed=6)
    yy = rng.standard_normal((33, 264)).astype(np.float32)
    assert np.array_equal(bits(awq.residual_add(to_dev_bf16(x, dev), to_dev_f32(yy, dev))),
                          O.residual_add(x, yy))


@pytest.mark.parametrize("M,F", [(1, 4), (3, 12), (1000, 1028), (257, 2048)])
def test_silu_mul_shapes(dev, M, F):
    # one quad, a few quads, several workgroups with a ragged last one, whole workgroups
    announce(f"silu_mul M={M} F={F}")
    y = (np.random.default_rng(M + F).standard_normal((M, 2 * F)) * 6).astype(np.float32)
    close_bf16(bits(awq.silu_mul(to_dev_f32(y, dev))), O.silu_mul(y, F))


def check_block_steps(dev, x, gamma, wgu, wd, n_grid, F, gram=False):
    """Run one block on the GPU and check each step against the oracle on the
    GPU's own inputs; returns the GPU's x_next (bit patterns)."""
    xd = to_dev_bf16(x, dev)
    r = awq.quantize_mlp_block(xd, to_dev_f32(gamma, dev), to_dev_bf16(wgu, dev),
                               to_dev_bf16(wd, dev), n_grid=n_grid, keep_intermediates=True,
                               gram=gram)
    torch.cuda.synchronize()
    u = bits(r["u"])
    close_bf16(u, O.rmsnorm(x, gamma, 1e-5)[0])
    gu = r["gate_up"]
    ref1 = O.search(u, wgu, 4, 128, n_grid)
    np.testing.assert_allclose(gu["losses"].cpu().numpy(), ref1["losses"], rtol=1e-4, atol=0)
    b1 = int(gu["best_idx"].item())
    assert ref1["losses"][b1] <= (1 + 1e-4) * ref1["losses"].min()
    s1 = gu["best_s"].cpu().numpy()
    rq, rs, rz = O.pack(*O.quantize(wgu, s1, 4, 128))
    assert np.array_equal(u32(gu["qweight"]), rq) and np.array_equal(gu["scales"].cpu().numpy(), rs)
    gamma_f = r["gamma_folded"].cpu().numpy()
    assert np.array_equal(gamma_f, O.divide_rows(gamma, s1))
    u_f = bits(r["u_f"])
    close_bf16(u_f, O.rmsnorm(x, gamma_f, 1e-5)[0])
    gemm_close(r["y_gu"].cpu().numpy(), O.deploy_gemm(u_f, rq, rs, rz, 128))
    h = bits(r["h"])
    close_bf16(h, O.silu_mul(r["y_gu"].cpu().numpy(), F))
    dn = r["down"]
    ref2 = O.search(h, wd, 4, 128, n_grid)
    np.testing.assert_allclose(dn["losses"].cpu().numpy(), ref2["losses"], rtol=1e-4, atol=0)
    b2 = int(dn["best_idx"].item())
    assert ref2["losses"][b2] <= (1 + 1e-4) * ref2["losses"].min()
    s2 = dn["best_s"].cpu().numpy()
    sf = r["scales_gu_folded"].cpu().numpy()
    assert np.array_equal(sf[:F], rs[:F]) and np.array_equal(sf[F:], O.divide_rows(rs[F:], s2))
    gemm_close(r["y_gu2"].cpu().numpy(), O.deploy_gemm(u_f, rq, sf, rz, 128))
    h2 = bits(r["h2"])
    close_bf16(h2, O.silu_mul(r["y_gu2"].cpu().numpy(), F))
    dq, ds, dz = O.pack(*O.quantize(wd, s2, 4, 128))
    gemm_close(r["y_down"].cpu().numpy(), O.deploy_gemm(h2, dq, ds, dz, 128))
    x_next = bits(r["x_next"])
    assert np.array_equal(x_next, O.residual_add(x, r["y_down"].cpu().numpy()))
    return x_next, (b1, b2)


def test_two_blocks_step_by_step(dev):
    M, d, F = 256, 256, 384
    x, blocks = synth.make_mlp_blocks(M, d, F, 2, seed=1)
    for b, (gamma, wgu, wd) in enumerate(blocks):
        announce("pipeline block", b)
        x, _ = check_block_steps(dev, x, gamma, wgu, wd, 20, F)


def test_two_blocks_step_by_step_gram_form(dev):
    """The same steps with both searches in the Gram form."""
    M, d, F = 512, 256, 384
    x, blocks = synth.make_mlp_blocks(M, d, F, 2, seed=3)
    for b, (gamma, wgu, wd) in enumerate(blocks):
        announce("pipeline block, Gram form", b)
        x, _ = check_block_steps(dev, x, gamma, wgu, wd, 20, F, gram=True)


def test_block_full_width_reduced_tokens(dev):
    """The Llama-2-7B feed-forward widths (4096 -> 2 x 11008 -> 4096) at 128
    tokens, every step checked."""
    announce("pipeline block, Llama-2-7B widths")
    x, blocks = synth.make_mlp_blocks(128, 4096, 11008, 1, seed=2)
    check_block_steps(dev, x, *blocks[0], 20, 11008)


def test_two_blocks_end_to_end(dev):
    """The chained blocks against the oracle's own chain: same choices (or
    ties) and outputs within a few bf16 steps."""
    announce("pipeline end to end")
    M, d, F = 192, 256, 384
    x0, blocks = synth.make_mlp_blocks(M, d, F, 2, seed=4)
    res = awq.quantize_mlp_blocks(to_dev_bf16(x0, dev),
                                  [(to_dev_f32(g, dev), to_dev_bf16(a, dev), to_dev_bf16(b, dev))
                                   for g, a, b in blocks], n_grid=20)
    torch.cuda.synchronize()
    x = x0
    for r, (g, a, b) in zip(res, blocks):
        ref = O.mlp_block(x, g, a, b, n_grid=20)
        for key in ("gate_up", "down"):
            i = int(r[key]["best_idx"].item())
            assert ref[key]["losses"][i] <= (1 + 1e-4) * ref[key]["losses"].min(), key
        x = ref["x_next"]
    got = O.bf16_bits_to_f64(bits(res[-1]["x_next"]))
    want = O.bf16_bits_to_f64(x)
    assert np.abs(got - want).max() <= 4 * 2.0 ** -8 * np.abs(want).max()
    assert (got != want).mean() <= 0.05
