"""The many-token W4A16 product through a staged operand (awq_w4a16_gemm_staged):
codes in 4-bit containers or dense INT3, dequantized once into the workspace
and contracted on the bf16 matrix cores (builderai AWQ page, "About": 4-bit
weights with 16-bit activations; sourcepulse AWQ project page, opening
paragraph: 3- and 4-bit weights).

Checked against the oracle's deploy product (elementwise, the GEMM
tolerance), beside the fused W4A16 kernel on the same codes (same operand,
contracted on the 32x32x16 matrix-core form instead of 16x16x32, so the two
agree to the contraction tolerance, not bit for bit); dense INT3 codes must
give exactly the result of the same codes in 4-bit containers.  The
deployment module runs dense INT3 layers at every token count.
"""

import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_stats_amd as awq
import synth
from gpu_util import announce, gemm_close, require_gpu, to_dev_bf16, to_dev_f32, u32

pytestmark = pytest.mark.gpu

# (M, K, N, seed): several 256x256 tiles with ragged M and N tails, one
# group, a single token, and a grid whose tile count is a multiple of 8.
SHAPES = [(300, 384, 200, 1), (513, 256, 520, 2), (1, 128, 64, 3), (77, 1024, 264, 4),
          (1024, 640, 768, 5), (1024, 1024, 512, 6)]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def ids(s):
    return f"M{s[0]}_K{s[1]}_N{s[2]}"


def packed(w, s, bits):
    q, z, st = O.quantize(w, s, bits, 128)
    qw, sc, ze = O.pack(q, z, st)
    return q, z, st, qw, sc, ze


@pytest.mark.parametrize("use_inv_s", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_staged_matches_fused_and_oracle(dev, shape, use_inv_s):
    announce("w4a16_gemm staged", ids(shape), use_inv_s)
    M, K, N, seed = shape
    x, w = synth.random_layer(M, K, N, seed=seed, n_outlier=4, outlier_factor=20.0)
    _, a = O.act_stats(x)
    s_ref, inv_ref = O.candidate_scales(a, 20)
    q, z, st, qw, sc, ze = packed(w, s_ref[9], 4)
    inv = inv_ref[9] if use_inv_s else None
    y_oracle = O.gemm(x, O.dequant_operand(q, z, st, 128, inv))
    y_ref32 = O.f32(O.gemm(x, O.bf16_bits_to_f64(w)))
    xd = to_dev_bf16(x, dev)
    qwd, scd, zed = torch.from_numpy(qw.view(np.int32)).to(dev), to_dev_f32(sc, dev), torch.from_numpy(ze).to(dev)
    invd = None if inv is None else to_dev_f32(inv, dev)
    yrd = to_dev_f32(y_ref32, dev)
    y_s, sse_s = awq.w4a16_gemm(xd, qwd, scd, zed, 4, 128, inv_s=invd, y_ref=yrd, staged=True)
    y_f, sse_f = awq.w4a16_gemm(xd, qwd, scd, zed, 4, 128, inv_s=invd, y_ref=yrd)
    torch.cuda.synchronize()
    gemm_close(y_s.cpu().numpy(), y_oracle)
    gemm_close(y_f.cpu().numpy(), y_oracle)
    sse_ref = float(np.sum((y_oracle - y_ref32) ** 2))
    assert float(sse_s.item()) == pytest.approx(sse_ref, rel=1e-4)
    assert float(sse_f.item()) == pytest.approx(sse_ref, rel=1e-4)
    # y only, and sse only, give the same numbers as the call with both
    assert torch.equal(awq.w4a16_gemm(xd, qwd, scd, zed, 4, 128, inv_s=invd, staged=True), y_s)
    _, sse_only = awq.w4a16_gemm(xd, qwd, scd, zed, 4, 128, inv_s=invd, y_ref=yrd,
                                 return_y=False, staged=True)
    assert float(sse_only.item()) == float(sse_s.item())


@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_staged_dense_int3(dev, shape):
    """Dense INT3 words give exactly the product of the same codes in 4-bit
    containers, and both match the oracle's product of the unpacked codes."""
    announce("w4a16_gemm staged dense INT3", ids(shape))
    M, K, N, seed = shape
    x, w = synth.random_layer(M, K, N, seed=seed + 50, n_outlier=4, outlier_factor=20.0)
    s = np.exp(np.random.default_rng(seed).uniform(-0.5, 0.5, K)).astype(np.float32)
    wd, sd, xd = to_dev_bf16(w, dev), to_dev_f32(s, dev), to_dev_bf16(x, dev)
    qw3, sc3, ze3 = awq.quantize_pack3(wd, sd)
    qw4, sc4, ze4 = awq.quantize_pack(wd, sd, 3)
    y3 = awq.w4a16_gemm(xd, qw3, sc3, ze3, 3, 128, layout=awq.LAYOUT_INT3_DENSE, staged=True)
    y4 = awq.w4a16_gemm(xd, qw4, sc4, ze4, 3, 128, staged=True)
    torch.cuda.synchronize()
    assert torch.equal(y3, y4)
    q3 = O.unpack3(u32(qw3))
    assert np.array_equal(q3, O.unpack(u32(qw4)))
    ref = O.gemm(x, O.dequant_operand(q3, ze3.cpu().numpy(), sc3.cpu().numpy(), 128))
    gemm_close(y3.cpu().numpy(), ref)


@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_fused_dense_int3(dev, shape):
    """The fused product on dense INT3 words (awq_w3a16_gemm) equals the fused
    product of the same codes in 4-bit containers bit for bit, with and
    without the inverse scale and the SSE epilogue, and matches the oracle's
    product of the unpacked codes."""
    announce("w3a16_gemm fused dense INT3", ids(shape))
    M, K, N, seed = shape
    x, w = synth.random_layer(M, K, N, seed=seed + 70, n_outlier=4, outlier_factor=20.0)
    rng = np.random.default_rng(seed + 7)
    s = np.exp(rng.uniform(-0.5, 0.5, K)).astype(np.float32)
    inv = (1.0 / s.astype(np.float64)).astype(np.float32)
    wd, sd, xd, invd = to_dev_bf16(w, dev), to_dev_f32(s, dev), to_dev_bf16(x, dev), to_dev_f32(inv, dev)
    qw3, sc3, ze3 = awq.quantize_pack3(wd, sd)
    qw4, sc4, ze4 = awq.quantize_pack(wd, sd, 3)
    y_ref = rng.standard_normal((M, N)).astype(np.float32) * 0.1
    yrd = to_dev_f32(y_ref, dev)
    y3, sse3 = awq.w4a16_gemm(xd, qw3, sc3, ze3, 3, 128, inv_s=invd, y_ref=yrd,
                              layout=awq.LAYOUT_INT3_DENSE)
    y4, sse4 = awq.w4a16_gemm(xd, qw4, sc4, ze4, 3, 128, inv_s=invd, y_ref=yrd)
    _, sse_only = awq.w4a16_gemm(xd, qw3, sc3, ze3, 3, 128, inv_s=invd, y_ref=yrd, return_y=False,
                                 layout=awq.LAYOUT_INT3_DENSE)
    y3n = awq.w4a16_gemm(xd, qw3, sc3, ze3, 3, 128, layout=awq.LAYOUT_INT3_DENSE)
    y4n = awq.w4a16_gemm(xd, qw4, sc4, ze4, 3, 128)
    torch.cuda.synchronize()
    assert torch.equal(y3, y4) and torch.equal(sse3, sse4) and torch.equal(sse_only, sse3)
    assert torch.equal(y3n, y4n)
    q3 = O.unpack3(u32(qw3))
    ref = O.gemm(x, O.dequant_operand(q3, ze3.cpu().numpy(), sc3.cpu().numpy(), 128, inv))
    gemm_close(y3.cpu().numpy(), ref)
    d = y3.cpu().numpy().astype(np.float64) - y_ref.astype(np.float64)
    assert abs(sse3.item() - float((d * d).sum())) <= 1e-6 * float((d * d).sum())


def test_staged_empty_and_errors(dev):
    announce("w4a16_gemm staged empty and errors")
    x = torch.zeros((0, 256), dtype=torch.bfloat16, device=dev)
    qw = torch.zeros((64, 32), dtype=torch.int32, device=dev)
    sc = torch.ones((64, 2), dtype=torch.float32, device=dev)
    ze = torch.zeros((64, 2), dtype=torch.uint8, device=dev)
    y = awq.w4a16_gemm(x, qw, sc, ze, staged=True)
    assert tuple(y.shape) == (0, 64)
    # refused by the wrapper before any call (the library refuses it too: ABI tests)
    with pytest.raises(ValueError, match="dense INT3 layout holds 3-bit codes"):
        awq.w4a16_gemm(torch.zeros((4, 256), dtype=torch.bfloat16, device=dev),
                       torch.zeros((64, 24), dtype=torch.int32, device=dev), sc, ze, 4,
                       layout=awq.LAYOUT_INT3_DENSE)


@pytest.mark.parametrize("M", [1, 16, 64, 65, 300])
def test_module_dense_int3_any_token_count(dev, M):
    """W4A16Linear on dense INT3 codes: the decode kernel up to 64 tokens
    (exact dequantized weight), the staged product above, both against the
    oracle; the same codes in 4-bit containers give the same outputs."""
    announce("W4A16Linear dense INT3", M)
    K, N = 1024, 328
    _, w = synth.random_layer(8, K, N, seed=71)
    s = np.exp(np.random.default_rng(5).uniform(-0.4, 0.4, K)).astype(np.float32)
    wd, sd = to_dev_bf16(w, dev), to_dev_f32(s, dev)
    qw3, sc, ze = awq.quantize_pack3(wd, sd)
    qw4, _, _ = awq.quantize_pack(wd, sd, 3)
    lin3 = awq.W4A16Linear(qw3, sc, ze, bits=3, layout=awq.LAYOUT_INT3_DENSE)
    lin4 = awq.W4A16Linear(qw4, sc, ze, bits=3)
    a = synth.decode_activations(K, M, seed=M)
    ad = to_dev_bf16(a, dev)
    y3, y4 = lin3(ad), lin4(ad)
    torch.cuda.synchronize()
    assert torch.equal(y3, y4)
    q3, scn, zen = u32(qw3), sc.cpu().numpy(), ze.cpu().numpy()
    if M <= 64:
        ref = O.decode_gemm3(a, q3, scn, zen, 128)
    else:
        ref = O.gemm(a, O.dequant_operand(O.unpack3(q3), zen, scn, 128))
    gemm_close(y3.cpu().numpy(), ref)
