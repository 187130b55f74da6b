"""GPU parity at the bench configuration's full size (Llama-2-7B fused QKV:
65536 calibration tokens, K = 4096 -> N = 12288, INT4, group 128, 20 grid
points), in the launch configuration bench.py times, plus every other
workload's layer shapes at a reduced token count.

At full size the oracle checks what it can compute: the statistics in full,
the candidate operands and the written weights on sampled rows (bit-exact),
the product on a sampled block; for the reductions, properties that hold at
any size (a candidate's squared error against its own product is exactly
zero; the difference operand is B - W exactly and its squared product equals
the error against the reference output; the search's losses are exactly the
standalone per-candidate squared errors; the chosen index is the first
minimum).
"""

import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_stats_amd as awq
import synth
from gpu_util import announce, gemm_close, require_gpu, to_dev_bf16, to_dev_f32, u32, ulp_distance_f32

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.fixture(scope="module")
def qkv(dev):
    announce("full-size inputs llama2_7b_qkv")
    x, w, spec = synth.make_layer("llama2_7b_qkv")
    return x, w, spec, to_dev_bf16(x, dev), to_dev_bf16(w, dev)


@pytest.fixture(scope="module")
def qkv_stats(qkv):
    x = qkv[0]
    return O.act_stats(x)


def sample_rows(n, k, seed):
    return np.sort(np.random.default_rng(seed).choice(n, size=k, replace=False))


def test_fullsize_stats(qkv, qkv_stats):
    announce("full-size act_stats")
    _, _, _, xd, _ = qkv
    got = awq.act_stats(xd).cpu().numpy().astype(np.float64)
    _, ref = qkv_stats
    assert (np.abs(got - ref) / np.maximum(ref, 1e-30)).max() <= 1e-6


def test_fullsize_candidates_and_operands(dev, qkv, qkv_stats):
    announce("full-size candidate scales + operands")
    x, w, spec, xd, wd = qkv
    a_gpu = awq.act_stats(xd)
    s_gpu, inv_gpu = awq.candidate_scales(a_gpu, spec.n_grid)
    s_ref, inv_ref = O.candidate_scales(qkv_stats[1], spec.n_grid)
    assert ulp_distance_f32(s_gpu.cpu().numpy(), s_ref).max() <= 1
    rows = sample_rows(spec.N, 48, 1)
    for i in (0, 9, 19):
        s_i, inv_i = s_gpu[i].cpu().numpy(), inv_gpu[i].cpu().numpy()
        b = awq.dequant_operand(wd, s_gpu[i], inv_gpu[i], 4).float().cpu().numpy()[rows]
        q, z, st = O.quantize(w[rows], s_i, 4, 128)
        assert np.array_equal(b.astype(np.float64), O.dequant_operand(q, z, st, 128, inv_i))
        qw, sc, ze = awq.quantize_pack(wd, s_gpu[i], 4)
        rq, rs, rz = O.pack(q, z, st)
        assert np.array_equal(u32(qw)[rows], rq)
        assert np.array_equal(sc.cpu().numpy()[rows], rs)
        assert np.array_equal(ze.cpu().numpy()[rows], rz)


def test_fullsize_products_sampled(dev, qkv):
    announce("full-size products, sampled block")
    x, w, spec, xd, wd = qkv
    ms = sample_rows(spec.M, 24, 2)
    ns = sample_rows(spec.N, 40, 3)
    y = awq.reference_gemm(xd, wd)
    gemm_close(y[ms][:, ns].cpu().numpy(), O.gemm(x[ms], O.bf16_bits_to_f64(w[ns])))
    del y
    s, inv = O.candidate_scales(O.act_stats(x[:4096])[1], 20)
    qw, sc, ze = awq.quantize_pack(wd, to_dev_f32(s[13], dev), 4)
    yq = awq.w4a16_gemm(xd, qw, sc, ze, 4, inv_s=to_dev_f32(inv[13], dev))
    q, z, st = O.quantize(w[ns], s[13], 4, 128)
    ref = O.gemm(x[ms], O.dequant_operand(q, z, st, 128, inv[13]))
    gemm_close(yq[ms][:, ns].cpu().numpy(), ref)


def test_fullsize_candidate_sse_properties(dev, qkv):
    announce("full-size candidate_sse properties")
    x, w, spec, xd, wd = qkv
    a = awq.act_stats(xd)
    s, inv = awq.candidate_scales(a, spec.n_grid)
    b = awq.dequant_operand(wd, s[6], inv[6], 4)
    y_b = awq.reference_gemm(xd, b)                      # the candidate's own product
    assert float(awq.candidate_sse(xd, b, y_b).item()) == 0.0
    y_ref = awq.reference_gemm(xd, wd)
    sse = float(awq.candidate_sse(xd, b, y_ref).item())
    direct = float(((y_b.double() - y_ref.double()) ** 2).sum().item())
    assert abs(sse - direct) <= 1e-9 * direct
    # the difference form measures the same error without y_ref
    d = awq.diff_operand(wd, s[6], inv[6], 4)
    assert torch.equal(d.float(), b.float() - wd.float())        # exact in bf16
    sq = float(awq.candidate_sse(xd, d, None).item())
    assert abs(sq - sse) <= 1e-5 * sse


def test_fullsize_search(dev, qkv, qkv_stats):
    """The bench's whole search at full size."""
    announce("full-size search_scale")
    x, w, spec, xd, wd = qkv
    out = awq.search_scale(xd, wd, 4, 128, spec.n_grid)
    losses = out["losses"].cpu().numpy()
    best = int(out["best_idx"].item())
    assert best == int(np.argmin(losses)) and np.isfinite(losses).all()
    a_gpu = out["mean_abs"]
    _, a_ref = qkv_stats
    assert (np.abs(a_gpu.cpu().numpy() - a_ref) / a_ref).max() <= 1e-6
    s, inv = awq.candidate_scales(a_gpu, spec.n_grid)
    MN = float(spec.M) * spec.N
    for i in range(spec.n_grid):
        d = awq.diff_operand(wd, s[i], inv[i], 4)
        assert float(awq.candidate_sse(xd, d, None).item()) / MN == losses[i], i
    s_ref, _ = O.candidate_scales(a_ref, spec.n_grid)
    best_s = out["best_s"].cpu().numpy()
    assert ulp_distance_f32(best_s, s_ref[best]).max() <= 1
    rows = sample_rows(spec.N, 48, 4)
    rq, rs, rz = O.pack(*O.quantize(w[rows], best_s, 4, 128))
    assert np.array_equal(u32(out["qweight"])[rows], rq)
    assert np.array_equal(out["scales"].cpu().numpy()[rows], rs)
    assert np.array_equal(out["zeros"].cpu().numpy()[rows], rz)
    # the outlier channels carry the largest scales (salient channels, 1%)
    cols, _ = synth.outlier_columns(spec)
    if best > 0:
        assert np.all(best_s[cols] > np.median(best_s))


def test_fullsize_search_gram(dev, qkv):
    """The Gram-form search at full size against the direct one: same
    statistics and scales, losses within 2e-5 relative, the same choice
    unless two losses tie to that precision."""
    announce("full-size search_scale_gram")
    x, w, spec, xd, wd = qkv
    a = awq.search_scale(xd, wd, 4, 128, spec.n_grid)
    g = awq.search_scale_gram(xd, wd, 4, 128, spec.n_grid)
    torch.cuda.synchronize()
    assert torch.equal(a["mean_abs"], g["mean_abs"])
    la, lg = a["losses"].cpu().numpy(), g["losses"].cpu().numpy()
    np.testing.assert_allclose(lg, la, rtol=2e-5, atol=0)
    ib, gb = int(a["best_idx"].item()), int(g["best_idx"].item())
    assert gb == int(np.argmin(lg))
    assert ib == gb or abs(la[ib] - la[gb]) <= 2e-5 * la[ib]
    if ib == gb:
        for k in ("best_s", "qweight", "scales", "zeros"):
            assert torch.equal(a[k], g[k]), k


@pytest.mark.parametrize("bits", [3, 4])
def test_fullsize_search_llama2_70b_down(dev, bits):
    """The largest layer of the workloads at full size (Llama-2-70B down
    projection: 16384 tokens x 28672 -> 8192): the direct and Gram-form
    searches agree (losses within 2e-5 relative, the same choice up to such
    ties), the statistics match the oracle's, and sampled rows of the final
    pack are bit-exact against the oracle given the chosen s."""
    announce("full-size search, Llama-2-70B down", bits)
    x, w, spec = synth.make_layer("llama2_70b_mlp", "down")
    xd, wd = to_dev_bf16(x, dev), to_dev_bf16(w, dev)
    a = awq.search_scale(xd, wd, bits, 128, spec.n_grid)
    g = awq.search_scale_gram(xd, wd, bits, 128, spec.n_grid)
    torch.cuda.synchronize()
    la, lg = a["losses"].cpu().numpy(), g["losses"].cpu().numpy()
    assert np.isfinite(la).all()
    np.testing.assert_allclose(lg, la, rtol=2e-5, atol=0)
    ib, gb = int(a["best_idx"].item()), int(g["best_idx"].item())
    assert ib == int(np.argmin(la))
    assert ib == gb or abs(la[ib] - la[gb]) <= 2e-5 * la[ib]
    a_ref = O.act_stats(x)[1]
    assert (np.abs(a["mean_abs"].cpu().numpy() - a_ref) / a_ref).max() <= 1e-6
    best_s = a["best_s"].cpu().numpy()
    rows = sample_rows(spec.N, 16, 9)
    rq, rs, rz = O.pack(*O.quantize(w[rows], best_s, bits, 128))
    assert np.array_equal(u32(a["qweight"])[rows], rq)
    assert np.array_equal(a["scales"].cpu().numpy()[rows], rs)
    assert np.array_equal(a["zeros"].cpu().numpy()[rows], rz)


@pytest.mark.parametrize("name", ["down", "gate_up"])
def test_fullsize_int3_dense_llama2_70b(dev, name):
    """The 70B-shaped INT3 layers at full size: dense words on sampled rows
    against the oracle, and the dense-INT3 decode contraction bit-identical to
    the 4-bit-container one at M = 1, 16 and 64 (at 64 tokens both layers take
    the column-split kernel with four token blocks), with a sampled oracle
    block."""
    announce("full-size dense INT3", name)
    spec = synth.layer_spec("llama2_70b_mlp", name)
    w = synth.make_weight(spec, 0)
    wd = to_dev_bf16(w, dev)
    s = np.exp(np.random.default_rng(2).uniform(-0.5, 0.5, spec.K)).astype(np.float32)
    qw3, sc, ze = awq.quantize_pack3(wd, to_dev_f32(s, dev))
    qw4, sc4, ze4 = awq.quantize_pack(wd, to_dev_f32(s, dev), 3)
    assert torch.equal(sc, sc4) and torch.equal(ze, ze4)
    rows = sample_rows(spec.N, 16, 5)
    q, z, st = O.quantize(w[rows], s, 3, 128)
    assert np.array_equal(u32(qw3)[rows], O.pack3(q))
    for M in (1, 16, 64):
        a = synth.decode_activations(spec.K, M, seed=M)
        ad = to_dev_bf16(a, dev)
        y3 = awq.decode_gemm3(ad, qw3, sc, ze)
        y4 = awq.decode_gemm(ad, qw4, sc4, ze4, 3)
        assert torch.equal(y3, y4), M
        cols = sample_rows(spec.N, 24, M)
        ref = O.decode_gemm3(a, u32(qw3)[cols], sc.cpu().numpy()[cols], ze.cpu().numpy()[cols], 128)
        gemm_close(y3.cpu().numpy()[:, cols], ref)


@pytest.mark.parametrize("name,bits,dense3", [("gate_up", 4, False), ("down", 3, True)])
def test_fullsize_compact_format_llama2_70b(dev, name, bits, dense3):
    """The compact deployment format on the 70B-shaped layers at full size:
    codes, binary16 steps and zero nibbles on sampled rows against the
    oracle, and the compact decode contraction on tiles bit-identical to the
    fp32-metadata one on the expanded metadata (M = 1, 16 and 64)."""
    announce("full-size compact format", name, bits, dense3)
    spec = synth.layer_spec("llama2_70b_mlp", name)
    w = synth.make_weight(spec, 0)
    wd = to_dev_bf16(w, dev)
    s = np.exp(np.random.default_rng(3).uniform(-0.5, 0.5, spec.K)).astype(np.float32)
    layout = awq.LAYOUT_INT3_DENSE if dense3 else awq.LAYOUT_NIBBLE
    qw, st, z4 = awq.quantize_pack16(wd, to_dev_f32(s, dev), bits, 128, layout)
    rows = sample_rows(spec.N, 16, 7)
    q, z, stp = O.quantize16(w[rows], s, bits, 128)
    sb, zb = O.pack_meta16(z, stp)
    words = O.pack3(q) if dense3 else O.pack(q, z, stp)[0]
    assert np.array_equal(u32(qw)[rows], words)
    assert np.array_equal(st.cpu().numpy().view(np.uint16)[rows], sb)
    assert np.array_equal(z4.cpu().numpy()[rows], zb)
    tiles = awq.decode_tiles(qw, spec.K, layout)
    sc, ze = awq.expand_meta16(st, z4)
    del wd, qw
    for M in (1, 16, 64):
        ad = to_dev_bf16(synth.decode_activations(spec.K, M, seed=M), dev)
        y16 = awq.decode_gemm_tiled16(ad, tiles, st, z4, layout)
        y32 = awq.decode_gemm_tiled(ad, tiles, sc, ze, layout)
        torch.cuda.synchronize()
        assert torch.equal(y16, y32), M


# Every other workload's layer shapes (real K, dtype and activation recipe),
# at 384 tokens and the first 256 output rows, against the oracle's search.
OTHER_LAYERS = [("llama2_7b_mlp", "gate_up", 4), ("llama2_7b_mlp", "down", 4),
                ("llama3_8b_block", "qkv", 4), ("llama3_8b_block", "o_proj", 4),
                ("llama3_8b_block", "gate_up", 4), ("llama3_8b_block", "down", 4),
                ("llama2_70b_mlp", "down", 3), ("llama2_70b_mlp", "down", 4),
                ("llama2_70b_mlp", "gate_up", 3)]


@pytest.mark.parametrize("workload,name,bits", OTHER_LAYERS,
                         ids=lambda v: str(v))
def test_workload_layers_reduced(dev, workload, name, bits):
    announce("search reduced", workload, name, bits)
    x, w, spec = synth.make_layer(workload, name, M=384, rows=256)
    out = awq.search_scale(to_dev_bf16(x, dev), to_dev_bf16(w, dev), bits, 128, spec.n_grid)
    ref = O.search(x, w, bits, 128, spec.n_grid)
    np.testing.assert_allclose(out["losses"].cpu().numpy(), ref["losses"], rtol=1e-4, atol=0)
    best = int(out["best_idx"].item())
    assert ref["losses"][best] <= (1 + 1e-4) * ref["losses"].min()
    best_s = out["best_s"].cpu().numpy().astype(np.float64)
    rq, rs, rz = O.pack(*O.quantize(w, best_s, bits, 128))
    assert np.array_equal(u32(out["qweight"]), rq)
    assert np.array_equal(out["scales"].cpu().numpy(), rs)
    assert np.array_equal(out["zeros"].cpu().numpy(), rz)
