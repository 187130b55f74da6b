"""GPU parity: every step of the HIP path against the CPU fp64 oracle on the
same seeded inputs, element by element.

Tolerances: codes, zeros, scales and packed words bit-exact given the
oracle's s; GEMM within 1e-3 relative (|d| <= 1e-3 max(|y|, rms Y) and
Frobenius); per-candidate losses within 1e-4 relative; the chosen candidate
equal, or (ties) within 1e-4 of the oracle's minimum; statistics within 1e-6
relative (fp64 sums of bf16 magnitudes are normally exact, so bit equality is
also counted).
"""

import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_stats_amd as awq
import synth
from gpu_util import (announce, gemm_close, require_gpu, to_dev_bf16, to_dev_f32, u32,
                      ulp_distance_f32)

pytestmark = pytest.mark.gpu

# (M, K, N, seed, n_outlier): several 256x256 tiles, ragged M / N tails,
# one group, a single token.
SHAPES = [
    (256, 512, 512, 0, 5),
    (300, 384, 200, 1, 4),
    (513, 256, 520, 2, 3),
    (1, 128, 64, 3, 1),
    (77, 1024, 264, 4, 10),
    (1024, 640, 768, 5, 6),
]


def layer(shape):
    M, K, N, seed, n_out = shape
    if (M, K, N) == (256, 512, 512):
        x, w, _ = synth.make_layer("single_linear_512")
        return x, w
    return synth.random_layer(M, K, N, seed=seed, n_outlier=n_out, outlier_factor=20.0)


def ids(s):
    return f"M{s[0]}_K{s[1]}_N{s[2]}"


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_act_stats(dev, shape):
    announce("act_stats", ids(shape))
    x, _ = layer(shape)
    got = awq.act_stats(to_dev_bf16(x, dev)).cpu().numpy().astype(np.float64)
    _, ref = O.act_stats(x)
    rel = np.abs(got - ref) / np.maximum(ref, 1e-30)
    assert rel.max() <= 1e-6
    assert np.mean(got == ref) > 0.99


def test_act_stats_long_and_ragged(dev):
    announce("act_stats long ragged")
    x, _ = synth.random_layer(5003, 1032, 8, seed=7, n_outlier=9)
    got = awq.act_stats(to_dev_bf16(x, dev)).cpu().numpy().astype(np.float64)
    _, ref = O.act_stats(x)
    assert (np.abs(got - ref) / ref).max() <= 1e-6


@pytest.mark.parametrize("K,n_grid", [(512, 20), (4096, 20), (1000, 7), (128, 1), (300, 64)])
def test_candidate_scales(dev, K, n_grid):
    announce("candidate_scales", K, n_grid)
    rng = np.random.default_rng(K + n_grid)
    a = O.f32(np.abs(rng.standard_normal(K)) * 0.8 + 0.01)
    a[rng.choice(K, size=max(1, K // 100), replace=False)] *= 30.0
    a[0] = 0.0   # a dead channel hits the floor
    a = O.f32(a)
    s, inv = awq.candidate_scales(to_dev_f32(a, dev), n_grid)
    s_ref, inv_ref = O.candidate_scales(a, n_grid)
    ds = ulp_distance_f32(s.cpu().numpy(), s_ref)
    di = ulp_distance_f32(inv.cpu().numpy(), inv_ref)
    # fp64 pow may differ from the host's in its last bit; that flips the
    # fp32 rounding with probability ~2^-29 per element.
    assert ds.max() <= 1 and di.max() <= 1
    assert np.mean(ds == 0) > 0.999
    assert np.all(s.cpu().numpy()[0] == 1.0)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_quantize_pack_bit_exact(dev, shape, bits):
    announce("quantize_pack", ids(shape), bits)
    x, w = layer(shape)
    _, a = O.act_stats(x)
    s_ref, _ = O.candidate_scales(a, 20)
    wd = to_dev_bf16(w, dev)
    for i in (None, 0, 6, 13, 19):
        s_row = None if i is None else s_ref[i]
        qw, sc, ze = awq.quantize_pack(wd, None if s_row is None else to_dev_f32(s_row, dev), bits)
        q, z, st = O.quantize(w, s_row, bits, 128)
        rq, rs, rz = O.pack(q, z, st)
        assert np.array_equal(u32(qw), rq), f"codes differ at candidate {i}"
        assert np.array_equal(sc.cpu().numpy(), rs), f"scales differ at candidate {i}"
        assert np.array_equal(ze.cpu().numpy(), rz), f"zeros differ at candidate {i}"


def test_quantize_special_groups(dev):
    announce("quantize special groups")
    N, K = 6, 256
    W = np.zeros((N, K), np.float32)
    W[1] = np.linspace(0.5, 3.0, K)                    # all positive
    W[2] = -np.linspace(0.5, 3.0, K)                   # all negative
    rng = np.random.default_rng(0)
    codes = rng.integers(0, 16, size=K)
    codes[0], codes[1], codes[128], codes[129] = 0, 15, 0, 15
    W[3] = (codes - 5) * 2.0 ** -6                      # on the 16-level grid
    W[4] = 1e-3 * rng.standard_normal(K)               # tiny values
    W[5, :128] = 7.0                                   # constant group
    w = synth.to_bf16_bits(W)
    for bits in (3, 4):
        qw, sc, ze = awq.quantize_pack(to_dev_bf16(w, dev), None, bits)
        rq, rs, rz = O.pack(*O.quantize(w, None, bits, 128))
        assert np.array_equal(u32(qw), rq)
        assert np.array_equal(sc.cpu().numpy(), rs)
        assert np.array_equal(ze.cpu().numpy(), rz)


def test_quantize_extreme_ranges(dev):
    """Groups whose range falls outside [2^-90, 2^100] take plain divides on
    the GPU; groups inside it with subnormal members take the fast quotient.
    Codes, steps and zeros must still match the oracle bit for bit."""
    announce("quantize extreme ranges")
    rng = np.random.default_rng(5)
    K = 1024
    rows = []
    for mag in (1e-38, 3e-33, 2.0 ** -91, 2.0 ** -89, 1e-20, 1.0, 1e25, 2.0 ** 99, 2.0 ** 101,
                1e35):
        rows.append(mag * rng.standard_normal(K))
    mixed = rng.standard_normal(K)
    mixed[::3] *= 1e-39                                # subnormal members
    rows.append(mixed)
    boundary = np.zeros(K)
    boundary[::128] = 15.0 * 2.0 ** -94                # range exactly at the cut
    boundary[1::128] = 2.0 ** -95
    rows.append(boundary)
    W = np.stack(rows).astype(np.float32)
    w = synth.to_bf16_bits(W)
    s = np.exp2(rng.uniform(-3, 3, K)).astype(np.float32)
    for bits in (3, 4):
        for sv in (None, s):
            qw, sc, ze = awq.quantize_pack(to_dev_bf16(w, dev),
                                           None if sv is None else to_dev_f32(sv, dev), bits)
            rq, rs, rz = O.pack(*O.quantize(w, sv, bits, 128))
            assert np.array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))
            assert np.array_equal(ze.cpu().numpy(), rz)
            assert np.array_equal(u32(qw), rq)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_dequant_operand_bit_exact(dev, shape, bits):
    """The search's per-candidate bf16 weight operand, bit for bit."""
    announce("dequant_operand", ids(shape), bits)
    x, w = layer(shape)
    _, a = O.act_stats(x)
    s_all, inv_all = O.candidate_scales(a, 20)
    wd = to_dev_bf16(w, dev)
    for i in (0, 7, 19):
        b = awq.dequant_operand(wd, to_dev_f32(s_all[i], dev), to_dev_f32(inv_all[i], dev), bits)
        q, z, st = O.quantize(w, s_all[i], bits, 128)
        ref = O.dequant_operand(q, z, st, 128, inv_all[i])
        got = b.float().cpu().numpy().astype(np.float64)
        assert np.array_equal(got, ref)
    b = awq.dequant_operand(wd, None, None, bits)
    q, z, st = O.quantize(w, None, bits, 128)
    assert np.array_equal(b.float().cpu().numpy().astype(np.float64),
                          O.dequant_operand(q, z, st, 128, None))


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_diff_operand_bit_exact(dev, shape, bits):
    """The search's per-candidate difference operand bf16(B - W), bit for bit."""
    announce("diff_operand", ids(shape), bits)
    x, w = layer(shape)
    _, a = O.act_stats(x)
    s_all, inv_all = O.candidate_scales(a, 20)
    wd = to_dev_bf16(w, dev)
    for i in (0, 7, 19):
        d = awq.diff_operand(wd, to_dev_f32(s_all[i], dev), to_dev_f32(inv_all[i], dev), bits)
        q, z, st = O.quantize(w, s_all[i], bits, 128)
        ref = O.diff_operand(w, O.dequant_operand(q, z, st, 128, inv_all[i]))
        assert np.array_equal(d.float().cpu().numpy().astype(np.float64), ref)
    d = awq.diff_operand(wd, None, None, bits)
    q, z, st = O.quantize(w, None, bits, 128)
    assert np.array_equal(d.float().cpu().numpy().astype(np.float64),
                          O.diff_operand(w, O.dequant_operand(q, z, st, 128, None)))


def test_operands_and_pack_many_rows(dev):
    """More rows than one pass of the operand modes' grid covers (65535 row
    slots of 4 rows), so their grid-stride loop runs, with a ragged tail of
    rows; the pack at the same shape.  Operands and codes bit for bit."""
    N, K = 4 * 65535 + 7, 256
    announce("quantize many rows", N, K)
    rng = np.random.default_rng(17)
    w = synth.to_bf16_bits((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    s = np.exp(rng.uniform(-0.5, 0.5, K)).astype(np.float32)
    inv = (1.0 / s.astype(np.float64)).astype(np.float32)
    wd = to_dev_bf16(w, dev)
    q, z, st = O.quantize(w, s, 4, 128)
    b_ref = O.dequant_operand(q, z, st, 128, inv)
    b = awq.dequant_operand(wd, to_dev_f32(s, dev), to_dev_f32(inv, dev), 4)
    assert np.array_equal(b.float().cpu().numpy().astype(np.float64), b_ref)
    d = awq.diff_operand(wd, to_dev_f32(s, dev), to_dev_f32(inv, dev), 4)
    assert np.array_equal(d.float().cpu().numpy().astype(np.float64), O.diff_operand(w, b_ref))
    qw, sc, ze = awq.quantize_pack(wd, to_dev_f32(s, dev), 4)
    rq, rs, rz = O.pack(q, z, st)
    assert np.array_equal(u32(qw), rq)
    assert np.array_equal(sc.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    assert np.array_equal(ze.cpu().numpy(), rz)


@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_candidate_sse_difference_form(dev, shape):
    """sum (X . D^T)^2 with the difference operand: the search's loss numerator."""
    announce("candidate_sse difference form", ids(shape))
    x, w = layer(shape)
    M, N = x.shape[0], w.shape[0]
    _, a = O.act_stats(x)
    s_all, inv_all = O.candidate_scales(a, 20)
    xd, wd = to_dev_bf16(x, dev), to_dev_bf16(w, dev)
    for i in (0, 11, 19):
        d = awq.diff_operand(wd, to_dev_f32(s_all[i], dev), to_dev_f32(inv_all[i], dev), 4)
        got = float(awq.candidate_sse(xd, d, None).item()) / (M * N)
        q, z, st = O.quantize(w, s_all[i], 4, 128)
        ref = O.output_mse(x, w, O.dequant_operand(q, z, st, 128, inv_all[i]))
        assert abs(got - ref) <= 1e-5 * ref


@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_candidate_sse(dev, shape):
    """The search's per-candidate loss numerator from the bf16 operand."""
    announce("candidate_sse", ids(shape))
    x, w = layer(shape)
    M, N = x.shape[0], w.shape[0]
    _, a = O.act_stats(x)
    s_all, inv_all = O.candidate_scales(a, 20)
    xd, wd = to_dev_bf16(x, dev), to_dev_bf16(w, dev)
    y_ref = awq.reference_gemm(xd, wd)
    for i in (0, 11):
        b = awq.dequant_operand(wd, to_dev_f32(s_all[i], dev), to_dev_f32(inv_all[i], dev), 4)
        got = float(awq.candidate_sse(xd, b, y_ref).item()) / (M * N)
        q, z, st = O.quantize(w, s_all[i], 4, 128)
        ref = O.output_mse(x, w, O.dequant_operand(q, z, st, 128, inv_all[i]))
        assert abs(got - ref) <= 1e-4 * ref


@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_reference_gemm(dev, shape):
    announce("reference_gemm", ids(shape))
    x, w = layer(shape)
    y = awq.reference_gemm(to_dev_bf16(x, dev), to_dev_bf16(w, dev)).cpu().numpy()
    gemm_close(y, O.gemm(x, O.bf16_bits_to_f64(w)))


@pytest.mark.parametrize("use_inv_s", [True, False])
@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_w4a16_gemm_and_sse(dev, shape, use_inv_s):
    announce("w4a16_gemm", ids(shape), use_inv_s)
    x, w = layer(shape)
    M, N = x.shape[0], w.shape[0]
    _, a = O.act_stats(x)
    s_ref, inv_ref = O.candidate_scales(a, 20)
    i = 11
    q, z, st = O.quantize(w, s_ref[i], 4, 128)
    qw, sc, ze = O.pack(q, z, st)
    inv = inv_ref[i] if use_inv_s else None
    B = O.dequant_operand(q, z, st, 128, inv)
    y_oracle = O.gemm(x, B)
    y_ref32 = O.f32(O.gemm(x, O.bf16_bits_to_f64(w)))
    xd = to_dev_bf16(x, dev)
    qwd = torch.from_numpy(qw.view(np.int32)).to(dev)
    scd = torch.from_numpy(sc).to(dev)
    zed = torch.from_numpy(ze).to(dev)
    invd = None if inv is None else to_dev_f32(inv, dev)
    y, sse = awq.w4a16_gemm(xd, qwd, scd, zed, 4, 128, inv_s=invd, y_ref=to_dev_f32(y_ref32, dev))
    gemm_close(y.cpu().numpy(), y_oracle)
    sse_ref = float(np.sum((y_oracle - y_ref32) ** 2))
    assert float(sse.item()) == pytest.approx(sse_ref, rel=1e-4)
    # y-only call gives the same numbers as the fused call
    y2 = awq.w4a16_gemm(xd, qwd, scd, zed, 4, 128, inv_s=invd)
    assert torch.equal(y, y2)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_search_scale(dev, shape, bits):
    announce("search_scale", ids(shape), bits)
    x, w = layer(shape)
    n_grid = 20
    out = awq.search_scale(to_dev_bf16(x, dev), to_dev_bf16(w, dev), bits, 128, n_grid)
    torch.cuda.synchronize()
    ref = O.search(x, w, bits, 128, n_grid)
    mean_abs = out["mean_abs"].cpu().numpy().astype(np.float64)
    assert (np.abs(mean_abs - ref["mean_abs"]) / np.maximum(ref["mean_abs"], 1e-30)).max() <= 1e-6
    losses = out["losses"].cpu().numpy()
    np.testing.assert_allclose(losses, ref["losses"], rtol=1e-4, atol=0)
    best = int(out["best_idx"].item())
    assert 0 <= best < n_grid
    assert ref["losses"][best] <= (1 + 1e-4) * ref["losses"].min()
    best_s = out["best_s"].cpu().numpy().astype(np.float64)
    assert ulp_distance_f32(best_s, ref["s"][best]).max() <= 1
    # the written weights are the quantization of W . diag(best_s), bit-exact
    rq, rs, rz = O.pack(*O.quantize(w, best_s, bits, 128))
    assert np.array_equal(u32(out["qweight"]), rq)
    assert np.array_equal(out["scales"].cpu().numpy(), rs)
    assert np.array_equal(out["zeros"].cpu().numpy(), rz)


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_search_scale_gram(dev, shape, bits):
    """Gram-form losses against the oracle's (fp64, Gram form), 1e-4 relative."""
    announce("search_scale_gram", ids(shape), bits)
    x, w = layer(shape)
    n_grid = 20
    out = awq.search_scale_gram(to_dev_bf16(x, dev), to_dev_bf16(w, dev), bits, 128, n_grid)
    torch.cuda.synchronize()
    ref = O.search(x, w, bits, 128, n_grid, loss_form="gram")
    losses = out["losses"].cpu().numpy()
    np.testing.assert_allclose(losses, ref["losses"], rtol=1e-4, atol=0)
    best = int(out["best_idx"].item())
    assert ref["losses"][best] <= (1 + 1e-4) * ref["losses"].min()
    best_s = out["best_s"].cpu().numpy().astype(np.float64)
    assert ulp_distance_f32(best_s, ref["s"][best]).max() <= 1
    rq, rs, rz = O.pack(*O.quantize(w, best_s, bits, 128))
    assert np.array_equal(u32(out["qweight"]), rq)
    assert np.array_equal(out["scales"].cpu().numpy(), rs)
    assert np.array_equal(out["zeros"].cpu().numpy(), rz)


def test_search_gram_matches_direct(dev):
    """Both forms on one layer: same statistics, losses within 2e-5 relative."""
    announce("search gram vs direct")
    x, w = layer(SHAPES[5])
    xd, wd = to_dev_bf16(x, dev), to_dev_bf16(w, dev)
    a = awq.search_scale(xd, wd)
    g = awq.search_scale_gram(xd, wd)
    torch.cuda.synchronize()
    assert torch.equal(a["mean_abs"], g["mean_abs"])
    la, lg = a["losses"].cpu().numpy(), g["losses"].cpu().numpy()
    np.testing.assert_allclose(lg, la, rtol=2e-5, atol=0)
    ib, gb = int(a["best_idx"].item()), int(g["best_idx"].item())
    assert ib == gb or abs(la[ib] - la[gb]) <= 2e-5 * la[ib]


def test_search_is_bit_reproducible(dev):
    announce("search determinism")
    x, w = layer(SHAPES[2])
    xd, wd = to_dev_bf16(x, dev), to_dev_bf16(w, dev)
    a = awq.search_scale(xd, wd)
    b = awq.search_scale(xd, wd)
    torch.cuda.synchronize()
    for k in a:
        assert torch.equal(a[k], b[k]), k


def test_searches_on_two_streams_at_once(dev):
    """Two searches in flight on two streams (each with its own outputs and
    workspace) give the same results as one after the other: the library
    keeps no mutable state between calls."""
    announce("search on two streams")
    layers = [layer(SHAPES[1]), layer(SHAPES[4])]
    dl = [(to_dev_bf16(x, dev), to_dev_bf16(w, dev)) for x, w in layers]
    seq = [awq.search_scale(xd, wd) for xd, wd in dl]
    torch.cuda.synchronize()
    streams = [torch.cuda.Stream(dev), torch.cuda.Stream(dev)]
    par = [None, None]
    for rep in range(3):
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                par[i] = awq.search_scale(*dl[i])
        torch.cuda.synchronize()
        for a, b in zip(seq, par):
            for k in a:
                assert torch.equal(a[k], b[k]), (rep, k)


def test_gemm_empty_and_degenerate(dev):
    announce("gemm empty")
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device=dev)
    qw = torch.zeros((8, 16), dtype=torch.int32, device=dev)
    sc = torch.ones((8, 1), dtype=torch.float32, device=dev)
    ze = torch.zeros((8, 1), dtype=torch.uint8, device=dev)
    yref = torch.zeros((0, 8), dtype=torch.float32, device=dev)
    y, sse = awq.w4a16_gemm(x, qw, sc, ze, y_ref=yref)
    assert y.shape == (0, 8) and float(sse.item()) == 0.0
    w0 = torch.zeros((0, 128), dtype=torch.bfloat16, device=dev)
    q0, s0, z0 = awq.quantize_pack(w0)
    assert q0.shape == (0, 16)


# ---------------------------------------------------------------- decode GEMM

def random_packed(N, K, bits, seed):
    """Seeded packed weights: random code words (codes < 2^bits in 4-bit
    containers), positive steps, zeros in [0, qmax]."""
    rng = np.random.default_rng(seed)
    qw = rng.integers(0, 2 ** 32, size=(N, K // 8), dtype=np.uint64).astype(np.uint32)
    if bits == 3:
        qw &= np.uint32(0x77777777)
    G = K // 128
    sc = (0.02 / 7.5 * rng.uniform(0.5, 1.5, size=(N, G))).astype(np.float32)
    ze = rng.integers(0, 2 ** bits, size=(N, G)).astype(np.uint8)
    return qw, sc, ze


def run_decode(dev, M, N, K, bits, seed):
    a = synth.decode_activations(K, M, seed=seed)
    qw, sc, ze = random_packed(N, K, bits, seed)
    y = awq.decode_gemm(to_dev_bf16(a, dev), torch.from_numpy(qw.view(np.int32)).to(dev),
                        to_dev_f32(sc, dev), torch.from_numpy(ze).to(dev), bits)
    return y.cpu().numpy(), (a, qw, sc, ze)


# (M, N, K): K within one workgroup (waves with one, several or no groups)
# and split across workgroups (K > 8192), ragged N, one group, odd token
# counts, narrow and wide layers (16-, 32- and 64-column workgroups), and
# more than 32 tokens split over several token groups of one or two 16-token
# blocks (the last group ragged at M = 33 and 45); up to 6 tokens, 65 to 128
# groups on one workgroup of 8 waves (the last wave's range ragged at 65),
# and more on several such workgroups.
DECODE_SHAPES = [(1, 64, 128), (2, 200, 256), (3, 1000, 1024), (4, 4096, 4096), (8, 520, 2048),
                 (13, 4104, 384), (16, 6144, 4096), (16, 40960, 512), (5, 16, 1152),
                 (2, 520, 16512), (1, 72, 32768), (16, 8200, 16384),
                 (17, 1000, 1024), (32, 6144, 4096), (48, 520, 16512), (64, 4096, 4096),
                 (64, 20000, 640), (33, 40, 128), (45, 8200, 256),
                 (1, 4096, 14336), (3, 200, 16384), (2, 40, 8320), (4, 16392, 8320),
                 (6, 40, 8320), (5, 520, 16512), (7, 40, 8320),
                 # above 8 tokens: 64 columns and two token blocks per
                 # workgroup with K splits, a ragged last column block
                 (40, 4104, 14336), (24, 4104, 11008),
                 # above 32 tokens on at least 96 Mi weights: the column-split
                 # kernel, with K splits and ragged column and token blocks,
                 # two token blocks and four (codes beyond 96 MiB)
                 (64, 12296, 8320), (36, 24584, 4224), (33, 8200, 24704)]


@pytest.mark.parametrize("bits", [4, 3])
@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: f"M{s[0]}_N{s[1]}_K{s[2]}")
def test_decode_gemm(dev, shape, bits):
    M, N, K = shape
    announce("decode_gemm", shape, bits)
    y, (a, qw, sc, ze) = run_decode(dev, M, N, K, bits, seed=M * 7 + bits)
    ref = O.decode_gemm(a, qw, sc, ze, 128)
    _, fro = gemm_close(y, ref)
    assert fro <= 1e-5     # fp32 sums of exact products: far inside the contract


@pytest.mark.parametrize("name", ["qkv", "o_proj", "gate_up", "down"])
def test_decode_gemm_llama3_block_shapes(dev, name):
    """The Llama-3-8B block's layers at their full sizes, M = 1, 16 and 64
    (gate_up at 64 tokens takes the column-split kernel)."""
    spec = synth.layer_spec("llama3_8b_block", name)
    for M in (1, 16, 64):
        announce("decode_gemm full size", name, M)
        y, (a, qw, sc, ze) = run_decode(dev, M, spec.N, spec.K, 4, seed=M)
        gemm_close(y, O.decode_gemm(a, qw, sc, ze, 128))


def test_decode_gemm_is_bit_reproducible(dev):
    announce("decode_gemm determinism")
    y1, _ = run_decode(dev, 16, 4096, 14336, 4, seed=9)
    y2, _ = run_decode(dev, 16, 4096, 14336, 4, seed=9)
    assert np.array_equal(y1.view(np.uint32), y2.view(np.uint32))


def test_decode_gemm_workspace_reuse(dev):
    """One workspace shared by a sequence of calls (different shapes and
    split counts, repeated) gives results bit-identical to fresh workspaces:
    nothing a call leaves in it changes a later call."""
    announce("decode_gemm workspace reuse")
    shapes = [(1, 6144, 4096), (2, 520, 33024), (3, 1000, 1024), (1, 72, 32768), (8, 520, 2048)]
    need = max(awq.workspace_size(awq.OP_DECODE_GEMM, M, N, K) for M, N, K in shapes)
    assert need > 0
    shared = torch.full((need,), 0x7F, dtype=torch.uint8, device=dev)
    for rep in range(2):
        for i, (M, N, K) in enumerate(shapes):
            a = synth.decode_activations(K, M, seed=i)
            qw, sc, ze = random_packed(N, K, 4, seed=i)
            args = (to_dev_bf16(a, dev), torch.from_numpy(qw.view(np.int32)).to(dev),
                    to_dev_f32(sc, dev), torch.from_numpy(ze).to(dev), 4)
            y_shared = awq.decode_gemm(*args, workspace=shared).cpu().numpy()
            y_fresh = awq.decode_gemm(*args).cpu().numpy()
            assert np.array_equal(y_shared.view(np.uint32), y_fresh.view(np.uint32)), (rep, i)


@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_quantize_pack3_bit_exact(dev, shape):
    """Dense INT3 words, steps and zeros, bit for bit, given the oracle's s."""
    announce("quantize_pack3", ids(shape))
    x, w = layer(shape)
    _, a = O.act_stats(x)
    s_all, _ = O.candidate_scales(a, 20)
    wd = to_dev_bf16(w, dev)
    for s in (None, s_all[13]):
        qw, sc, ze = awq.quantize_pack3(wd, None if s is None else to_dev_f32(s, dev))
        q, z, st = O.quantize(w, s, 3, 128)
        _, rs, rz = O.pack(q, z, st)
        assert np.array_equal(u32(qw), O.pack3(q))
        assert np.array_equal(sc.cpu().numpy(), rs)
        assert np.array_equal(ze.cpu().numpy(), rz)


INT3_DECODE_SHAPES = [(1, 64, 128), (3, 1000, 1024), (16, 6144, 4096), (16, 40960, 512),
                      (2, 520, 16512), (64, 4096, 4096), (33, 40, 128), (1, 72, 32768),
                      (45, 8200, 256), (2, 40, 8320), (64, 12296, 8320)]


@pytest.mark.parametrize("shape", INT3_DECODE_SHAPES, ids=lambda s: f"M{s[0]}_N{s[1]}_K{s[2]}")
def test_decode_gemm3(dev, shape):
    """The dense-INT3 contraction: bit-identical to the 4-bit-container one on
    the same codes, and against the oracle's product from the dense words."""
    M, N, K = shape
    announce("decode_gemm3", shape)
    a = synth.decode_activations(K, M, seed=M + 3)
    qw4, sc, ze = random_packed(N, K, 3, seed=M + 5)
    q = O.unpack(qw4)
    qw3 = O.pack3(q)
    ad, sd, zd = to_dev_bf16(a, dev), to_dev_f32(sc, dev), torch.from_numpy(ze).to(dev)
    y3 = awq.decode_gemm3(ad, torch.from_numpy(qw3.view(np.int32)).to(dev), sd, zd)
    y4 = awq.decode_gemm(ad, torch.from_numpy(qw4.view(np.int32)).to(dev), sd, zd, 3)
    torch.cuda.synchronize()
    assert torch.equal(y3, y4)
    _, fro = gemm_close(y3.cpu().numpy(), O.decode_gemm3(a, qw3, sc, ze, 128))
    assert fro <= 1e-5


@pytest.mark.parametrize("dense3", [False, True], ids=["nibble", "int3dense"])
def test_decode_tiles_bit_exact(dev, dense3):
    """Decode tiles against the oracle's layout (ragged N, several groups)."""
    announce("decode_tiles", dense3)
    for N, K in ((37, 384), (520, 2048), (16, 128)):
        qw4, _, _ = random_packed(N, K, 3 if dense3 else 4, seed=N)
        qw = O.pack3(O.unpack(qw4)) if dense3 else qw4
        t = awq.decode_tiles(torch.from_numpy(qw.view(np.int32)).to(dev), K,
                             awq.LAYOUT_INT3_DENSE if dense3 else awq.LAYOUT_NIBBLE)
        got = t.cpu().numpy().view(np.uint8)
        assert np.array_equal(got, O.decode_tiles(qw, K, dense3)), (N, K)


@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: f"M{s[0]}_N{s[1]}_K{s[2]}")
def test_decode_gemm_tiled_matches_row_major(dev, shape):
    """The tiled contraction is bit-identical to the row-major one, for the
    4-bit containers and for dense INT3."""
    M, N, K = shape
    announce("decode_gemm_tiled", shape)
    a = synth.decode_activations(K, M, seed=M + 9)
    qw4, sc, ze = random_packed(N, K, 3, seed=M + 11)
    qw3 = O.pack3(O.unpack(qw4))
    ad, sd, zd = to_dev_bf16(a, dev), to_dev_f32(sc, dev), torch.from_numpy(ze).to(dev)
    q4d = torch.from_numpy(qw4.view(np.int32)).to(dev)
    q3d = torch.from_numpy(qw3.view(np.int32)).to(dev)
    y4 = awq.decode_gemm(ad, q4d, sd, zd, 3)
    y4t = awq.decode_gemm_tiled(ad, awq.decode_tiles(q4d, K), sd, zd, awq.LAYOUT_NIBBLE)
    y3t = awq.decode_gemm_tiled(ad, awq.decode_tiles(q3d, K, awq.LAYOUT_INT3_DENSE), sd, zd,
                                awq.LAYOUT_INT3_DENSE)
    torch.cuda.synchronize()
    assert torch.equal(y4t, y4)
    assert torch.equal(y3t, y4)


def test_decode_gemm_matches_search_operand_when_exact(dev):
    """Power-of-two steps make (q - z) * step exact in bf16: the decode kernel
    and the general W4A16 kernel then compute the same products."""
    announce("decode vs general w4a16")
    M, N, K = 16, 512, 1024
    a = synth.decode_activations(K, M, seed=4)
    qw, _, ze = random_packed(N, K, 4, seed=4)
    rng = np.random.default_rng(4)
    sc = np.exp2(rng.integers(-10, -4, size=(N, K // 128))).astype(np.float32)
    ad = to_dev_bf16(a, dev)
    qd = torch.from_numpy(qw.view(np.int32)).to(dev)
    sd, zd = to_dev_f32(sc, dev), torch.from_numpy(ze).to(dev)
    y_dec = awq.decode_gemm(ad, qd, sd, zd, 4).cpu().numpy()
    y_gen = awq.w4a16_gemm(ad, qd, sd, zd, 4).cpu().numpy()
    ref = O.decode_gemm(a, qw, sc, ze, 128)
    gemm_close(y_dec, ref)
    gemm_close(y_gen, ref)
