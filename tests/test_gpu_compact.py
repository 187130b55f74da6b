"""The compact deployment format (binary16 steps, two 4-bit zeros per byte)
on the GPU against the oracle: the final pack bit for bit, the metadata
expansion bit for bit, the metadata tiles bit for bit, and the decode
contraction on decode tiles reading the compact metadata or its tiles
(bit-identical to each other and to the fp32-metadata kernel on the expanded
metadata, and within the contraction tolerance of the oracle)."""

import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_stats_amd as awq
import synth
from gpu_util import announce, gemm_close, require_gpu, to_dev_bf16, to_dev_f32, u32

pytestmark = pytest.mark.gpu

# (M, K, N, seed, n_outlier): several tiles, ragged N, odd group counts
# (K = 384, 640: G = 3, 5), one group.
SHAPES = [(300, 384, 200, 1, 4), (1, 128, 64, 3, 1), (77, 1024, 264, 4, 10),
          (64, 640, 768, 5, 6), (32, 4096, 520, 6, 8)]


def ids(s):
    return f"K{s[1]}_N{s[2]}"


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def oracle_compact(w, s, bits, dense3):
    q, z, st = O.quantize16(w, s, bits, 128)
    sb, zb = O.pack_meta16(z, st)
    words = O.pack3(q) if dense3 else O.pack(q, z, st)[0]
    return words, sb, zb


def check_pack16(dev, w, s, bits, dense3):
    layout = awq.LAYOUT_INT3_DENSE if dense3 else awq.LAYOUT_NIBBLE
    qw, st, ze = awq.quantize_pack16(to_dev_bf16(w, dev), None if s is None else to_dev_f32(s, dev),
                                     bits, 128, layout)
    rq, rs, rz = oracle_compact(w, s, bits, dense3)
    assert np.array_equal(u32(qw), rq), "codes differ"
    assert np.array_equal(st.cpu().numpy().view(np.uint16), rs), "binary16 steps differ"
    assert np.array_equal(ze.cpu().numpy(), rz), "zero bytes differ"


@pytest.mark.parametrize("variant", [(4, False), (3, False), (3, True)],
                         ids=["int4", "int3_nibble", "int3_dense"])
@pytest.mark.parametrize("shape", SHAPES, ids=ids)
def test_quantize_pack16_bit_exact(dev, shape, variant):
    bits, dense3 = variant
    announce("quantize_pack16", ids(shape), bits, dense3)
    M, K, N, seed, n_out = shape
    x, w = synth.random_layer(M, K, N, seed=seed, n_outlier=n_out, outlier_factor=20.0)
    s_all, _ = O.candidate_scales(O.act_stats(x)[1], 20)
    for s in (None, s_all[7], s_all[19]):
        check_pack16(dev, w, s, bits, dense3)


def test_quantize_pack16_clamped_subnormal_and_extreme_steps(dev):
    """Steps below 2^-24 (clamped), binary16-subnormal steps, steps beyond
    65504 (clamped, codes saturate), zero and constant groups, and the fp32
    path's extreme ranges (plain divides outside [2^-90, 2^100])."""
    announce("quantize_pack16 extreme steps")
    rng = np.random.default_rng(8)
    K = 640
    rows = [1e-9 * rng.standard_normal(K), 1e-5 * rng.standard_normal(K),
            3e-4 * rng.standard_normal(K), 1e6 * rng.standard_normal(K),
            np.zeros(K), np.full(K, 7.0)]
    for mag in (1e-38, 2.0 ** -91, 2.0 ** -89, 1e-20, 1.0, 1e25, 2.0 ** 101, 1e35):
        rows.append(mag * rng.standard_normal(K))
    edge = np.zeros(K)
    edge[0::256] = 15.0 * 65504.0                      # groups 0, 2, 4: step near the limit
    edge[128::256] = 15.0 * 2.0 ** -24 * 0.75          # groups 1, 3: step just under 2^-24
    rows.append(edge)
    w = synth.to_bf16_bits(np.stack(rows).astype(np.float32))
    s = np.exp2(rng.uniform(-3, 3, K)).astype(np.float32)
    for bits, dense3 in ((4, False), (3, False), (3, True)):
        for sv in (None, s):
            check_pack16(dev, w, sv, bits, dense3)


def random_compact_meta(N, G, bits, seed):
    """binary16 steps around 0.02/7.5 and random zeros in [0, qmax], as the
    stored arrays (high nibble past the last group 0)."""
    rng = np.random.default_rng(seed)
    st = (0.02 / 7.5 * rng.uniform(0.5, 1.5, size=(N, G))).astype(np.float16)
    z = rng.integers(0, 2 ** bits, size=(N, G + (G & 1)))
    z[:, G:] = 0
    zb = (z[:, 0::2] | (z[:, 1::2] << 4)).astype(np.uint8)
    return st.view(np.uint16), zb


def test_expand_meta16_exact(dev):
    announce("expand_meta16")
    rng = np.random.default_rng(9)
    for N, G in ((7, 1), (33, 5), (520, 32)):
        bits = rng.integers(0, 0x7C00, size=(N, G)).astype(np.uint16)   # finite, non-negative
        zb = rng.integers(0, 256, size=(N, (G + 1) // 2)).astype(np.uint8)
        if G & 1:
            zb[:, -1] &= 0x0F
        sc, ze = awq.expand_meta16(torch.from_numpy(bits.view(np.float16)).to(dev),
                                   torch.from_numpy(zb).to(dev))
        st_ref, z_ref = O.unpack_meta16(bits, zb, G)
        assert np.array_equal(sc.cpu().numpy().astype(np.float64), st_ref)
        assert np.array_equal(ze.cpu().numpy().astype(np.int64), z_ref)


DECODE_SHAPES = [(1, 64, 128), (2, 200, 384), (3, 1000, 1152), (16, 6144, 4096),
                 (16, 40960, 512), (2, 520, 16512), (1, 72, 32768), (33, 40, 640),
                 (64, 4096, 4096), (48, 520, 16512), (45, 8200, 256),
                 (3, 200, 16384), (4, 4096, 4096), (5, 200, 384), (6, 1000, 1152),
                 (7, 520, 16512), (8, 6144, 4096), (8, 72, 32768), (64, 12296, 8320)]


@pytest.mark.parametrize("dense3", [False, True], ids=["nibble", "int3dense"])
@pytest.mark.parametrize("shape", DECODE_SHAPES, ids=lambda s: f"M{s[0]}_N{s[1]}_K{s[2]}")
def test_decode_gemm_tiled16(dev, shape, dense3):
    M, N, K = shape
    G = K // 128
    bits = 3 if dense3 else 4
    announce("decode_gemm_tiled16", shape, dense3)
    rng = np.random.default_rng(M * 31 + N)
    q = rng.integers(0, 2 ** bits, size=(N, K))
    words = O.pack3(q) if dense3 else O.pack(q, np.zeros((N, G)), np.ones((N, G)))[0]
    layout = awq.LAYOUT_INT3_DENSE if dense3 else awq.LAYOUT_NIBBLE
    sb, zb = random_compact_meta(N, G, bits, seed=M + N)
    a = synth.decode_activations(K, M, seed=M + 13)
    ad = to_dev_bf16(a, dev)
    tiles = awq.decode_tiles(torch.from_numpy(words.view(np.int32)).to(dev), K, layout)
    st_d = torch.from_numpy(sb.view(np.float16)).to(dev)
    zb_d = torch.from_numpy(zb).to(dev)
    y16 = awq.decode_gemm_tiled16(ad, tiles, st_d, zb_d, layout)
    sc, ze = awq.expand_meta16(st_d, zb_d)
    y32 = awq.decode_gemm_tiled(ad, tiles, sc, ze, layout)
    meta = awq.decode_meta(st_d, zb_d)
    ymt = awq.decode_gemm_tiled_meta(ad, tiles, meta, N, layout)
    torch.cuda.synchronize()
    assert np.array_equal(meta.cpu().numpy().view(np.uint32), O.decode_meta(sb, zb, K))
    assert torch.equal(y16, y32)
    assert torch.equal(ymt, y16)
    _, fro = gemm_close(y16.cpu().numpy(), O.decode_gemm16(a, words, sb, zb, 128, dense3=dense3))
    assert fro <= 1e-5


def test_linear_module_compact_format(dev):
    """W4A16Linear in the compact format: decode path (M <= 64) against the
    oracle's compact product, and the many-token path through the expanded
    metadata against the oracle's bf16-operand product."""
    announce("W4A16Linear compact")
    x, w = synth.random_layer(200, 640, 264, seed=21, n_outlier=5, outlier_factor=20.0)
    s_all, _ = O.candidate_scales(O.act_stats(x)[1], 20)
    s = s_all[9]
    lin = awq.W4A16Linear.compact_from_weight(to_dev_bf16(w, dev), to_dev_f32(s, dev))
    assert lin.compact
    rq, rs, rz = oracle_compact(w, s, 4, False)
    st_ref, z_ref = O.unpack_meta16(rs, rz, 640 // 128)
    for M in (1, 16, 64, 65, 200):
        a = synth.decode_activations(640, M, seed=M + 2)
        y = lin(to_dev_bf16(a, dev)).cpu().numpy()
        if M <= 64:
            _, fro = gemm_close(y, O.decode_gemm16(a, rq, rs, rz, 128))
            assert fro <= 1e-5
        else:
            gemm_close(y, O.deploy_gemm(a, rq, st_ref.astype(np.float32), z_ref.astype(np.uint8), 128))
