"""The deployment module: construction checks and the scale fold (CPU), and
its routing by token count against the direct contractions and the oracle
(GPU)."""

import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_stats_amd as awq
import synth
from gpu_util import announce, gemm_close, require_gpu, to_dev_bf16, u32


def test_module_rejects_bad_shapes():
    qw = torch.zeros((8, 16), dtype=torch.int32)
    with pytest.raises(ValueError):
        awq.W4A16Linear(qw, torch.zeros((8, 2)), torch.zeros((8, 2), dtype=torch.uint8))
    with pytest.raises(ValueError):
        awq.W4A16Linear(qw.to(torch.int64), torch.zeros((8, 1)), torch.zeros((8, 1), dtype=torch.uint8))
    m = awq.W4A16Linear(qw, torch.zeros((8, 1)), torch.zeros((8, 1), dtype=torch.uint8))
    assert (m.in_features, m.out_features) == (128, 8)
    with pytest.raises(ValueError):
        m(torch.zeros((2, 64), dtype=torch.bfloat16))


def test_module_compact_format_shapes():
    """float16 steps select the compact format: zeros two per byte, [N][ceil(G/2)]."""
    qw = torch.zeros((8, 48), dtype=torch.int32)                  # K = 384, G = 3
    st = torch.zeros((8, 3), dtype=torch.float16)
    m = awq.W4A16Linear(qw, st, torch.zeros((8, 2), dtype=torch.uint8))
    assert m.compact and m.scales.dtype == torch.float16
    with pytest.raises(ValueError):
        awq.W4A16Linear(qw, st, torch.zeros((8, 3), dtype=torch.uint8))
    m32 = awq.W4A16Linear(qw, st.float(), torch.zeros((8, 3), dtype=torch.uint8))
    assert not m32.compact and m32.scales.dtype == torch.float32
    assert "compact=True" in repr(m)


def test_fold_inverse_scale_needs_gpu_tensors():
    """The fold runs in the library (awq_divide_rows), never in torch."""
    g = torch.ones(16, dtype=torch.float32)
    with pytest.raises(ValueError, match="GPU tensor"):
        awq.fold_inverse_scale(g, torch.ones(16))
    with pytest.raises(ValueError, match="16 elements"):
        awq.fold_inverse_scale(g, torch.ones(8))


@pytest.mark.gpu
def test_fold_inverse_scale():
    """Folding 1/s into a gain or into a previous layer's rows makes its
    output X / s: (diag(g) X) / s = diag(g / s) X; each element is one IEEE
    fp32 division, bit-exact against the oracle's divide_rows."""
    dev = require_gpu()
    announce("fold_inverse_scale")
    rng = np.random.default_rng(3)
    K = 16
    g = rng.uniform(0.5, 2.0, K).astype(np.float32)
    s = rng.uniform(0.25, 4.0, K).astype(np.float32)
    folded = awq.fold_inverse_scale(torch.from_numpy(g).to(dev), torch.from_numpy(s).to(dev))
    assert folded.dtype == torch.float32
    assert np.array_equal(folded.cpu().numpy().astype(np.float64), O.divide_rows(g, s))
    Wp = rng.standard_normal((K, 7)).astype(np.float32)             # previous layer rows
    fw = awq.fold_inverse_scale(torch.from_numpy(Wp).to(dev).to(torch.bfloat16),
                                torch.from_numpy(s).to(dev))
    wp_bf16 = torch.from_numpy(Wp).to(torch.bfloat16).float().numpy()
    assert np.array_equal(fw.cpu().numpy().astype(np.float64), O.divide_rows(wp_bf16, s))
    h = rng.standard_normal((5, 7))
    np.testing.assert_allclose(h @ fw.cpu().double().numpy().T,
                               (h @ wp_bf16.astype(np.float64).T) / s.astype(np.float64),
                               rtol=1e-5, atol=1e-6)


@pytest.mark.gpu
def test_module_routes_by_token_count():
    dev = require_gpu()
    announce("W4A16Linear routing")
    x, w = synth.random_layer(300, 512, 200, seed=11, n_outlier=5, outlier_factor=20.0)
    res = awq.search_scale(to_dev_bf16(x, dev), to_dev_bf16(w, dev))
    lin = awq.W4A16Linear.from_search(res)
    qw, sc, ze = u32(res["qweight"]), res["scales"].cpu().numpy(), res["zeros"].cpu().numpy()
    for M in (1, 17, 64, 65, 300):
        a = synth.decode_activations(512, M, seed=M)
        ad = to_dev_bf16(a, dev)
        y = lin(ad)
        torch.cuda.synchronize()
        if M <= 64:
            direct = awq.decode_gemm(ad, res["qweight"], res["scales"], res["zeros"])
            _, fro = gemm_close(y.cpu().numpy(), O.decode_gemm(a, qw, sc, ze, 128))
            assert fro <= 1e-5
        else:
            direct = awq.w4a16_gemm(ad, res["qweight"], res["scales"], res["zeros"])
            gemm_close(y.cpu().numpy(), O.deploy_gemm(a, qw, sc, ze, 128))
        assert torch.equal(y, direct), M
    y3 = lin(to_dev_bf16(synth.decode_activations(512, 6, seed=1), dev).reshape(2, 3, 512))
    assert tuple(y3.shape) == (2, 3, 200)
