"""The seeded input generators (CPU): determinism, prefix consistency and the
outlier recipe."""

import numpy as np

import synth


def test_weight_rows_are_a_prefix_of_the_full_draw():
    spec = synth.layer_spec("llama3_8b_block", "o_proj")
    full = synth.make_weight(spec)
    assert full.shape == (spec.N, spec.K) and full.dtype == np.uint16
    assert np.array_equal(synth.make_weight(spec, rows=37), full[:37])


def test_activation_tokens_are_a_prefix_and_deterministic():
    spec = synth.layer_spec("llama2_7b_qkv")
    a = synth.make_activations(spec, M=300)
    b = synth.make_activations(spec, M=100)
    assert np.array_equal(a[:100], b)
    assert np.array_equal(a, synth.make_activations(spec, M=300))
    assert not np.array_equal(a, synth.make_activations(spec, M=300, seed=1))


def test_outlier_recipe():
    spec = synth.layer_spec("llama2_7b_qkv")
    cols, f = synth.outlier_columns(spec)
    assert len(cols) == round(0.01 * spec.K) == len(np.unique(cols))
    assert np.all((f >= 10.0) & (f <= 50.0))
    x = synth.bf16_bits_to_f32(synth.make_activations(spec, M=2048)).astype(np.float64)
    mean_abs = np.abs(x).mean(axis=0)
    others = np.setdiff1d(np.arange(spec.K), cols)
    assert mean_abs[cols].min() > 5 * mean_abs[others].max()


def test_mlp_blocks_deterministic_and_shaped():
    x, blocks = synth.make_mlp_blocks(32, 256, 384, 2, seed=3)
    x2, blocks2 = synth.make_mlp_blocks(32, 256, 384, 2, seed=3)
    assert x.shape == (32, 256) and x.dtype == np.uint16 and np.array_equal(x, x2)
    assert len(blocks) == 2
    for (g, wgu, wd), (g2, wgu2, wd2) in zip(blocks, blocks2):
        assert g.shape == (256,) and g.dtype == np.float32 and 0.5 <= g.min() and g.max() <= 1.5
        assert wgu.shape == (768, 256) and wd.shape == (256, 384)
        assert np.array_equal(g, g2) and np.array_equal(wgu, wgu2) and np.array_equal(wd, wd2)
    assert not np.array_equal(blocks[0][1], blocks[1][1])
