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
