"""The whole GPU search against the oracle's losses at full K and N.

The scale is the grid point whose candidate gives the smallest output error
of the layer over the calibration tokens (robotsatlas.com, "AWQ", How it
works; Key mechanisms).  tests/golden/search_losses.json holds the oracle's
20 losses and first-minimum choice per case, written on the CPU by
tests/golden/make_search_losses.py from the seeded inputs (oracle and input
generators only).  Each test draws the same inputs, checks their
fingerprints against the file, runs awq_search_scale and compares:

  * every loss within 1e-4 relative of the oracle's;
  * the chosen index: the GPU's first minimum of its own losses, and the
    oracle's loss at it within 1e-4 of the oracle's minimum (ties);
  * the statistics within 1e-6 relative of the oracle's;
  * sampled rows of the final pack bit-exact against the oracle's pack at
    the GPU's chosen scale.

Cases: the Llama-2-7B fused QKV layer in full (the oracle's Gram form); every
other workload layer at full K and N on 1024 calibration tokens (four
256-row tiles, a grid whose tile count is a multiple of 8, so the XCD remap
and the 4-row-tile grouping are on); and the Llama-2-70B gate/up layer at
full size, with every weight row outside a seeded sample of 256 set to zero,
in the launch configuration of the full layer.
"""

import json
import os
import sys

import numpy as np
import pytest
import torch

import oracle as O
import post_weight_quantization_stats_amd as awq
import synth
from gpu_util import announce, require_gpu, to_dev_bf16, u32

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_search_losses as gold  # noqa: E402

pytestmark = pytest.mark.gpu

with open(gold.OUT) as _f:
    GOLD = json.load(_f)["cases"]


@pytest.fixture(scope="module")
def dev():
    return require_gpu()


def _inputs(entry):
    spec = synth.layer_spec(entry["workload"], entry["layer"])
    x = synth.make_activations(spec, entry["M"], seed=0)
    w = synth.make_weight(spec, 0)
    assert gold.fingerprint(x) == entry["x_blake2b"], "activation generator changed"
    assert gold.fingerprint(w) == entry["w_blake2b"], "weight generator changed"
    return spec, x, w


def _check(entry, out, x, w, check_rows):
    ref = np.array([float.fromhex(v) for v in entry["losses"]])
    got = out["losses"].cpu().numpy()
    assert np.isfinite(got).all()
    np.testing.assert_allclose(got, ref, rtol=1e-4, atol=0)
    best = int(out["best_idx"].item())
    assert best == O.first_argmin(got)
    assert ref[best] <= (1 + 1e-4) * ref.min(), (best, entry["best_idx"])
    _, a_ref = O.act_stats(x)
    a_gpu = out["mean_abs"].cpu().numpy()
    assert (np.abs(a_gpu - a_ref) / a_ref).max() <= 1e-6
    best_s = out["best_s"].cpu().numpy()
    rq, rs, rz = O.pack(*O.quantize(w[check_rows], best_s, entry["bits"], entry["group"]))
    assert np.array_equal(u32(out["qweight"])[check_rows], rq)
    assert np.array_equal(out["scales"].cpu().numpy()[check_rows], rs)
    assert np.array_equal(out["zeros"].cpu().numpy()[check_rows], rz)
    return got, ref


def _rows(N, k, seed):
    return np.sort(np.random.default_rng(seed).choice(N, size=k, replace=False))


@pytest.mark.parametrize("case", sorted(k for k, v in GOLD.items() if v["form"] != "rows"))
def test_search_against_oracle(dev, case):
    entry = GOLD[case]
    announce("search vs stored oracle losses", case)
    spec, x, w = _inputs(entry)
    out = awq.search_scale(to_dev_bf16(x, dev), to_dev_bf16(w, dev), entry["bits"],
                           entry["group"], entry["n_grid"])
    got, ref = _check(entry, out, x, w, _rows(spec.N, 32, 11))
    print(f"[case] {case}: max rel loss diff {np.max(np.abs(got / ref - 1)):.2e}, "
          f"alpha index {int(out['best_idx'].item())} (oracle {entry['best_idx']})", flush=True)


@pytest.mark.parametrize("case", sorted(k for k, v in GOLD.items() if v["form"] == "rows"))
def test_search_full_launch_sampled_rows(dev, case):
    """Full M, K and N (the launch the bench times); rows outside the sample
    are zero, so their candidates' errors are exactly zero and the losses
    are the oracle's over the sampled rows."""
    entry = GOLD[case]
    announce("full-size search, sampled weight rows", case)
    spec, x, w = _inputs(entry)
    rows = np.asarray(entry["rows"])
    assert np.array_equal(rows, gold.sampled_rows(spec.N, len(rows), entry["rows_seed"]))
    w_s = np.zeros_like(w)
    w_s[rows] = w[rows]
    del w
    out = awq.search_scale(to_dev_bf16(x, dev), to_dev_bf16(w_s, dev), entry["bits"],
                           entry["group"], entry["n_grid"])
    got, ref = _check(entry, out, x, w_s, rows[::8])
    # the zero rows were written as zero codes, unit steps and zero points
    zero_rows = np.setdiff1d(np.arange(0, spec.N, 997), rows)
    assert not u32(out["qweight"])[zero_rows].any()
    assert np.all(out["scales"].cpu().numpy()[zero_rows] == 1.0)
    assert not out["zeros"].cpu().numpy()[zero_rows].any()
    print(f"[case] {case}: max rel loss diff {np.max(np.abs(got / ref - 1)):.2e}", flush=True)
