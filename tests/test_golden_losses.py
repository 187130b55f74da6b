"""The stored oracle losses (tests/golden/search_losses.json) on the CPU:
complete, well formed, and reproduced by the oracle.

The file is written by tests/golden/make_search_losses.py, which evaluates
the oracle's search loop row chunk by row chunk in threads.  Here: the chunked
evaluation equals O.search on small layers (direct and Gram form, and the
zeroed-rows form against a search on the zeroed weight), and the cheapest
stored case is recomputed from its seeded inputs and must match to the bit.
"""

import json
import os
import sys

import numpy as np
import pytest

import oracle as O
import synth

sys.path.insert(0, os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden"))
import make_search_losses as gold  # noqa: E402

with open(gold.OUT) as _f:
    GOLD = json.load(_f)["cases"]


def test_every_case_is_stored_and_well_formed():
    names = [c[0] for c in gold.cases()]
    assert sorted(names) == sorted(GOLD)
    for name, e in GOLD.items():
        losses = np.array([float.fromhex(v) for v in e["losses"]])
        assert losses.shape == (e["n_grid"],) and np.all(np.isfinite(losses)) and np.all(losses > 0)
        assert e["best_idx"] == O.first_argmin(losses), name
        assert losses[e["best_idx"]] <= losses[0]              # never worse than plain rounding
        assert len(e["x_blake2b"]) == 32 and len(e["w_blake2b"]) == 32
        if e["form"] == "rows":
            assert e["rows"] == [int(r) for r in gold.sampled_rows(e["N"], len(e["rows"]),
                                                                   e["rows_seed"])]


@pytest.mark.parametrize("gram", [False, True])
def test_chunked_losses_equal_the_oracle_search(gram):
    spec = synth.layer_spec("llama3_8b_block", "qkv")
    x = synth.make_activations(spec, 192)
    w = synth.make_weight(spec, rows=700)
    ref = O.search(x, w, 4, 128, 8, loss_form="gram" if gram else "direct")
    got, a32 = gold.oracle_losses(x, w, 4, 8, gram, workers=4)
    np.testing.assert_allclose(got, ref["losses"], rtol=1e-13, atol=0)
    assert np.array_equal(a32, ref["mean_abs"])


def test_zeroed_rows_losses_equal_a_search_on_the_zeroed_weight():
    spec = synth.layer_spec("llama2_70b_mlp", "gate_up")
    x = synth.make_activations(spec, 160)
    w = synth.make_weight(spec, rows=640)
    rows = gold.sampled_rows(640, 48, 5)
    w_z = np.zeros_like(w)
    w_z[rows] = w[rows]
    ref = O.search(x, w_z, 3, 128, 6)
    got, _ = gold.oracle_losses(x, w[rows], 3, 6, False, workers=4, n_rows_total=640)
    np.testing.assert_allclose(got, ref["losses"], rtol=1e-13, atol=0)


def test_cheapest_stored_case_is_reproduced():
    name = "llama3_8b_block/o_proj/int4/prefix1024"
    e = GOLD[name]
    spec = synth.layer_spec(e["workload"], e["layer"])
    x = synth.make_activations(spec, e["M"])
    w = synth.make_weight(spec)
    assert gold.fingerprint(x) == e["x_blake2b"] and gold.fingerprint(w) == e["w_blake2b"]
    got, _ = gold.oracle_losses(x, w, e["bits"], e["n_grid"], False,
                                workers=min(8, len(os.sched_getaffinity(0))))
    assert [float(v).hex() for v in got] == e["losses"]
