#!/usr/bin/env python3
"""Writes tests/golden/search_losses.json: the oracle's per-candidate losses
and first-minimum choice for every workload layer at full K and N, computed
on the CPU from the seeded synthetic inputs.  Only the oracle (oracle/) and
the input generators (synth/, which hold none of the method's arithmetic)
are called; nothing here comes from the HIP library.

The scale is the grid point whose candidate gives the smallest output error
of the layer over the calibration tokens (robotsatlas.com, "AWQ", How it
works; Key mechanisms).  The cases:

  full      the Llama-2-7B fused QKV layer in full (65536 tokens x 4096 ->
            12288), losses in the oracle's Gram form sum_n D_n G D_n^T with
            G = X^T X, the same value as the direct form (exact identity);
  prefix    every other workload layer at its full K and N on the first
            1024 calibration tokens (direct form, X (B - W)^T), both bit
            widths where the workload has two;
  rows      the Llama-2-70B gate/up layer at its full token count, K and N,
            with every weight row outside a seeded sample of 256 set to zero
            (the zero rows quantize to zero codes and contribute nothing),
            so the oracle's direct losses over the sampled rows are the
            whole layer's losses.

The loss is a sum over output rows, so each candidate's loss is evaluated
over chunks of rows (each chunk quantized by the oracle's own quantize, its
operand by dequant_operand, its error by output_mse / output_mse_gram) and
the chunks' sums are added in row order; jobs run in threads (numpy's
element-wise loops and BLAS release the GIL), each with single-threaded BLAS.

Inputs are fingerprinted (BLAKE2b of the bf16 bytes) so a test can tell that
the generator still draws the same layer.

    python tests/golden/make_search_losses.py [--only NAME ...] [--workers N]
"""

from __future__ import annotations

import argparse
import concurrent.futures as cf
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import oracle as O  # noqa: E402
import synth  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "search_losses.json")
PREFIX_M = 1024
ROW_SAMPLE = 256
ROW_SAMPLE_SEED = 17


def fingerprint(bits: np.ndarray) -> str:
    return hashlib.blake2b(np.ascontiguousarray(bits).view(np.uint8), digest_size=16).hexdigest()


def sampled_rows(N: int, k: int = ROW_SAMPLE, seed: int = ROW_SAMPLE_SEED) -> np.ndarray:
    """Seeded sample of weight rows (shared with the test that reads the file)."""
    return np.sort(np.random.default_rng(seed).choice(N, size=k, replace=False))


def cases():
    """(name, workload, layer, M or None for the full token count, bits, form)."""
    out = [("llama2_7b_qkv/qkv/full", "llama2_7b_qkv", "qkv", None, 4, "full")]
    for wl, layers in (("llama2_7b_mlp", ("gate_up", "down")),
                       ("llama3_8b_block", ("qkv", "o_proj", "gate_up", "down")),
                       ("llama2_70b_mlp", ("down", "gate_up"))):
        for name in layers:
            for bits in synth.layer_spec(wl, name).bits:
                out.append((f"{wl}/{name}/int{bits}/prefix{PREFIX_M}", wl, name, PREFIX_M, bits,
                            "prefix"))
    for bits in (3, 4):
        out.append((f"llama2_70b_mlp/gate_up/int{bits}/rows{ROW_SAMPLE}", "llama2_70b_mlp",
                    "gate_up", None, bits, "rows"))
    return out


def oracle_losses(x_bits, w_bits, bits: int, n_grid: int, gram: bool, workers: int,
                  n_rows_total: int | None = None):
    """The oracle's search losses (O.search's loop), row chunk by row chunk.

    Returns (losses, a32): MSE over M * n_rows_total outputs (n_rows_total
    defaults to the rows of w_bits; rows left out are zero rows whose error
    is exactly zero) and the fp32 statistics."""
    from threadpoolctl import threadpool_limits
    M, K = x_bits.shape
    N = w_bits.shape[0]
    n_total = N if n_rows_total is None else n_rows_total
    _, a32 = O.act_stats(x_bits)
    s32, inv32 = O.candidate_scales(a32, n_grid)
    G = O.gram(x_bits) if gram else None
    chunk = max(64, (1 << 23) // K)
    starts = list(range(0, N, chunk))

    def job(i, r0):
        wc = w_bits[r0:r0 + chunk]
        q, z, st = O.quantize(wc, s32[i], bits, 128)
        b = O.dequant_operand(q, z, st, 128, inv32[i])
        mse = O.output_mse_gram(G, M, wc, b) if gram else O.output_mse(x_bits, wc, b)
        return mse * wc.shape[0] * M          # this chunk's sum of squared errors

    sse = np.zeros((n_grid, len(starts)))
    with threadpool_limits(limits=1, user_api="blas"):
        with cf.ThreadPoolExecutor(max_workers=workers) as ex:
            futs = {ex.submit(job, i, r0): (i, c) for i in range(n_grid)
                    for c, r0 in enumerate(starts)}
            for f in cf.as_completed(futs):
                i, c = futs[f]
                sse[i, c] = f.result()
    losses = np.array([sum(sse[i, c] for c in range(len(starts))) for i in range(n_grid)])
    return losses / (float(M) * float(n_total)), a32


def run_case(name, wl, layer, M, bits, form, workers):
    t0 = time.perf_counter()
    spec = synth.layer_spec(wl, layer)
    x = synth.make_activations(spec, M, seed=0)
    w = synth.make_weight(spec, 0)
    entry = {"workload": wl, "layer": layer, "M": int(x.shape[0]), "K": spec.K, "N": spec.N,
             "bits": bits, "group": spec.group, "n_grid": spec.n_grid, "form": form,
             "x_blake2b": fingerprint(x), "w_blake2b": fingerprint(w)}
    if form == "rows":
        rows = sampled_rows(spec.N)
        entry["rows_seed"] = ROW_SAMPLE_SEED
        entry["rows"] = [int(r) for r in rows]
        losses, a32 = oracle_losses(x, w[rows], bits, spec.n_grid, False, workers,
                                    n_rows_total=spec.N)
    else:
        losses, a32 = oracle_losses(x, w, bits, spec.n_grid, form == "full", workers)
    entry["losses"] = [float(v).hex() for v in losses]
    entry["best_idx"] = O.first_argmin(losses)
    entry["seconds"] = round(time.perf_counter() - t0, 1)
    print(f"{name}: best {entry['best_idx']} losses {losses[0]:.6e} .. {losses.min():.6e} "
          f"({entry['seconds']} s)", flush=True)
    return entry


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--only", nargs="*", default=None, help="case names (substring match)")
    ap.add_argument("--workers", type=int, default=min(16, len(os.sched_getaffinity(0))))
    args = ap.parse_args()
    data = {}
    if os.path.exists(OUT):
        with open(OUT) as f:
            data = json.load(f)
    data.setdefault("about", (
        "Oracle losses (fp64, float.hex) and first-minimum index per workload layer, "
        "written by tests/golden/make_search_losses.py from the seeded synthetic inputs; "
        "robotsatlas.com 'AWQ', How it works: the scale minimises the layer's output error."))
    data.setdefault("cases", {})
    for c in cases():
        if args.only and not any(o in c[0] for o in args.only):
            continue
        data["cases"][c[0]] = run_case(*c, workers=args.workers)
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1, sort_keys=True)
            f.write("\n")
    return 0


if __name__ == "__main__":
    sys.exit(main())
