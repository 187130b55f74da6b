#!/usr/bin/env python3
"""Throughput of the AWQ per-layer scale search on one MI355X.

One step = one whole search over one layer (activation statistics, 20
candidate scales, 20 x (quantize to the candidate's difference operand +
contraction with the fused sum of squares), loss reduction, argmin, final
quantize + pack) with the inputs already resident in HBM.  Default workload:
the workloads' largest layer, a Llama-2-70B-shaped MLP gate/up projection,
16384 calibration tokens, K=8192 -> N=2x28672, INT4, group 128, 20 grid
points, seeded synthetic data; the same layer at INT3, the Llama-2-7B fused
QKV layer and every other workload layer are reported beside it.

Prints ONE JSON line.  Per-kernel durations come from HIP events recorded on
the stream the kernels are launched on; the roofline block uses the
per-candidate contraction with the squared-error epilogue (the dominant
kernel).  The packed W4A16 contraction and the decode-shaped W4A16 kernel are
timed beside it.  cpu_baseline times the CPU oracle on a bounded
sample of the same layer and scales it to the full layer.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
METRIC = "AWQ search: layers/s + W4A16 GEMM TFLOP/s (% MFMA peak), quant GB/s (% HBM)"
PROFILES = os.path.join(ROOT, "profiles")
HEADLINE = ("llama2_70b_mlp", "gate_up", 4)


def traffic_file(workload: str, layer: str) -> str:
    return os.path.join(PROFILES, f"search_contraction_{workload}_{layer}_traffic.txt")
# The search's per-candidate contraction X . D^T with the sum-of-squares epilogue.
DOMINANT_KERNEL = "mfma16_kernel<false, 1>"
GEMM_SOURCES = ["w4a16_gemm.hip", "device_common.h", "awq_internal.h"]


def gemm_source_hash() -> str:
    """Hash of the contraction kernel sources (ties counter data to a kernel version)."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "post_weight_quantization_stats_amd", "csrc")
    for name in GEMM_SOURCES:
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def committed_traffic(workload: str, layer: str):
    """HBM bytes per launch of the search's dominant contraction on this
    layer from the committed rocprofv3 counter summary, or None when there is
    none or the kernel source changed since it was taken."""
    try:
        fields = {}
        with open(traffic_file(workload, layer)) as f:
            for line in f:
                if ":" in line and not line.startswith("#"):
                    k, v = line.split(":", 1)
                    fields[k.strip()] = v.strip()
        if fields.get("kernel_source_hash") != gemm_source_hash():
            return None
        return float(fields["hbm_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


# ---- rocprofv3 output summaries (run on the host after a profiled bench) ----

# The decode kernel's few-token template flags (one token, two to four, five
# to eight), as the demangled name spells them, and their labels.
FEW_TOKENS = {"false, false, false": "", "true, false, false": ", one token",
              "false, true, false": ", 2-4 tokens", "false, false, true": ", 5-8 tokens"}

KERNEL_LABELS = [
    # mfma16_kernel<store Y, epilogue (0 none, 1 sum of squares, 2 SSE vs Y_ref, 3 dot with Y_ref)>
    ("mfma16_kernel<false, 1>", "search contraction X.D^T (difference operand, sum of squares)"),
    ("mfma16_kernel<false, 3>", "Gram-form contraction (split D . split G, dot epilogue)"),
    ("mfma16_kernel<false, 2>", "candidate_sse vs y_ref (bf16 operand, squared-error epilogue)"),
    ("mfma16_kernel<true, 2>", "staged W4A16 product with SSE (bf16 operand, Y and SSE)"),
    ("mfma16_kernel<true, 0>", "reference_gemm / Gram matrix / staged W4A16 (bf16, fp32 out)"),
    # gemm_kernel<packed, 1/s, waves/2, store Y, SSE, dot, dense INT3>
    ("gemm_kernel<true, true, 2, false, true, false, false>",
     "w4a16_gemm_sse (INT4 operand, 1/s folded, SSE epilogue)"),
    ("gemm_kernel<true, true, 2, false, true, false, true>",
     "w3a16_gemm_sse (dense INT3 operand, 1/s folded, SSE epilogue)"),
    ("gemm_kernel<true", "w4a16_gemm / w3a16_gemm (packed operand, other epilogues)"),
    ("quantize_kernel<4, 1,", "dequant_operand (quantize -> bf16 B)"),
    ("quantize_kernel<3, 1,", "dequant_operand (quantize -> bf16 B)"),
    ("quantize_kernel<4, 2,", "Gram-form quantize (split D, fp32 D)"),
    ("quantize_kernel<3, 2,", "Gram-form quantize (split D, fp32 D)"),
    ("quantize_kernel<4, 3,", "diff_operand (quantize -> bf16 B - W)"),
    ("quantize_kernel<3, 3,", "diff_operand (quantize -> bf16 B - W)"),
    ("quantize_kernel<4, 0, true>", "quantize_pack16 (compact format)"),
    ("quantize_kernel<3, 0, true>", "quantize_pack16 (compact format)"),
    ("quantize_kernel<3, 4, true>", "quantize_pack16 (compact format, dense INT3)"),
    ("quantize_kernel<3, 4,", "quantize_pack3 (dense INT3)"),
    ("dequant_nibble_kernel", "staged operand from 4-bit containers"),
    ("dequant_int3_kernel", "staged operand from dense INT3"),
    ("expand_meta16", "compact metadata expansion"),
    ("decode_tiles_kernel", "decode tiles"),
    ("transpose_pad_kernel", "X^T (Gram form)"),
    ("gram_split_kernel", "G split (Gram form)"),
    # decode_gemm_kernel<column blocks, token blocks, INT3 dense, tiled,
    # metadata source (0 fp32 table, 1 compact table, 2 metadata tiles), waves,
    # one token, two to four tokens, five to eight tokens>
    *[(("decode_gemm_kernel<", f", {flags}, {waves}, {few}>"),
       label + ("" if waves == 4 else ", 8 waves") + FEW_TOKENS[few])
      for flags, label in (("false, true, 2", "decode GEMM, tiles, metadata tiles"),
                           ("true, true, 2", "decode GEMM, dense INT3 tiles, metadata tiles"),
                           ("false, true, 1", "decode GEMM, tiles, compact metadata"),
                           ("true, true, 1", "decode GEMM, dense INT3 tiles, compact metadata"),
                           ("false, true, 0", "decode GEMM, tiles"),
                           ("true, true, 0", "decode GEMM, dense INT3 tiles"),
                           ("false, false, 0", "decode GEMM, row-major words"),
                           ("true, false, 0", "decode GEMM, dense INT3 row-major"))
      for waves in (4, 8) for few in FEW_TOKENS],
    # decode_cols_kernel<column blocks per wave, token blocks, code ring,
    # INT3 dense, tiled, metadata source>: large layers above 32 tokens
    *[(("decode_cols_kernel<", f", {mb}, 4, {flags}>"),
       f"decode GEMM, column split, {16 * mb} tokens per workgroup, " + label)
      for flags, label in (("false, true, 2", "tiles, metadata tiles"),
                           ("true, true, 2", "dense INT3 tiles, metadata tiles"),
                           ("false, true, 1", "tiles, compact metadata"),
                           ("true, true, 1", "dense INT3 tiles, compact metadata"),
                           ("false, true, 0", "tiles"),
                           ("true, true, 0", "dense INT3 tiles"),
                           ("false, false, 0", "row-major words"),
                           ("true, false, 0", "dense INT3 row-major"))
      for mb in (2, 4)],
    ("meta_tiles_kernel", "metadata tiles"),
    ("mfma_ceiling_kernel", "ceiling: matrix cores from registers"),
    ("copy_ceiling_kernel", "ceiling: copy"),
    ("read_ceiling_kernel", "ceiling: read"),
    ("write_ceiling_kernel", "ceiling: write"),
    ("decode_gemm", "decode W4A16 GEMM (M <= 64)"),
    ("decode_reduce", "decode split-K reduce"),
    ("act_stats_partial", "act_stats partial sums"),
    ("act_stats_finalize", "act_stats finalize"),
    ("quantize_kernel", "quantize_pack"),
    ("scales_r_kernel", "candidate scales (powers)"),
    ("scales_norm_kernel", "candidate scales (normalise)"),
    ("loss_reduce_kernel", "loss reduce"),
    ("argmin_kernel", "argmin"),
    ("select_row_kernel", "select s*"),
    ("fill_f64_kernel", "fill"),
    ("Cijk_", "hipBLASLt bf16 GEMM (vendor yardstick, same operands)"),
    ("FillFunctor<float>", "one-element fill (launch floor; also torch fills)"),
]


def _label(name: str) -> str:
    for key, label in KERNEL_LABELS:
        keys = key if isinstance(key, tuple) else (key,)
        if all(k in name for k in keys):
            return label
    return name[:60]


def _read_csv(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _find(d: str, suffix: str) -> str:
    import glob
    hits = sorted(glob.glob(os.path.join(d, "**", "*" + suffix), recursive=True))
    if not hits:
        raise SystemExit(f"no *{suffix} under {d}")
    return hits[0]


def _bench_line(log_path):
    try:
        with open(log_path) as f:
            for line in f:
                if line.startswith("{"):
                    return json.loads(line)
    except OSError:
        pass
    return None


N_XCD, N_CU, SIMD_PER_CU = 8, 256, 4


def summarize_mfma(pmc_dir: str, command: str) -> str:
    """Clock and matrix-core occupancy per kernel from one counter pass
    (GRBM_GUI_ACTIVE summed over the XCDs, SQ_BUSY_CU_CYCLES over the CUs,
    SQ_VALU_MFMA_BUSY_CYCLES over the SIMDs, SQ_INSTS_VALU_MFMA_MOPS_BF16 in
    units of 512 flops)."""
    rows = _read_csv(_find(pmc_dir, "counter_collection.csv"))
    per = {}
    for r in rows:
        name = r["Kernel_Name"]
        if "awq::" not in name and "Cijk_" not in name:
            continue
        key = (r["Dispatch_Id"], name)
        d = per.setdefault(key, {"dur": (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9})
        d[r["Counter_Name"]] = float(r["Counter_Value"])
    by = {}
    for (_, name), d in per.items():
        by.setdefault(_label(name), []).append(d)
    out = ["# rocprofv3 counters: clock and matrix-core occupancy per kernel (medians over dispatches)",
           f"# command: {command}",
           "# clock = GRBM_GUI_ACTIVE / 8 XCDs / duration; mfma_busy = SQ_VALU_MFMA_BUSY_CYCLES /",
           "# (4 SIMDs x SQ_BUSY_CU_CYCLES); tflops = 512 x SQ_INSTS_VALU_MFMA_MOPS_BF16 / duration",
           "# (the clock is meaningful only for kernels much longer than the counter window)", ""]
    out.append(f"{'kernel':<62} {'n':>3} {'dur_ms':>8} {'clock_GHz':>9} {'mfma_busy':>9} {'tflops':>8}")
    for label, ds in sorted(by.items()):
        if not all("GRBM_GUI_ACTIVE" in d and "SQ_VALU_MFMA_BUSY_CYCLES" in d for d in ds):
            continue
        med = lambda f: float(np.median([f(d) for d in ds]))
        dur = med(lambda d: d["dur"])
        clock = med(lambda d: d["GRBM_GUI_ACTIVE"] / N_XCD / d["dur"] / 1e9)
        busy = med(lambda d: d["SQ_VALU_MFMA_BUSY_CYCLES"] / (SIMD_PER_CU * max(d["SQ_BUSY_CU_CYCLES"], 1)))
        tfl = med(lambda d: 512.0 * d.get("SQ_INSTS_VALU_MFMA_MOPS_BF16", 0.0) / d["dur"] / 1e12)
        out.append(f"{label:<62} {len(ds):>3} {dur * 1e3:>8.3f} {clock:>9.2f} {busy:>9.1%} {tfl:>8.0f}")
    return "\n".join(out) + "\n"


def summarize_trace(trace_dir: str, command: str, log_path: str | None) -> str:
    rows = _read_csv(_find(trace_dir, "kernel_stats.csv"))
    out = ["# rocprofv3 kernel-trace statistics", f"# command: {command}", ""]
    out.append(f"{'kernel':<62} {'calls':>6} {'avg_us':>10} {'min_us':>10} {'max_us':>10} {'pct':>6}")
    for r in rows:
        name = r["Name"]
        if "awq::" not in name and "Cijk_" not in name and "FillFunctor<float>" not in name:
            continue
        out.append(f"{_label(name):<62} {int(r['Calls']):>6} {float(r['AverageNs']) / 1e3:>10.1f} "
                   f"{float(r['MinNs']) / 1e3:>10.1f} {float(r['MaxNs']) / 1e3:>10.1f} "
                   f"{float(r['Percentage']):>6.2f}")
    line = _bench_line(log_path) if log_path else None
    if line and "int4" in line:
        out += ["", "# same run, bench.py figures (HIP-graph replays, weights rotated beyond the LLC):"]
        for case, v in line["int4"].items():
            if not isinstance(v, dict):
                out.append(f"{case}: {v:.2f}")
                continue
            out.append(f"{case}: tiles {v['us']:.2f} us ({v['gbs']:.0f} GB/s), row-major "
                       f"{v['row_major_us']:.2f} us, compact metadata {v['compact_us']:.2f} us "
                       f"({v['compact_gbs']:.0f} GB/s)")
    elif line:
        rf = line["roofline"]
        out += ["", "# same run, bench.py HIP-event figures:",
                f"search ms/layer: {line['ms_per_step']:.2f}",
                f"dominant kernel ms_per_launch (events): {rf['ms_per_launch']:.3f}",
                f"kernel_source_hash: {rf['kernel_source_hash']}"]
        for k, v in line["kernels"].items():
            if isinstance(v, dict) and all(isinstance(b, (int, float)) for b in v.values()):
                out.append(f"{k}: " + ", ".join(f"{a}={b:.4g}" for a, b in v.items()))
    return "\n".join(out) + "\n"


def summarize_counters(dirs, command: str) -> str:
    """Per-kernel medians of every counter in one or more rocprofv3 --pmc
    runs, with the dispatch's grid, workgroup and register counts.  FETCH_SIZE
    is in KiB per dispatch and reads half the bytes moved (the calibration of
    the search-contraction traffic summary), so bytes = 2 x 1024 x FETCH_SIZE;
    SQ_WAVES counts the waves launched."""
    per = {}
    for d in dirs:
        for r in _read_csv(_find(d, "counter_collection.csv")):
            name = r["Kernel_Name"]
            if "awq::" not in name and "FillFunctor<float>" not in name:
                continue
            key = _label(name) if "awq::" in name else "one-element fill (launch floor)"
            e = per.setdefault(key, {"dur": [], "meta": (r["Grid_Size"], r["Workgroup_Size"],
                                                         r["VGPR_Count"], r["LDS_Block_Size"])})
            e.setdefault(r["Counter_Name"], []).append(float(r["Counter_Value"]))
            if r["Counter_Name"] == sorted({x for x in e if x not in ("dur", "meta")})[0]:
                e["dur"].append((int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-3)
    out = ["# rocprofv3 counters per kernel (medians over dispatches)", f"# commands: {command}", ""]
    for key, e in sorted(per.items()):
        grid, wg, vgpr, lds = e["meta"]
        out.append(f"{key}: grid {grid} threads, workgroup {wg}, {vgpr} VGPRs, {lds} B LDS, "
                   f"waves {int(grid) // 64}; duration in the counter run {np.median(e['dur']):.2f} us")
        for c, v in sorted(e.items()):
            if c in ("dur", "meta"):
                continue
            extra = f"  (= {2 * 1024 * np.median(v) / 1e6:.2f} MB)" if c == "FETCH_SIZE" else ""
            out.append(f"    {c:<24} {np.median(v):>14.6g}{extra}")
    return "\n".join(out) + "\n"


def _per_kernel_counter(rows, counter):
    """Counter value per dispatch, grouped by kernel label."""
    per = {}
    for r in rows:
        if r["Counter_Name"] != counter:
            continue
        per.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
    return per


def summarize_pmc(fetch_dir: str, write_dir: str, commands: str, M: int, K: int) -> str:
    """HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE (KiB per dispatch),
    each scaled by what the counter reads for the calibration copy (bf16 X ->
    fp32: 2MK bytes read, 4MK bytes written)."""
    fetch = _per_kernel_counter(_read_csv(_find(fetch_dir, "counter_collection.csv")), "FETCH_SIZE")
    write = _per_kernel_counter(_read_csv(_find(write_dir, "counter_collection.csv")), "WRITE_SIZE")

    def calib(per, nbytes):
        # The bench's calibration copy is torch's bf16 -> fp32 conversion of
        # X (other copies, e.g. of W, can be larger, so match it by name).
        cands = [(v[0], k) for k, v in per.items() if "bfloat16tofloat32" in k]
        if not cands:
            raise SystemExit("calibration copy kernel (bf16 -> fp32) not found")
        kib, _ = cands[0]
        return nbytes / (kib * 1024.0), kib

    f_read, kib_r = calib(fetch, 2.0 * M * K)
    f_write, kib_w = calib(write, 4.0 * M * K)
    out = ["# rocprofv3 HBM traffic per dispatch (FETCH_SIZE and WRITE_SIZE, separate runs)",
           f"# commands: {commands}",
           f"# calibration copy (bf16 X -> fp32, M={M} K={K}): FETCH_SIZE {kib_r:.0f} KiB for "
           f"{2 * M * K} B read -> read factor {f_read:.4f}; WRITE_SIZE {kib_w:.0f} KiB for "
           f"{4 * M * K} B written -> write factor {f_write:.4f}", ""]
    gemm_bytes = None
    for name in sorted(set(fetch) | set(write), key=_label):
        if "awq::" not in name and "Cijk_" not in name:
            continue
        fr = fetch.get(name, [float("nan")])
        wr = write.get(name, [float("nan")])
        rb = float(np.median(fr)) * 1024.0 * f_read
        wb = float(np.median(wr)) * 1024.0 * f_write
        out.append(f"{_label(name):<62} read {rb / 2**20:>10.1f} MiB  write {wb / 2**20:>9.1f} MiB  "
                   f"(dispatches {len(fr)}/{len(wr)})")
        if DOMINANT_KERNEL in name:
            gemm_bytes = rb + wb
    out.append("")
    out.append(f"kernel_source_hash: {gemm_source_hash()}")
    if gemm_bytes is not None:
        out.append(f"hbm_bytes_per_launch: {gemm_bytes:.0f}")
    return "\n".join(out) + "\n"


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def event_time_ms(fn, reps: int, stream) -> float:
    """Average duration of fn() over reps launches, HIP events on `stream`,
    after one untimed call (first-use setup, e.g. a library's kernel load)."""
    import torch
    fn()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    start.record(stream)
    for _ in range(reps):
        fn()
    end.record(stream)
    end.synchronize()
    return start.elapsed_time(end) / reps


def measure_ceilings(awq, dev, stream, src) -> dict:
    """What this GPU sustains, from the library's ceiling kernels: the
    matrix cores fed from registers (bf16 16x16x32, random and zero
    operands) and streaming copy / read / write over the bytes of `src`
    (larger than the last-level cache).  Kernels are reported as fractions
    of these beside their fractions of the spec."""
    import torch
    nbytes = src.numel() * src.element_size() // 16 * 16
    dst = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    sink = torch.zeros(4, dtype=torch.float32, device=dev)
    gbs = lambda nb, ms: nb / (ms * 1e-3) / 1e9
    # The best grid of each kernel (it differs by kernel and part), up to one
    # pass over the bytes (one 16-byte step per lane; the read kernel's
    # unrolled step covers four).
    n16 = nbytes // 16
    grids = (1024, 4096, 16384, 65536, n16 // 1024, n16 // 256)
    t_copy, t_read, t_write = (min(event_time_ms(
        lambda: awq.ceiling_stream(mode, a, b, nbytes, g), 5, stream) for g in grids)
        for mode, a, b in ((awq.CEILING_COPY, src, dst), (awq.CEILING_READ, src, sink),
                           (awq.CEILING_WRITE, None, dst)))
    blocks, iters = 1024, 5000
    flops = awq.ceiling_mfma(sink, blocks, iters)
    t_mfma = event_time_ms(lambda: awq.ceiling_mfma(sink, blocks, iters), 3, stream)
    t_mfma0 = event_time_ms(lambda: awq.ceiling_mfma(sink, blocks, iters, zero=True), 3, stream)
    out = {"copy_gbs": gbs(2.0 * nbytes, t_copy), "read_gbs": gbs(nbytes, t_read),
           "write_gbs": gbs(nbytes, t_write), "stream_bytes": nbytes, "stream_grids": grids,
           "mfma_bf16_tflops": flops / (t_mfma * 1e-3) / 1e12,
           "mfma_bf16_zero_operands_tflops": flops / (t_mfma0 * 1e-3) / 1e12,
           "mfma_flops_per_launch": flops}
    log(f"measured ceilings: copy {out['copy_gbs']:.0f} GB/s, read {out['read_gbs']:.0f} GB/s, "
        f"write {out['write_gbs']:.0f} GB/s; bf16 matrix cores from registers "
        f"{out['mfma_bf16_tflops']:.0f} TFLOP/s (zero operands {out['mfma_bf16_zero_operands_tflops']:.0f})")
    del dst, sink
    return out


def _graph_time_ms(fn, reps: int, stream) -> float:
    """Average time of fn(i), i = 0..reps-1, captured in one HIP graph and
    replayed (host launch overhead excluded)."""
    import torch
    fn(0)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(reps):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    ms = event_time_ms(g.replay, 5, stream) / reps
    del g
    return ms


def bench_decode(awq, dev, stream, reps: int = 96, layers=("qkv", "o_proj", "gate_up", "down"),
                 token_counts=(1, 2, 4, 8, 16, 32, 64)) -> dict:
    """Decode-shaped W4A16 contraction on the Llama-3-8B block's layers
    (M = 1, 2, 4, 8, 16, 32 and 64 tokens, random packed INT4 weights), on decode tiles
    with fp32 steps and u8 zeros, on the row-major packed words, on decode
    tiles with the compact metadata (binary16 steps, 4-bit zeros) and on
    decode tiles with metadata tiles (the compact metadata as one u32 per row
    and group, the deployment module's path).  Launches cycle
    through enough copies of the packed weights (>= 768 MiB in all) that each
    one streams from HBM rather than the 256 MiB last-level cache."""
    import torch

    import synth
    out = {}
    # Fixed per-launch floor: a kernel with no work to speak of (a one-element
    # fill), replayed from a graph exactly like the decode calls.
    z1 = torch.zeros(1, device=dev)
    floor_ms = _graph_time_ms(lambda i: z1.fill_(float(i) + 1.0), reps, stream)
    out["empty_kernel_us"] = floor_ms * 1e3
    log(f"one-element kernel (launch floor) in a graph replay: {floor_ms * 1e3:.2f} us")
    for name in layers:
        spec = synth.layer_spec("llama3_8b_block", name)
        N, K = spec.N, spec.K
        wbytes = N * K / 2 + 5.0 * N * K / 128
        copies = int(min(32, max(2, -(-(768 << 20) // int(wbytes)))))
        gen = torch.Generator(device=dev).manual_seed(7)
        packs = []
        for _ in range(copies):
            qw = torch.randint(-2 ** 31, 2 ** 31 - 1, (N, K // 8), dtype=torch.int32, device=dev,
                               generator=gen)
            sc = torch.rand((N, K // 128), device=dev, generator=gen) * 0.003 + 0.001
            ze = torch.randint(0, 16, (N, K // 128), dtype=torch.uint8, device=dev, generator=gen)
            z4 = torch.randint(0, 256, (N, (K // 128 + 1) // 2), dtype=torch.uint8, device=dev,
                               generator=gen)
            st16 = sc.half()
            packs.append((qw, awq.decode_tiles(qw, K), sc, ze, st16, z4, awq.decode_meta(st16, z4)))
        for M in token_counts:
            a = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
            y = torch.empty((M, N), dtype=torch.float32, device=dev)
            need = awq.workspace_size(awq.OP_DECODE_GEMM, M, N, K)
            ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

            def tiled(i):
                _, tl, sc, ze, _, _, _ = packs[i % copies]
                awq.decode_gemm_tiled(a, tl, sc, ze, awq.LAYOUT_NIBBLE, out=y, workspace=ws)

            def row_major(i):
                qw, _, sc, ze, _, _, _ = packs[i % copies]
                awq.decode_gemm(a, qw, sc, ze, 4, out=y, workspace=ws)

            def compact(i):
                _, tl, _, _, st16, z4, _ = packs[i % copies]
                awq.decode_gemm_tiled16(a, tl, st16, z4, awq.LAYOUT_NIBBLE, out=y, workspace=ws)

            def meta_tiles(i):
                _, tl, _, _, _, _, mt = packs[i % copies]
                awq.decode_gemm_tiled_meta(a, tl, mt, N, awq.LAYOUT_NIBBLE, out=y, workspace=ws)
            if M == token_counts[0]:
                _graph_time_ms(tiled, reps, stream)   # untimed: first touch of this layer's copies
            ms = _graph_time_ms(tiled, reps, stream)
            ms_rm = _graph_time_ms(row_major, reps, stream)
            ms_c = _graph_time_ms(compact, reps, stream)
            ms_m = _graph_time_ms(meta_tiles, reps, stream)
            io = 2.0 * M * K + 4.0 * M * N
            nbytes = wbytes + io
            gbs = nbytes / (ms * 1e-3) / 1e9
            cbytes = N * K / 2 + 2.5 * N * K / 128 + io
            cgbs = cbytes / (ms_c * 1e-3) / 1e9
            mbytes = N * K / 2 + 4.0 * N * K / 128 + io
            mgbs = mbytes / (ms_m * 1e-3) / 1e9
            out[f"{name}_M{M}"] = {"N": N, "K": K, "us": ms * 1e3, "gbs": gbs,
                                   "frac_hbm_peak": gbs / PEAK_HBM_GBS, "bytes": nbytes,
                                   "row_major_us": ms_rm * 1e3, "compact_us": ms_c * 1e3,
                                   "compact_bytes": cbytes, "compact_gbs": cgbs,
                                   "meta_tiles_us": ms_m * 1e3, "meta_tiles_bytes": mbytes,
                                   "meta_tiles_gbs": mgbs,
                                   "meta_tiles_frac_hbm_peak": mgbs / PEAK_HBM_GBS,
                                   "weight_copies": copies}
            log(f"decode {name} M={M} N={N} K={K}: tiles {ms * 1e3:.2f} us = {gbs:.0f} GB/s; "
                f"row-major {ms_rm * 1e3:.2f} us; compact metadata {ms_c * 1e3:.2f} us = "
                f"{cgbs:.0f} GB/s; metadata tiles {ms_m * 1e3:.2f} us = {mgbs:.0f} GB/s "
                f"({copies} weight copies)")
        del packs
        torch.cuda.empty_cache()
    return out


def bench_decode_int3(awq, dev, stream, reps: int = 64) -> dict:
    """Decode-shaped contraction on the Llama-2-70B MLP's INT3 layers, dense
    INT3 words (3 bits per weight) beside the same codes in 4-bit containers,
    both as decode tiles, M = 1, 16 and 64 (at 64 tokens both layers take the
    column-split kernel), weights rotated beyond the last-level cache."""
    import torch

    import synth
    out = {}
    for name in ("down", "gate_up"):
        spec = synth.layer_spec("llama2_70b_mlp", name)
        N, K = spec.N, spec.K
        gen = torch.Generator(device=dev).manual_seed(11)
        sz_bytes = 5.0 * N * K / 128
        for layout in ("dense", "container"):
            wbytes = (3.0 * N * K / 8 if layout == "dense" else N * K / 2) + sz_bytes
            copies = int(min(16, max(2, -(-(768 << 20) // int(wbytes)))))
            packs = []
            for _ in range(copies):
                words = 3 * K // 32 if layout == "dense" else K // 8
                qw = torch.randint(-2 ** 31, 2 ** 31 - 1, (N, words), dtype=torch.int32,
                                   device=dev, generator=gen)
                if layout == "container":
                    qw &= 0x77777777          # 3-bit codes in 4-bit fields
                sc = torch.rand((N, K // 128), device=dev, generator=gen) * 0.003 + 0.001
                ze = torch.randint(0, 8, (N, K // 128), dtype=torch.uint8, device=dev,
                                   generator=gen)
                lay = awq.LAYOUT_INT3_DENSE if layout == "dense" else awq.LAYOUT_NIBBLE
                packs.append((awq.decode_tiles(qw, K, lay), sc, ze))
                del qw
            for M in (1, 16, 64):
                a = torch.randn((M, K), device=dev, generator=gen).to(torch.bfloat16)
                y = torch.empty((M, N), dtype=torch.float32, device=dev)
                need = awq.workspace_size(awq.OP_DECODE_GEMM, M, N, K, 3)
                ws = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)

                def fn(i):
                    tl, sc, ze = packs[i % copies]
                    awq.decode_gemm_tiled(a, tl, sc, ze, lay, out=y, workspace=ws)
                ms = _graph_time_ms(fn, reps, stream)
                nbytes = wbytes + 2.0 * M * K + 4.0 * M * N
                gbs = nbytes / (ms * 1e-3) / 1e9
                out[f"{name}_{layout}_M{M}"] = {"N": N, "K": K, "us": ms * 1e3, "gbs": gbs,
                                                "frac_hbm_peak": gbs / PEAK_HBM_GBS,
                                                "bytes": nbytes, "weight_copies": copies}
                log(f"decode int3 {layout} (tiles) {name} M={M} N={N} K={K}: {ms * 1e3:.2f} us = "
                    f"{gbs:.0f} GB/s")
            del packs
            torch.cuda.empty_cache()
    return out


def bench_gram(awq, xd, wd, spec, bits: int, direct: dict, steps: int, direct_ms: float) -> dict:
    """The same search with Gram-form losses (G = X^T X once, then per
    candidate D G D^T against a two-term bf16 split of G): a second workload
    with the same result, reported beside the headline, never in its place."""
    import torch

    M, K, N, G = spec.M, spec.K, spec.N, spec.n_grid
    ws = torch.empty(awq.workspace_size(awq.OP_SEARCH_SCALE_GRAM, M, N, K, bits, spec.group, G),
                     dtype=torch.uint8, device=xd.device)
    g = awq.search_scale_gram(xd, wd, bits, spec.group, G, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g = awq.search_scale_gram(xd, wd, bits, spec.group, G, workspace=ws)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    la, lg = direct["losses"].double(), g["losses"].double()
    rel = float(((lg - la).abs() / la.abs()).max().item())
    same = int(direct["best_idx"].item()) == int(g["best_idx"].item())
    flops = 2.0 * M * K * K + G * 4.0 * N * K * K
    log(f"gram-form search: {ms:.2f} ms/layer ({direct_ms / ms:.2f}x the direct form); "
        f"max relative loss difference {rel:.2e}; same choice {same}")
    del ws
    return {"ms_per_layer": ms, "layers_per_s": 1e3 / ms, "speedup_vs_direct": direct_ms / ms,
            "contraction_flops_per_layer": flops, "max_rel_loss_diff_vs_direct": rel,
            "same_choice": same}


def bench_largest_layer(awq, dev, steps: int = 3) -> dict:
    """The search on the workloads' largest layer, the Llama-2-70B down
    projection (16384 tokens x 28672 -> 8192), INT3 and INT4, direct and
    Gram form (here 3K > M, so the Gram form costs as much as the direct)."""
    import torch

    import synth
    spec = synth.layer_spec("llama2_70b_mlp", "down")
    x_bits, w_bits, _ = synth.make_layer(spec.workload, spec.name)
    xd = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    wd = torch.from_numpy(w_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    del x_bits, w_bits
    out = {"M": spec.M, "K": spec.K, "N": spec.N}
    flops = 2.0 * spec.M * spec.N * spec.K * spec.n_grid
    for bits in spec.bits:
        for form, fn in (("direct", awq.search_scale), ("gram", awq.search_scale_gram)):
            fn(xd, wd, bits, spec.group, spec.n_grid)
            torch.cuda.synchronize()
            t0 = time.perf_counter()
            for _ in range(steps):
                r = fn(xd, wd, bits, spec.group, spec.n_grid)
            torch.cuda.synchronize()
            ms = (time.perf_counter() - t0) * 1e3 / steps
            out[f"int{bits}_{form}"] = {"ms_per_layer": ms, "layers_per_s": 1e3 / ms,
                                        "best_idx": int(r["best_idx"].item())}
            extra = f", {flops / (ms * 1e-3) / 1e12:.0f} TFLOP/s in the candidate products" \
                if form == "direct" else ""
            log(f"largest layer (Llama-2-70B down) INT{bits} {form}: {ms:.1f} ms/layer{extra}; "
                f"alpha index {out[f'int{bits}_{form}']['best_idx']}")
    del xd, wd
    torch.cuda.empty_cache()
    return out


def bench_workload_layers(awq, dev, workload: str, names, steps: int = 2) -> dict:
    """The search over the layers of one workload, each on its own synthetic
    inputs, reported per layer and in total.  A down projection's input
    H = silu(X . Wg^T) * (X . Wu^T), from its gate/up layer's inputs and
    unquantized weights, is formed in fp64 on the GPU (torch) and rounded to
    bf16, the generator's own formula, so the host does not spend a minute
    on it."""
    import torch

    import synth
    res, total, sources = {}, 0.0, {}
    for name in names:
        spec = synth.layer_spec(workload, name)
        w_bits = synth.make_weight(spec, 0)
        wd = torch.from_numpy(w_bits.view(np.int16)).to(dev).view(torch.bfloat16)
        if spec.x_kind == "silu_gate_up":
            xg, wg = sources.pop(spec.source)
            F = spec.K
            xd = torch.empty((spec.M, F), dtype=torch.bfloat16, device=dev)
            for r0 in range(0, spec.M, 8192):
                xc = xg[r0:r0 + 8192].double()
                g = xc @ wg[:F].double().T
                u = xc @ wg[F:].double().T
                xd[r0:r0 + 8192] = (g * torch.sigmoid(g) * u).float().to(torch.bfloat16)
                del xc, g, u
        else:
            x_bits = synth.make_activations(spec, seed=0)
            xd = torch.from_numpy(x_bits.view(np.int16)).to(dev).view(torch.bfloat16)
            if any(synth.layer_spec(workload, n).source == name for n in names):
                sources[name] = (xd, wd)
        bits = spec.bits[-1]
        awq.search_scale(xd, wd, bits, spec.group, spec.n_grid)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(steps):
            r = awq.search_scale(xd, wd, bits, spec.group, spec.n_grid)
        torch.cuda.synchronize()
        ms = (time.perf_counter() - t0) * 1e3 / steps
        total += ms
        tflops = 2.0 * spec.M * spec.N * spec.K * spec.n_grid / (ms * 1e-3) / 1e12
        res[name] = {"M": spec.M, "K": spec.K, "N": spec.N, "bits": bits, "ms_per_layer": ms,
                     "best_idx": int(r["best_idx"].item()), "tflops_candidate_products": tflops}
        log(f"{workload} {name} ({spec.M} x {spec.K} -> {spec.N}, INT{bits}): {ms:.1f} ms/layer, "
            f"{tflops:.0f} TFLOP/s in the candidate products, alpha index {res[name]['best_idx']}")
        del xd, wd
        torch.cuda.empty_cache()
    res["ms_total"] = total
    res["per_s"] = 1e3 / total
    log(f"{workload}: {total:.1f} ms for its {len(names)} layers, {1e3 / total:.2f} per second")
    return res


def bench_pipeline(awq, dev, stream, n_blocks: int = 2, M: int = 65536, d: int = 4096,
                   F: int = 11008) -> dict:
    """The search layer after layer through synthetic feed-forward blocks at
    the Llama-2-7B widths (each block: gate_up 4096 -> 2 x 11008 and down
    11008 -> 4096 searched, the scales folded, the quantized layers run as
    deployed), plus the block ops' own kernels against HBM."""
    import torch

    import synth
    t0 = time.perf_counter()
    x0, blocks = synth.make_mlp_blocks(M, d, F, n_blocks, seed=0)
    log(f"pipeline inputs ({n_blocks} blocks, {M} tokens) in {time.perf_counter() - t0:.1f} s")
    xd = torch.from_numpy(x0.view(np.int16)).to(dev).view(torch.bfloat16)
    bd = [(torch.from_numpy(g).to(dev),
           torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16),
           torch.from_numpy(b.view(np.int16)).to(dev).view(torch.bfloat16)) for g, a, b in blocks]
    awq.quantize_mlp_blocks(xd, bd)            # warm-up
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res = awq.quantize_mlp_blocks(xd, bd)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3
    alphas = [(int(r["gate_up"]["best_idx"].item()), int(r["down"]["best_idx"].item())) for r in res]
    log(f"pipeline: {n_blocks} blocks in {ms:.1f} ms ({ms / n_blocks:.1f} ms per block, "
        f"{2 * n_blocks * 1e3 / ms:.2f} layers/s); alpha indices {alphas}")
    # The same blocks with Gram-form losses in both searches.
    awq.quantize_mlp_blocks(xd, bd, gram=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    res_g = awq.quantize_mlp_blocks(xd, bd, gram=True)
    torch.cuda.synchronize()
    ms_g = (time.perf_counter() - t0) * 1e3
    alphas_g = [(int(r["gate_up"]["best_idx"].item()), int(r["down"]["best_idx"].item()))
                for r in res_g]
    del res_g
    log(f"pipeline, Gram-form searches: {ms_g / n_blocks:.1f} ms per block "
        f"({2 * n_blocks * 1e3 / ms_g:.2f} layers/s); alpha indices {alphas_g}")
    # the block ops on their own
    gamma = bd[0][0]
    y = torch.randn((M, 2 * F), device=dev)
    yd = torch.randn((M, d), device=dev)
    t_rms = event_time_ms(lambda: awq.rmsnorm(xd, gamma), 10, stream)
    t_silu = event_time_ms(lambda: awq.silu_mul(y), 10, stream)
    t_res = event_time_ms(lambda: awq.residual_add(xd, yd), 10, stream)
    del y, yd
    gbs = lambda nbytes, t: nbytes / (t * 1e-3) / 1e9
    ops = {"rmsnorm": (4.0 * M * d + 4.0 * d, t_rms), "silu_mul": (10.0 * M * F, t_silu),
           "residual_add": (8.0 * M * d, t_res)}
    for k, (nb, t) in ops.items():
        log(f"{k}: {t * 1e3:.1f} us = {gbs(nb, t):.0f} GB/s")
    return {"blocks": n_blocks, "M": M, "d": d, "F": F, "ms": ms, "ms_per_block": ms / n_blocks,
            "layers_per_s": 2 * n_blocks * 1e3 / ms, "alpha_indices": alphas,
            "gram_form": {"ms_per_block": ms_g / n_blocks, "layers_per_s": 2 * n_blocks * 1e3 / ms_g,
                          "alpha_indices": alphas_g},
            "ops": {k: {"us": t * 1e3, "gbs": gbs(nb, t), "frac_hbm_peak": gbs(nb, t) / PEAK_HBM_GBS,
                        "bytes": nb} for k, (nb, t) in ops.items()}}


def cpu_baseline(x_bits, w_bits, spec, bits: int, m_sample: int, n_sample: int) -> dict:
    """Oracle (numpy fp64) on a token prefix x output-row prefix; each phase is
    scaled to the full layer by the dimension it is linear in.  Records the
    host's CPU model and the ROCm version beside the figure."""
    import oracle as O
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:
        threads = len(os.sched_getaffinity(0))
    xs = np.ascontiguousarray(x_bits[:m_sample])
    ws = np.ascontiguousarray(w_bits[:n_sample])
    t = {}
    t0 = time.perf_counter()
    O.search(xs, ws, bits, spec.group, spec.n_grid, loss_form="direct", timings=t)
    wall = time.perf_counter() - t0
    M, N = spec.M, spec.N
    full = (t["stats_and_scales"] * (M / m_sample) + t["quantize"] * (N / n_sample) +
            t["loss"] * (M / m_sample) * (N / n_sample) + t["final_pack"] * (N / n_sample))
    info = host_info()
    return {"value": 1.0 / full, "unit": "layers/s", "cores": int(threads), "kind": "oracle",
            "sample": (f"full {spec.n_grid}-point INT{bits} search on the first {m_sample} tokens x "
                       f"first {n_sample} output rows (K={spec.K}) in {wall:.1f} s; phases scaled "
                       f"to M={M}, N={N} (stats by M, quantize by N, loss by M*N)"),
            "seconds_sample": wall, "seconds_full_layer_est": full,
            "cpu_model": info["cpu_model"], "host_threads": info["host_threads"],
            "rocm": info["rocm"]}


def host_info() -> dict:
    """CPU model, host threads and the ROCm / torch versions of this run."""
    info = {"cpu_model": None, "host_threads": len(os.sched_getaffinity(0)), "rocm": None}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    info["cpu_model"] = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    try:
        with open("/opt/rocm/.info/version") as f:
            info["rocm"] = f.read().strip()
    except OSError:
        pass
    try:
        import torch
        info["torch"] = torch.__version__
        info["torch_hip"] = torch.version.hip
    except Exception:
        pass
    return info


def to_dev(bits: np.ndarray, dev):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def time_search(awq, xd, wd, bits: int, spec, steps: int, warmup: int = 1, ws=None):
    """Wall time per layer of awq_search_scale (device-synchronised)."""
    import torch
    out = None
    for _ in range(warmup):
        out = awq.search_scale(xd, wd, bits, spec.group, spec.n_grid, workspace=ws)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        out = awq.search_scale(xd, wd, bits, spec.group, spec.n_grid, workspace=ws)
    torch.cuda.synchronize()
    return (time.perf_counter() - t0) * 1e3 / steps, out


def bench_qkv_layer(awq, dev, stream, steps: int, reps: int, with_gram: bool) -> dict:
    """The Llama-2-7B fused QKV layer (65536 tokens x 4096 -> 12288, INT4):
    the search, its contraction, and the Gram-form search (which pays here,
    since 2K < M)."""
    import torch

    import synth
    spec = synth.layer_spec("llama2_7b_qkv")
    x_bits, w_bits, _ = synth.make_layer(spec.workload, spec.name)
    xd, wd = to_dev(x_bits, dev), to_dev(w_bits, dev)
    del x_bits, w_bits
    ms, out = time_search(awq, xd, wd, 4, spec, steps, warmup=2)
    M, K, N, G = spec.M, spec.K, spec.N, spec.n_grid
    s_all, inv_all = awq.candidate_scales(out["mean_abs"], G)
    d_mid = awq.diff_operand(wd, s_all[G // 2], inv_all[G // 2], 4, spec.group)
    gws = torch.empty(max(awq.workspace_size(awq.OP_W4A16_GEMM, M, N, K), 256), dtype=torch.uint8,
                      device=dev)
    t_sse = event_time_ms(lambda: awq.candidate_sse(xd, d_mid, None, workspace=gws), reps, stream)
    flops = 2.0 * M * N * K
    res = {"M": M, "K": K, "N": N, "bits": 4, "ms_per_layer": ms, "layers_per_s": 1e3 / ms,
           "best_idx": int(out["best_idx"].item()),
           "search_contraction": {"ms": t_sse, "tflops": flops / (t_sse * 1e-3) / 1e12,
                                  "frac_mfma_peak": flops / (t_sse * 1e-3) / 1e12 / PEAK_BF16_TFLOPS}}
    log(f"llama2_7b_qkv search: {ms:.2f} ms/layer ({1e3 / ms:.2f} layers/s); contraction "
        f"{t_sse:.3f} ms = {res['search_contraction']['tflops']:.0f} TFLOP/s")
    del d_mid, gws
    torch.cuda.empty_cache()
    if with_gram:
        res["gram_form"] = bench_gram(awq, xd, wd, spec, 4, out, steps, ms)
    del xd, wd, out
    torch.cuda.empty_cache()
    return res


def main() -> int:
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default=HEADLINE[0])
    ap.add_argument("--layer", default=HEADLINE[1])
    ap.add_argument("--bits", type=int, default=HEADLINE[2])
    ap.add_argument("--kernel-reps", type=int, default=10)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true", help="skip the decode-shaped GEMM figures")
    ap.add_argument("--no-gram", action="store_true", help="skip the Gram-form search figure")
    ap.add_argument("--no-pipeline", action="store_true",
                    help="skip the layer-by-layer block pipeline figure")
    ap.add_argument("--no-power-probe", action="store_true",
                    help="skip the constant-operand launch (keeps profiles to the synthetic data)")
    ap.add_argument("--no-variants", action="store_true",
                    help="only the headline layer and its kernels (for profiler runs)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode-shaped GEMM figures (prints them as JSON)")
    ap.add_argument("--no-largest", action="store_true",
                    help="skip the searches on the other workload layers")
    ap.add_argument("--decode-case", default=None, metavar="LAYER:M",
                    help="only one decode case of the Llama-3-8B block, e.g. gate_up:1")
    ap.add_argument("--cpu-m", type=int, default=4096)
    ap.add_argument("--cpu-n", type=int, default=2048)
    ap.add_argument("--summarize-trace", metavar="DIR", default=None,
                    help="write a summary of a rocprofv3 --kernel-trace --stats run and exit")
    ap.add_argument("--summarize-pmc", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                    help="write HBM bytes per dispatch from FETCH_SIZE / WRITE_SIZE runs and exit")
    ap.add_argument("--summarize-mfma", metavar="PMC_DIR", default=None,
                    help="write clock / matrix-core occupancy from a counter pass and exit")
    ap.add_argument("--summarize-counters", nargs="+", metavar="PMC_DIR", default=None,
                    help="write per-kernel medians of the counters of --pmc runs and exit")
    ap.add_argument("--bench-log", default=None, help="log of the profiled bench run")
    ap.add_argument("--profile-command", default="", help="command text recorded in a summary")
    ap.add_argument("--summary-out", default=None)
    args = ap.parse_args()

    if args.summarize_trace or args.summarize_pmc or args.summarize_mfma or args.summarize_counters:
        import synth
        spec = synth.layer_spec(args.workload, args.layer)
        if args.summarize_counters:
            text = summarize_counters(args.summarize_counters, args.profile_command)
        elif args.summarize_mfma:
            text = summarize_mfma(args.summarize_mfma, args.profile_command)
        elif args.summarize_trace:
            text = summarize_trace(args.summarize_trace, args.profile_command, args.bench_log)
        else:
            text = summarize_pmc(*args.summarize_pmc, args.profile_command, spec.M, spec.K)
        if args.summary_out:
            with open(args.summary_out, "w") as f:
                f.write(text)
        print(text, end="")
        return 0

    if args.gpus != 1:
        print(json.dumps({"error": "this implementation runs on one GPU; --gpus must be 1",
                          "n_gpus": args.gpus}))
        return 2

    import torch

    import post_weight_quantization_stats_amd as awq
    import synth

    dev = torch.device("cuda:0")
    if args.decode_case:
        # One decode case only (for a profiler run): layer name and token count.
        st = torch.cuda.current_stream(dev)
        name, m = args.decode_case.split(":")
        print(json.dumps({"int4": bench_decode(awq, dev, st, layers=(name,),
                                               token_counts=(int(m),))}), flush=True)
        return 0
    if args.decode_only:
        st = torch.cuda.current_stream(dev)
        print(json.dumps({"int4": bench_decode(awq, dev, st), "int3": bench_decode_int3(awq, dev, st)}),
              flush=True)
        return 0
    spec = synth.layer_spec(args.workload, args.layer)
    bits = args.bits
    if bits not in spec.bits:
        raise SystemExit(f"{spec.workload}/{spec.name} is quantized to {spec.bits} bits")
    M, K, N, G = spec.M, spec.K, spec.N, spec.n_grid
    log(f"workload {spec.workload}/{spec.name}: M={M} K={K} N={N} bits={bits} grid={G}")
    t0 = time.perf_counter()
    x_bits, w_bits, _ = synth.make_layer(spec.workload, spec.name)
    log(f"synthetic inputs in {time.perf_counter() - t0:.1f} s")
    xd, wd = to_dev(x_bits, dev), to_dev(w_bits, dev)
    ws_bytes = awq.workspace_size(awq.OP_SEARCH_SCALE, M, N, K, bits, spec.group, G)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream(dev)

    # Calibration copy of known size for scaling the FETCH_SIZE / WRITE_SIZE
    # counters: reads 2*M*K bytes of bf16, writes 4*M*K bytes of fp32.
    calib = xd.to(torch.float32)
    torch.cuda.synchronize()
    log(f"calibration copy: read {2 * M * K} B, write {4 * M * K} B")
    del calib

    log(f"warmup {args.warmup}")
    out = None
    for _ in range(args.warmup):
        out = awq.search_scale(xd, wd, bits, spec.group, G, workspace=ws)
    torch.cuda.synchronize()
    log(f"timing {args.steps} steps")
    t0 = time.perf_counter()
    for _ in range(args.steps):
        out = awq.search_scale(xd, wd, bits, spec.group, G, workspace=ws)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_per_step = elapsed * 1e3 / args.steps
    log(f"search: {ms_per_step:.2f} ms/layer; alpha*={int(out['best_idx'].item()) / G:.2f}")

    # ---- per-kernel durations (HIP events on the launch stream) ----
    reps = args.kernel_reps
    mean_abs = awq.act_stats(xd)
    s_all, inv_all = awq.candidate_scales(mean_abs, G)
    i_mid = G // 2
    d_mid = awq.diff_operand(wd, s_all[i_mid], inv_all[i_mid], bits, spec.group)
    gemm_ws = torch.empty(max(awq.workspace_size(awq.OP_W4A16_GEMM, M, N, K), 256),
                          dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()
    t_sse = event_time_ms(lambda: awq.candidate_sse(xd, d_mid, None, workspace=gemm_ws), reps,
                          stream)
    flops = 2.0 * M * N * K
    tf = lambda ms: flops / (ms * 1e-3) / 1e12
    log(f"search contraction {t_sse:.3f} ms = {tf(t_sse):.1f} TFLOP/s")
    kern = {"search_contraction": None}
    if not args.no_variants:
        # The vendor library's plain bf16 GEMM on the same operands (hipBLASLt
        # via torch.mm, bf16 out): a yardstick, not part of the path.
        d_t = d_mid.t().contiguous()
        y_mm = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        t_mm = event_time_ms(lambda: torch.mm(xd, d_t, out=y_mm), max(2, reps // 2), stream)
        del d_t, y_mm
        # The same launch on constant operands: identical instructions and
        # memory traffic, almost no bit toggling in the matrix cores.
        t_sse_c = None
        if not args.no_power_probe:
            x_one, d_one = torch.ones_like(xd), torch.ones_like(d_mid)
            t_sse_c = event_time_ms(lambda: awq.candidate_sse(x_one, d_one, None, workspace=gemm_ws),
                                    max(2, reps // 2), stream)
            del x_one, d_one
        qw, sc, ze = awq.quantize_pack(wd, s_all[i_mid], bits, spec.group)
        b_mid = awq.dequant_operand(wd, s_all[i_mid], inv_all[i_mid], bits, spec.group)
        yref = awq.reference_gemm(xd, wd)
        t_sse_y = event_time_ms(lambda: awq.candidate_sse(xd, b_mid, yref, workspace=gemm_ws),
                                max(2, reps // 2), stream)
        t_w4 = event_time_ms(lambda: awq.w4a16_gemm(xd, qw, sc, ze, bits, spec.group,
                                                    inv_s=inv_all[i_mid], y_ref=yref,
                                                    return_y=False, workspace=gemm_ws),
                             max(2, reps // 2), stream)
        # The same fused product on dense INT3 codes (awq_w3a16_gemm).
        qw3, sc3, ze3 = awq.quantize_pack3(wd, s_all[i_mid], spec.group)
        t_w3 = event_time_ms(lambda: awq.w4a16_gemm(xd, qw3, sc3, ze3, 3, spec.group,
                                                    inv_s=inv_all[i_mid], y_ref=yref,
                                                    return_y=False, workspace=gemm_ws,
                                                    layout=awq.LAYOUT_INT3_DENSE),
                             max(2, reps // 2), stream)
        del qw3, sc3, ze3
        t_ref = event_time_ms(lambda: awq.reference_gemm(xd, wd), max(2, reps // 2), stream)
        del yref, b_mid
        torch.cuda.empty_cache()
        log(f"against y_ref {t_sse_y:.3f} ms = {tf(t_sse_y):.1f} TFLOP/s; constant operands "
            f"{(t_sse_c or float('nan')):.3f} ms; hipBLASLt bf16 mm {t_mm:.3f} ms = "
            f"{tf(t_mm):.1f} TFLOP/s; packed w4a16+sse {t_w4:.3f} ms = {tf(t_w4):.1f} TFLOP/s "
            f"(dense INT3 {t_w3:.3f} ms = {tf(t_w3):.1f} TFLOP/s); "
            f"reference {t_ref:.3f} ms = {tf(t_ref):.1f} TFLOP/s")
    t_stats = event_time_ms(lambda: awq.act_stats(xd), reps, stream)
    t_quant = event_time_ms(lambda: awq.quantize_pack(wd, s_all[i_mid], bits, spec.group),
                            reps * 5, stream)
    t_deq = event_time_ms(lambda: awq.dequant_operand(wd, s_all[i_mid], inv_all[i_mid], bits,
                                                      spec.group), reps * 5, stream)
    t_diff = event_time_ms(lambda: awq.diff_operand(wd, s_all[i_mid], inv_all[i_mid], bits,
                                                    spec.group), reps * 5, stream)
    # Yardstick for the read-and-write kernels: a plain device copy (torch)
    # moving as many bytes as the difference operand's kernel (read W, write D).
    cp_src, cp_dst = wd.clone(), torch.empty_like(wd)
    t_copy = event_time_ms(lambda: cp_dst.copy_(cp_src), reps * 5, stream)
    del cp_src, cp_dst
    ceil = measure_ceilings(awq, dev, stream, wd)
    stats_bytes = 2.0 * M * K + 4.0 * K
    quant_bytes = 2.0 * N * K + 4.0 * K + N * K / 2 + 5.0 * N * K / spec.group
    deq_bytes = 2.0 * N * K + 8.0 * K + 2.0 * N * K
    gbs = lambda nbytes, ms: nbytes / (ms * 1e-3) / 1e9
    log(f"stats {t_stats * 1e3:.1f} us = {gbs(stats_bytes, t_stats):.0f} GB/s; quantize+pack "
        f"{t_quant * 1e3:.1f} us = {gbs(quant_bytes, t_quant):.0f} GB/s; dequant operand "
        f"{t_deq * 1e3:.1f} us = {gbs(deq_bytes, t_deq):.0f} GB/s; difference operand "
        f"{t_diff * 1e3:.1f} us = {gbs(deq_bytes, t_diff):.0f} GB/s; plain device copy of W "
        f"{t_copy * 1e3:.1f} us = {gbs(4.0 * N * K, t_copy):.0f} GB/s")

    def mfma_entry(ms):
        return {"ms": ms, "tflops": tf(ms), "frac_mfma_peak": tf(ms) / PEAK_BF16_TFLOPS,
                "frac_measured_mfma": tf(ms) / ceil["mfma_bf16_tflops"]}

    def hbm_entry(nbytes, ms, ceiling="copy_gbs"):
        return {"us": ms * 1e3, "gbs": gbs(nbytes, ms), "frac_hbm_peak": gbs(nbytes, ms) / PEAK_HBM_GBS,
                "frac_measured_ceiling": gbs(nbytes, ms) / ceil[ceiling], "ceiling": ceiling,
                "bytes": nbytes}

    kern = {"search_contraction": mfma_entry(t_sse)}
    if not args.no_variants:
        kern.update({
            "candidate_sse_vs_yref": mfma_entry(t_sse_y),
            "search_contraction_constant_operands": mfma_entry(t_sse_c) if t_sse_c else None,
            "vendor_bf16_gemm_same_shape": mfma_entry(t_mm),
            "w4a16_gemm_sse": mfma_entry(t_w4),
            "w3a16_gemm_sse": mfma_entry(t_w3),
            "reference_gemm": mfma_entry(t_ref)})
    kern.update({
        "act_stats": hbm_entry(stats_bytes, t_stats, "read_gbs"),
        "quantize_pack": hbm_entry(quant_bytes, t_quant),
        "dequant_operand": hbm_entry(deq_bytes, t_deq),
        "diff_operand": hbm_entry(deq_bytes, t_diff),
        "device_copy_same_bytes": hbm_entry(4.0 * N * K, t_copy)})
    result = {
        "metric": METRIC,
        "value": 1e3 / ms_per_step,
        "unit": "layers/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"{spec.workload}/{spec.name}", "M": M, "K": K, "N": N,
                   "bits": bits, "group": spec.group, "n_grid": G},
        "roofline": {"bound": "mfma", "achieved": tf(t_sse), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": tf(t_sse) / PEAK_BF16_TFLOPS,
                     "traffic": committed_traffic(spec.workload, spec.name),
                     "kernel": "per-candidate contraction X.D^T (D = B - W) with fused sum of squares",
                     "flops_per_launch": flops, "ms_per_launch": t_sse,
                     "algorithmic_bytes_per_launch": 2.0 * M * K + 2.0 * N * K,
                     "kernel_source_hash": gemm_source_hash(),
                     "measured_peak": ceil["mfma_bf16_tflops"],
                     "frac_measured_peak": tf(t_sse) / ceil["mfma_bf16_tflops"]},
        "ceilings": ceil,
        "kernels": kern,
        "host": host_info(),
        "cpu_baseline": None,
    }
    del d_mid, gemm_ws
    torch.cuda.empty_cache()
    result["variants"] = {}
    if not args.no_variants:
        other = [b for b in spec.bits if b != bits]
        for b in other:
            ms_b, out_b = time_search(awq, xd, wd, b, spec, args.steps, ws=None)
            result["variants"][f"search_{spec.workload}_{spec.name}_int{b}"] = {
                "ms_per_layer": ms_b, "layers_per_s": 1e3 / ms_b,
                "best_idx": int(out_b["best_idx"].item()),
                "tflops_candidate_products": flops * G / (ms_b * 1e-3) / 1e12}
            log(f"{spec.workload}/{spec.name} INT{b} search: {ms_b:.2f} ms/layer "
                f"({1e3 / ms_b:.2f} layers/s)")
            del out_b
    del ws, xd, wd, out
    torch.cuda.empty_cache()
    if not args.no_decode and not args.no_variants:
        result["kernels"]["decode_gemm_llama3_8b"] = bench_decode(awq, dev, stream)
        result["kernels"]["decode_gemm_int3_llama2_70b"] = bench_decode_int3(awq, dev, stream)
    if not args.no_variants:
        result["variants"]["search_llama2_7b_qkv"] = bench_qkv_layer(
            awq, dev, stream, args.steps, reps, not args.no_gram)
        torch.cuda.empty_cache()
    if not args.no_pipeline and not args.no_variants:
        result["variants"]["block_pipeline_llama2_7b_mlp"] = bench_pipeline(awq, dev, stream)
        torch.cuda.empty_cache()
    if not args.no_largest and not args.no_variants:
        result["variants"]["search_llama2_7b_mlp"] = bench_workload_layers(
            awq, dev, "llama2_7b_mlp", ("gate_up", "down"))
        result["variants"]["search_llama3_8b_block"] = bench_workload_layers(
            awq, dev, "llama3_8b_block", ("qkv", "o_proj", "gate_up", "down"))
        result["variants"]["search_llama2_70b_down"] = bench_largest_layer(awq, dev)
    if not args.no_cpu_baseline:
        log(f"cpu baseline: oracle on {args.cpu_m} tokens x {args.cpu_n} rows")
        result["cpu_baseline"] = cpu_baseline(x_bits, w_bits, spec, bits, args.cpu_m, args.cpu_n)
    print(json.dumps(result), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
