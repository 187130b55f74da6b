"""Pins for the CPU oracle: closed forms, invariants, special cases, library
routines and brute force, each independent of the oracle's own code.

Citations are to the pages by address and section:
  builderai.tools AWQ page ("About"), robotsatlas.com AWQ page ("How it works",
  "Key mechanisms", "Components", "Hyperparameters", "Computational
  complexity", "Benchmark notes"), vectordb.ever.works AWQ page ("Features",
  "Comparison"), aquanode.io "What is AWQ?" ("The core idea").
"""

import json
import math
import os
import struct

import numpy as np
import pytest

import oracle as O
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def bits_of(values):
    """bf16 patterns of values that are exactly representable in bf16."""
    v = np.asarray(values, dtype=np.float32)
    u = v.view(np.uint32)
    assert np.all((u & 0xFFFF) == 0), "value not exactly bf16"
    return (u >> 16).astype(np.uint16)


# ---------------------------------------------------------------- pure Python

def py_f32(x: float) -> float:
    return struct.unpack("<f", struct.pack("<f", x))[0]


def py_bf16(x: float) -> float:
    """RNE to bf16 by integer arithmetic on the fp32 pattern (not the oracle's method)."""
    u = struct.unpack("<I", struct.pack("<f", x))[0]
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return struct.unpack("<f", struct.pack("<I", (u << 16) & 0xFFFFFFFF))[0]


def py_rint(x: float) -> float:
    f = math.floor(x)
    d = x - f
    if d > 0.5 or (d == 0.5 and f % 2 == 1):
        f += 1
    return float(f)


def py_search(X, W, bits, group, n_grid):
    """The whole search in pure Python loops on lists of floats (tiny sizes)."""
    M, K, N = len(X), len(X[0]), len(W)
    qmax = (1 << bits) - 1
    a = [py_f32(sum(abs(X[m][k]) for m in range(M)) / M) for k in range(K)]
    losses, S = [], []
    for i in range(n_grid):
        alpha = i / n_grid
        r = [max(a[k] ** alpha, 1e-4) for k in range(K)]
        c = math.sqrt(max(r) * min(r))
        s = [py_f32(r[k] / c) for k in range(K)]
        inv = [py_f32(1.0 / s[k]) for k in range(K)]
        S.append(s)
        B = [[0.0] * K for _ in range(N)]
        for n in range(N):
            for g0 in range(0, K, group):
                ws = [py_f32(W[n][k] * s[k]) for k in range(g0, g0 + group)]
                mx, mn = max(max(ws), 0.0), min(min(ws), 0.0)
                step = py_f32(py_f32(mx - mn) / qmax)
                if step == 0.0:
                    step = 1.0
                z = min(max(py_rint(py_f32(-mn / step)), 0.0), qmax)
                for j, k in enumerate(range(g0, g0 + group)):
                    q = min(max(py_rint(py_f32(ws[j] / step)) + z, 0.0), qmax)
                    B[n][k] = py_bf16(py_f32(py_f32((q - z) * step) * inv[k]))
        sse = 0.0
        for m in range(M):
            for n in range(N):
                yq = math.fsum(X[m][k] * B[n][k] for k in range(K))
                y = math.fsum(X[m][k] * W[n][k] for k in range(K))
                sse += (yq - y) ** 2
        losses.append(sse / (M * N))
    best = min(range(n_grid), key=lambda i: (losses[i], i))
    return a, S, losses, best


# ------------------------------------------------------------ number formats

def test_bf16_rounding_matches_torch_cast():
    """Library-routine pin: the oracle's bf16 RNE equals torch's CPU cast."""
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(1)
    hi = np.arange(1 << 16, dtype=np.uint32) << 16
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], dtype=np.uint32)
    edge = (hi[:, None] | lows[None, :]).ravel()
    rand = rng.integers(0, 1 << 32, size=1 << 22, dtype=np.uint64).astype(np.uint32)
    u = np.concatenate([edge, rand])
    x = u.view(np.float32)
    finite = np.isfinite(x)
    got = O.bf16_rne_bits(x[finite])
    ref = torch.from_numpy(x[finite].copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    # NaN stays NaN
    assert np.isnan(O.bf16_round(np.array([np.nan], np.float32)))[0]


def test_bf16_rounding_matches_integer_rne():
    """Second method: integer RNE on the fp32 pattern, pure Python."""
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(3000) * 10.0 ** rng.integers(-6, 6, 3000)).astype(np.float32)
    got = O.bf16_round(x)
    ref = np.array([py_bf16(float(v)) for v in x])
    assert np.array_equal(got, ref)


def test_f32_ops_match_numpy_float32():
    """Library-routine pin: fp64-evaluate-then-round equals numpy's fp32 ops."""
    rng = np.random.default_rng(3)
    a = (rng.standard_normal(200000) * 10.0 ** rng.integers(-8, 8, 200000)).astype(np.float32)
    b = (rng.standard_normal(200000) * 10.0 ** rng.integers(-8, 8, 200000)).astype(np.float32)
    b[b == 0] = 1.0
    A, B = a.astype(np.float64), b.astype(np.float64)
    assert np.array_equal(O.f32(A / B), (a / b).astype(np.float64))
    assert np.array_equal(O.f32(A * B), (a * b).astype(np.float64))
    assert np.array_equal(O.f32(A - B), (a - b).astype(np.float64))


# ------------------------------------------------------------- stats (step 1)

def test_stats_closed_form_constant_columns():
    """Constant column c gives mean |x| = |c|; +-c alternation too."""
    cols = np.array([0.5, -3.0, 0.0, 1.25, -0.0078125, 96.0, 2.0, -2.0], np.float32)
    M = 64
    X = np.tile(cols, (M, 1))
    X[1::2, 6] *= -1  # alternating signs
    a64, a32 = O.act_stats(bits_of(X))
    assert np.array_equal(a32, np.abs(cols).astype(np.float64))


def test_stats_row_permutation_and_power_of_two_scaling():
    x, _ = synth.random_layer(96, 256, 8, seed=4, n_outlier=3)
    _, a = O.act_stats(x)
    perm = np.random.default_rng(5).permutation(96)
    _, ap = O.act_stats(x[perm])
    assert np.array_equal(a, ap)
    x4 = bits_of(synth.bf16_bits_to_f32(x) * np.float32(4.0))
    _, a4 = O.act_stats(x4)
    assert np.array_equal(a4, 4.0 * a)


def test_stats_brute_force():
    x, _ = synth.random_layer(17, 128, 8, seed=6)
    X = synth.bf16_bits_to_f32(x).astype(np.float64)
    ref = [py_f32(math.fsum(abs(X[m, k]) for m in range(17)) / 17) for k in range(128)]
    assert np.array_equal(O.act_stats(x)[1], np.array(ref))


# ------------------------------------------------------ candidates (step 2)

def test_alpha_grid_and_alpha0_is_identity():
    """alpha = i/20 over [0,1): includes 0 (plain rounding), excludes 1."""
    g = O.alpha_grid(20)
    assert g[0] == 0.0 and g[-1] == 0.95 and len(g) == 20
    a = np.array([0.3, 2.0, 7.5, 0.0], dtype=np.float64)
    s, inv = O.candidate_scales(a, 20)
    assert np.all(s[0] == 1.0) and np.all(inv[0] == 1.0)


def test_candidates_closed_form():
    """a = [1, 4], alpha = 1/2: r = [1, 2], s = r / sqrt(2)."""
    s, inv = O.candidate_scales(np.array([1.0, 4.0]), 2)
    assert s[1, 0] == py_f32(1.0 / math.sqrt(2.0))
    assert s[1, 1] == py_f32(2.0 / math.sqrt(2.0))
    assert inv[1, 1] == py_f32(1.0 / s[1, 1])


def test_candidates_floor_on_dead_channel():
    s, inv = O.candidate_scales(np.array([0.0, 1.0, 100.0]), 4)
    # alpha = 0.5: r = [1e-4, 1, 10]; normaliser sqrt(10 * 1e-4) = 0.1
    assert s[2, 0] == py_f32(1e-4 / math.sqrt(10.0 * 1e-4))
    assert s[2, 2] == py_f32(10.0 / math.sqrt(10.0 * 1e-4))
    assert np.all(np.isfinite(inv))


def test_candidates_invariant_under_activation_scaling():
    """X -> 2^p X leaves s unchanged: the normaliser removes 2^(p alpha)."""
    rng = np.random.default_rng(7)
    a = O.f32(np.abs(rng.standard_normal(4096)) + 0.05)
    s1, _ = O.candidate_scales(a, 20)
    s2, _ = O.candidate_scales(a * 8.0, 20)
    rel = np.abs(s1 - s2) / s1
    assert rel.max() <= 2.0 ** -23
    assert np.mean(s1 == s2) > 0.999


def test_candidates_normalised_and_monotone():
    rng = np.random.default_rng(8)
    a = O.f32(np.abs(rng.standard_normal(512)) + 0.01)
    s, _ = O.candidate_scales(a, 20)
    for i in range(1, 20):
        assert abs(s[i].max() * s[i].min() - 1.0) < 1e-6
        order = np.argsort(a, kind="stable")
        assert np.all(np.diff(s[i][order]) >= 0)


# ------------------------------------------------------ quantizer (step 3)

def test_quantizer_worked_group():
    with open(os.path.join(GOLDEN, "quant_group_worked.json")) as f:
        g = json.load(f)
    vals = np.full(g["group"], g["tail_value"], np.float32)
    vals[:len(g["values_head"])] = g["values_head"]
    q, z, step = O.quantize(bits_of(vals[None, :]), None, g["bits"], g["group"])
    assert step[0, 0] == g["expected_step"]
    assert z[0, 0] == g["expected_zero"]
    assert list(q[0, :8]) == g["expected_codes_head"]
    assert np.all(q[0, 8:] == g["expected_code_tail"])


@pytest.mark.parametrize("bits", [3, 4])
def test_quantizer_codes_range_and_half_step_bound(bits):
    """Codes in [0, qmax]; |ws - (q - z) step| <= step/2 (plus one fp32 rounding)."""
    x, w = synth.random_layer(64, 512, 48, seed=9, n_outlier=5)
    _, a = O.act_stats(x)
    s, _ = O.candidate_scales(a, 20)
    qmax = (1 << bits) - 1
    W = O.bf16_bits_to_f64(w)
    for i in (0, 7, 19):
        q, z, step = O.quantize(w, s[i], bits, 128)
        assert q.min() >= 0 and q.max() <= qmax and z.min() >= 0 and z.max() <= qmax
        ws = O.f32(W * s[i][None, :])
        st = np.repeat(step, 128, axis=1)
        err = np.abs(ws - (q - np.repeat(z, 128, axis=1)) * st)
        assert np.all(err <= st / 2 * (1 + 2.0 ** -20))


def test_quantizer_brute_force_nearest_grid_point():
    """Each code is the nearest of the qmax+1 levels to ws/step + z (ties: even rint)."""
    x, w = synth.random_layer(32, 256, 12, seed=10, n_outlier=2)
    s = O.candidate_scales(O.act_stats(x)[1], 20)[0][13]
    for bits in (3, 4):
        qmax = (1 << bits) - 1
        q, z, step = O.quantize(w, s, bits, 128)
        W = synth.bf16_bits_to_f32(w).astype(np.float64)
        for n in range(12):
            for g in range(2):
                ws = [py_f32(W[n, k] * s[k]) for k in range(128 * g, 128 * g + 128)]
                st, zz = step[n, g], z[n, g]
                for j, v in enumerate(ws):
                    t = py_f32(v / st)
                    best = min(range(qmax + 1),
                               key=lambda c: (abs(t - (c - zz)), (c - zz) % 2))
                    assert q[n, 128 * g + j] == best


def test_quantizer_special_groups():
    """All-zero group: step 1, codes = zero = 0.  All-positive group: zero 0."""
    vals = np.zeros((2, 128), np.float32)
    vals[1] = np.linspace(0.5, 3.0, 128, dtype=np.float32)
    vals[1] = synth.bf16_bits_to_f32(synth.to_bf16_bits(vals[1]))
    q, z, step = O.quantize(synth.to_bf16_bits(vals), None, 4, 128)
    assert step[0, 0] == 1.0 and z[0, 0] == 0 and np.all(q[0] == 0)
    # all-positive: the range runs from 0 to the max, so step = max / 15
    assert z[1, 0] == 0 and q[1].max() == 15
    assert step[1, 0] == py_f32(float(vals[1].max()) / 15.0)
    assert np.all(np.abs(vals[1] - q[1] * step[1, 0]) <= step[1, 0] / 2)


def test_quantizer_power_of_two_weight_scaling():
    _, w = synth.random_layer(8, 256, 16, seed=11)
    q1, z1, st1 = O.quantize(w, None, 4, 128)
    w2 = bits_of(synth.bf16_bits_to_f32(w) * np.float32(0.25))
    q2, z2, st2 = O.quantize(w2, None, 4, 128)
    assert np.array_equal(q1, q2) and np.array_equal(z1, z2)
    assert np.array_equal(st2, st1 * 0.25)


def test_quantizer_group_min_maps_to_zero_code():
    _, w = synth.random_layer(8, 256, 16, seed=12)
    q, z, _ = O.quantize(w, None, 4, 128)
    W = synth.bf16_bits_to_f32(w).reshape(16, 2, 128)
    qq = q.reshape(16, 2, 128)
    idx = W.argmin(axis=2)
    assert np.all(np.take_along_axis(qq, idx[:, :, None], 2) == 0)


# ---------------------------------------------------------------- packing

def test_pack_worked_and_roundtrip():
    with open(os.path.join(GOLDEN, "pack_worked.json")) as f:
        g = json.load(f)
    q = np.array([g["codes"]], np.int64)
    words, _, _ = O.pack(q, np.zeros((1, 1), np.int64), np.ones((1, 1)))
    assert [hex(int(v)) for v in words[0]] == g["expected_words_hex"]
    rng = np.random.default_rng(13)
    q = rng.integers(0, 16, size=(7, 256))
    assert np.array_equal(O.unpack(O.pack(q, np.zeros((7, 2)), np.ones((7, 2)))[0]), q)


def test_pack3_worked_words():
    with open(os.path.join(GOLDEN, "pack3_worked.json")) as f:
        g = json.load(f)
    q = np.array(g["codes"], dtype=np.int64)[None, :]
    words = O.pack3(q)
    assert [hex(int(x)) for x in words[0]] == g["expected_words_hex"]
    assert np.array_equal(O.unpack3(words), q)


def test_pack3_big_integer_brute_force():
    """Each 32-code run as one Python integer, built code by code."""
    rng = np.random.default_rng(31)
    q = rng.integers(0, 8, size=(7, 256))
    words = O.pack3(q)
    assert words.shape == (7, 24) and words.dtype == np.uint32
    for n in range(7):
        for c in range(8):
            v = 0
            for i in range(32):
                v += int(q[n, 32 * c + i]) * 8 ** i
            assert [int(x) for x in words[n, 3 * c:3 * c + 3]] == [v % 2 ** 32, (v >> 32) % 2 ** 32,
                                                                   v >> 64]
    assert np.array_equal(O.unpack3(words), q)
    with pytest.raises(ValueError):
        O.pack3(np.full((1, 32), 8))


def test_decode_meta_brute_force():
    """Every word of the metadata tiles, found by walking the definition in
    pure Python: word r of tile b*G + g is row 16b + r's binary16 step bits
    for group g, plus its zero (the nibble of byte g // 2, low for even g)
    shifted to bit 16; rows past N give 0."""
    rng = np.random.default_rng(43)
    N, K = 37, 640
    G = K // 128
    steps16 = rng.integers(0, 2 ** 16, size=(N, G), dtype=np.uint64).astype(np.uint16)
    zeros4 = rng.integers(0, 256, size=(N, (G + 1) // 2), dtype=np.uint64).astype(np.uint8)
    zeros4[:, -1] &= 0x0F                  # G odd: the high nibble past the last group is 0
    meta = O.decode_meta(steps16, zeros4, K)
    NB = -(-N // 16)
    assert meta.dtype == np.uint32 and meta.size == NB * G * 16
    for b in range(NB):
        for g in range(G):
            for r in range(16):
                n = 16 * b + r
                want = 0
                if n < N:
                    byte = int(zeros4[n, g // 2])
                    z = (byte >> 4) if g % 2 else (byte & 15)
                    want = int(steps16[n, g]) + z * 65536
                assert int(meta[(b * G + g) * 16 + r]) == want, (b, g, r)


def test_dense_int3_storage_and_product():
    """Dense INT3 takes 3 bits per weight plus 40 bits per group (3.31 bits,
    4.83x smaller than bf16), and the product from its words equals the
    product from the 4-bit containers for the same codes."""
    assert O.packed3_bytes(64, 4096, 128) * 8 / (64 * 4096) == 3 + 40 / 128
    assert 16 / (3 + 40 / 128) == pytest.approx(4.83, abs=0.01)
    x, w = synth.random_layer(5, 256, 24, seed=17)
    q, z, st = O.quantize(w, None, 3, 128)
    qw, sc, ze = O.pack(q, z, st)
    a = x[:5]
    assert np.array_equal(O.decode_gemm3(a, O.pack3(q), sc, ze, 128), O.decode_gemm(a, qw, sc, ze, 128))


@pytest.mark.parametrize("dense3", [False, True])
def test_decode_tiles_brute_force(dense3):
    """Every byte of the tile layout, found by walking the definition in pure
    Python: tile b*G + g holds rows 16b .. 16b+15 of group g, row r's piece
    for channels 32q .. 32q+31 at byte P*(r + 16q), rows past N zero; inside
    a piece, pair p = (channel 2p, channel 2p+1) goes to nibbles (t, 4+t) of
    word j for p = 4j + t (4-bit containers) or to bits (3(p%5), 16+3(p%5))
    of word p//5, pair 15 to bits 15 and 31 of the three words (dense INT3).
    The codes are read from the packed words bit by bit."""
    rng = np.random.default_rng(41)
    N, K = 37, 384
    G, P = K // 128, (12 if dense3 else 16)
    nwords = 3 * K // 32 if dense3 else K // 8
    qw = rng.integers(0, 2 ** 32, size=(N, nwords), dtype=np.uint64).astype(np.uint32)
    if dense3:
        big = [int.from_bytes(qw[n].astype("<u4").tobytes(), "little") for n in range(N)]
        code = lambda n, k: (big[n] >> (3 * k)) & 7
    else:
        code = lambda n, k: (int(qw[n, k // 8]) >> (4 * (k % 8))) & 15
    tiles = O.decode_tiles(qw, K, dense3)
    NB = -(-N // 16)
    assert tiles.size == NB * G * 64 * P
    for b in range(NB):
        for g in range(G):
            for q in range(4):
                for r in range(16):
                    n = 16 * b + r
                    c = [code(n, 128 * g + 32 * q + i) if n < N else 0 for i in range(32)]
                    words = [0] * (P // 4)
                    for p in range(16):
                        lo, hi = c[2 * p], c[2 * p + 1]
                        if not dense3:
                            words[p // 4] |= (lo << (4 * (p % 4))) | (hi << (16 + 4 * (p % 4)))
                        elif p < 15:
                            words[p // 5] |= (lo << (3 * (p % 5))) | (hi << (16 + 3 * (p % 5)))
                        else:
                            for i in range(3):
                                words[i] |= (((lo >> i) & 1) << 15) | (((hi >> i) & 1) << 31)
                    want = b"".join(w.to_bytes(4, "little") for w in words)
                    got = tiles[(b * G + g) * 64 * P + P * (r + 16 * q):][:P].tobytes()
                    assert got == want, (b, g, q, r)


def test_storage_about_four_times_smaller():
    """~4x smaller than 16-bit and ~4.x bits per weight (vectordb 'Features',
    robotsatlas 'Computational complexity')."""
    N, K = 12288, 4096
    nbytes = O.packed_bytes(N, K, 128)
    ratio = 2 * N * K / nbytes
    bits_per_weight = 8 * nbytes / (N * K)
    assert 3.5 < ratio < 4.0 and ratio == pytest.approx(3.7101, abs=1e-3)
    assert 4.0 < bits_per_weight < 5.0 and bits_per_weight == 4.3125


# ------------------------------------------------------------- loss (step 4)

def test_scaling_preserves_product_before_rounding():
    """(W diag(s)) (X diag(1/s))^T = W X^T exactly in real arithmetic
    (robotsatlas 'How it works' / 'Components')."""
    x, w = synth.random_layer(64, 256, 32, seed=14, n_outlier=3)
    X, W = O.bf16_bits_to_f64(x), O.bf16_bits_to_f64(w)
    s = O.candidate_scales(O.act_stats(x)[1], 20)[0][11]
    Y = X @ W.T
    Ys = (X / s[None, :]) @ (W * s[None, :]).T
    assert np.max(np.abs(Ys - Y)) <= 1e-12 * np.max(np.abs(Y))


def test_loss_two_forms_and_literal_difference():
    x, w = synth.random_layer(200, 384, 40, seed=15, n_outlier=4)
    s, inv = O.candidate_scales(O.act_stats(x)[1], 20)
    G = O.gram(x)
    for i in (0, 9, 19):
        q, z, st = O.quantize(w, s[i], 4, 128)
        B = O.dequant_operand(q, z, st, 128, inv[i])
        direct = O.output_mse(x, w, B)
        g = O.output_mse_gram(G, 200, w, B)
        literal = np.mean((O.gemm(x, B) - O.gemm(x, O.bf16_bits_to_f64(w))) ** 2)
        assert g == pytest.approx(direct, rel=1e-10)
        assert literal == pytest.approx(direct, rel=1e-9)


@pytest.mark.parametrize("bits", [3, 4])
def test_difference_operand_is_exact(bits):
    """B - W needs no rounding in bf16: every nonzero B lies within a factor
    of two of W with the same sign (Sterbenz's lemma then makes the
    difference of the two bf16 values a bf16 value), and X . D^T is the
    output error against the literal products X . B^T - X . W^T."""
    x, w = synth.random_layer(96, 512, 64, seed=21, n_outlier=5, outlier_factor=30.0)
    X, W = O.bf16_bits_to_f64(x), O.bf16_bits_to_f64(w)
    s, inv = O.candidate_scales(O.act_stats(x)[1], 20)
    for i in range(20):
        q, z, st = O.quantize(w, s[i], bits, 128)
        B = O.dequant_operand(q, z, st, 128, inv[i])
        nz = B != 0
        ratio = B[nz] / W[nz]
        assert ratio.min() >= 0.5 and ratio.max() <= 2.0
        D = O.diff_operand(w, B)
        assert np.array_equal(D, B - W)
        err = X @ B.T - X @ W.T
        assert np.abs(X @ D.T - err).max() <= 1e-12 * np.abs(X @ B.T).max()


def test_difference_operand_rounds_where_inexact():
    """Away from the quantizer's grid the contract still rounds: a difference
    that needs more than 8 significant bits goes to the nearest bf16."""
    b = np.array([[1.0, 0.0, 2.0 ** -10]])
    w = synth.to_bf16_bits(np.array([[2.0 ** -9, 0.5, 1.0]], np.float32))
    D = O.diff_operand(w, b)
    assert D[0, 1] == -0.5
    assert D[0, 2] == -1.0                    # 2^-10 - 1 rounds back to -1
    assert D[0, 0] == 1.0                     # 1 - 2^-9: a tie, to the even neighbour


def rtn_mse(x_bits, w_bits, bits, group):
    """Plain round-to-nearest, written separately: no scale, per-group asymmetric
    min/max quantization in fp32 (numpy float32 arithmetic)."""
    W = synth.bf16_bits_to_f32(w_bits)
    X = synth.bf16_bits_to_f32(x_bits).astype(np.float64)
    qmax = np.float32((1 << bits) - 1)
    N, K = W.shape
    Bq = np.empty_like(W)
    for n in range(N):
        for g0 in range(0, K, group):
            v = W[n, g0:g0 + group]
            hi = max(v.max(), np.float32(0))
            lo = min(v.min(), np.float32(0))
            step = np.float32(hi - lo) / qmax
            if step == 0:
                step = np.float32(1)
            zero = np.clip(np.rint(-lo / step), 0, qmax)
            code = np.clip(np.rint(v / step) + zero, 0, qmax)
            Bq[n, g0:g0 + group] = np.float32(code - zero) * step
    Bq = synth.bf16_bits_to_f32(synth.to_bf16_bits(Bq)).astype(np.float64)
    return float(np.mean((X @ Bq.T - X @ W.astype(np.float64).T) ** 2))


@pytest.mark.parametrize("bits", [3, 4])
def test_alpha0_loss_is_plain_rtn(bits):
    x, w = synth.random_layer(128, 256, 24, seed=16, n_outlier=3)
    res = O.search(x, w, bits=bits, group=128, n_grid=20)
    assert res["losses"][0] == pytest.approx(rtn_mse(x, w, bits, 128), rel=1e-12)
    assert res["losses"].min() <= res["losses"][0]   # never worse than RTN


def test_grid_exact_weights_have_zero_rtn_loss():
    """Weights already on each group's 16-level grid quantize exactly at alpha 0."""
    rng = np.random.default_rng(17)
    N, K = 16, 256
    codes = rng.integers(0, 16, size=(N, K))
    codes[:, 0::128] = 0
    codes[:, 1::128] = 15
    W = ((codes - 5) * 2.0 ** -6).astype(np.float32)
    x, _ = synth.random_layer(64, K, 4, seed=18, n_outlier=2)
    res = O.search(x, bits_of(W), 4, 128, 20)
    assert res["losses"][0] == 0.0 and res["best_idx"] == 0
    assert np.array_equal(res["q"], codes)


def test_losses_scale_by_four_to_the_p():
    x, w = synth.random_layer(96, 256, 16, seed=19, n_outlier=3)
    r1 = O.search(x, w, 4, 128, 20)
    x2 = bits_of(synth.bf16_bits_to_f32(x) * np.float32(2.0))
    r2 = O.search(x2, w, 4, 128, 20)
    w2 = bits_of(synth.bf16_bits_to_f32(w) * np.float32(0.5))
    r3 = O.search(x, w2, 4, 128, 20)
    assert r2["best_idx"] == r1["best_idx"] == r3["best_idx"]
    assert np.allclose(r2["losses"], 4.0 * r1["losses"], rtol=1e-6, atol=0)
    assert np.array_equal(r3["losses"], r1["losses"] / 4.0)


@pytest.mark.parametrize("M,N,K,bits,seed", [(24, 8, 128, 4, 20), (16, 6, 256, 3, 21),
                                             (40, 4, 128, 4, 22)])
def test_whole_search_brute_force_tiny(M, N, K, bits, seed):
    """Every step recomputed in pure Python loops on a tiny layer."""
    x, w = synth.random_layer(M, K, N, seed=seed, n_outlier=2, outlier_factor=15.0)
    n_grid = 10
    res = O.search(x, w, bits, 128, n_grid)
    X = synth.bf16_bits_to_f32(x).astype(np.float64).tolist()
    W = synth.bf16_bits_to_f32(w).astype(np.float64).tolist()
    a, S, losses, best = py_search(X, W, bits, 128, n_grid)
    assert np.array_equal(res["mean_abs"], np.array(a))
    assert np.array_equal(res["s"], np.array(S))
    assert np.allclose(res["losses"], losses, rtol=1e-12, atol=0)
    assert res["best_idx"] == best


def test_outlier_channels_get_the_largest_scales():
    """~1% salient channels (builderai 'About', aquanode 'The core idea'): on the
    outlier recipe the search picks alpha > 0 and s peaks on the outliers."""
    x, w, spec = synth.make_layer("single_linear_512")
    res = O.search(x, w, 4, 128, 20)
    cols, _ = synth.outlier_columns(spec)
    assert res["best_idx"] > 0
    top = np.argsort(res["best_s"])[-len(cols):]
    assert set(top) == set(cols)
    assert res["losses"][res["best_idx"]] < 0.9 * res["losses"][0]


def test_first_argmin_ties_and_nan():
    assert O.first_argmin([3.0, 1.0, 1.0, 2.0]) == 1
    assert O.first_argmin([np.nan, 2.0, np.nan, 1.5]) == 3
    assert O.first_argmin([np.nan, np.nan]) == -1


# ------------------------------------------------------------ deploy GEMM

def test_deploy_gemm_exact_sums():
    x, w = synth.random_layer(5, 256, 7, seed=23)
    q, z, st = O.quantize(w, None, 4, 128)
    qw, sc, ze = O.pack(q, z, st)
    Y = O.deploy_gemm(x, qw, sc, ze, 128)
    X = synth.bf16_bits_to_f32(x).astype(np.float64)
    for m in range(5):
        for n in range(7):
            terms = []
            for k in range(256):
                d = py_bf16(py_f32((q[n, k] - z[n, k // 128]) * float(st[n, k // 128])))
                terms.append(X[m, k] * d)
            assert Y[m, n] == pytest.approx(math.fsum(terms), rel=1e-13, abs=1e-300)


# ------------------------------------------------------------ decode contraction

def test_decode_gemm_brute_force_from_words():
    """Nibbles decoded bit by bit from the packed words in pure Python; the
    dequantized weight (q - z) * step is exact in binary64."""
    rng = np.random.default_rng(31)
    M, N, K = 3, 8, 256
    x, w = synth.random_layer(M, K, N, seed=31)
    q, z, st = O.quantize(w, None, 4, 128)
    qw, sc, ze = O.pack(q, z, st)
    Y = O.decode_gemm(x, qw, sc, ze, 128)
    X = synth.bf16_bits_to_f32(x).astype(np.float64)
    words = qw.astype(np.uint64)
    for m in range(M):
        for n in range(N):
            terms = []
            for k in range(K):
                code = (int(words[n, k // 8]) >> (4 * (k % 8))) & 15
                g = k // 128
                terms.append(X[m, k] * ((code - int(ze[n, g])) * float(sc[n, g])))
            assert Y[m, n] == pytest.approx(math.fsum(terms), rel=1e-13, abs=1e-300)
    del rng


def test_decode_gemm_codes_at_zero_point_give_zero():
    M, N, K = 4, 16, 384
    x, _ = synth.random_layer(M, K, N, seed=32)
    rng = np.random.default_rng(32)
    ze = rng.integers(0, 16, size=(N, K // 128)).astype(np.uint8)
    q = np.repeat(ze.astype(np.int64), 128, axis=1)
    qw = O.pack(q, ze, np.ones((N, K // 128), np.float32))[0]
    sc = rng.uniform(0.01, 2.0, size=(N, K // 128)).astype(np.float32)
    assert np.all(O.decode_gemm(x, qw, sc, ze, 128) == 0.0)


def test_decode_gemm_unit_codes_closed_form():
    """q = z + 1 everywhere: Y[m][n] = sum_g step[n][g] * (sum of A[m] over group g)."""
    M, N, K = 5, 8, 512
    x, _ = synth.random_layer(M, K, N, seed=33)
    rng = np.random.default_rng(33)
    ze = rng.integers(0, 15, size=(N, K // 128)).astype(np.uint8)
    q = np.repeat(ze.astype(np.int64) + 1, 128, axis=1)
    qw = O.pack(q, ze, np.ones((N, K // 128), np.float32))[0]
    sc = rng.uniform(0.01, 2.0, size=(N, K // 128)).astype(np.float32)
    A = synth.bf16_bits_to_f32(x).astype(np.float64)
    colsum = A.reshape(M, K // 128, 128).sum(axis=2)            # [M][G]
    ref = colsum @ sc.astype(np.float64).T
    np.testing.assert_allclose(O.decode_gemm(x, qw, sc, ze, 128), ref, rtol=1e-13, atol=1e-12)


def test_decode_gemm_equals_deploy_when_dequant_is_bf16_exact():
    """With power-of-two steps, (q - z) * step is exact in bf16, so the exact
    decode product and the bf16-operand product coincide bit for bit."""
    M, N, K = 4, 24, 256
    x, _ = synth.random_layer(M, K, N, seed=34)
    rng = np.random.default_rng(34)
    q = rng.integers(0, 16, size=(N, K)).astype(np.int64)
    ze = rng.integers(0, 16, size=(N, K // 128)).astype(np.uint8)
    sc = np.exp2(rng.integers(-12, 4, size=(N, K // 128))).astype(np.float32)
    qw = O.pack(q, ze, sc)[0]
    assert np.array_equal(O.decode_gemm(x, qw, sc, ze, 128), O.deploy_gemm(x, qw, sc, ze, 128))


# ------------------------------------------- compact format: 16-bit steps, 4-bit zeros

def py_f16_bits(x: float) -> int:
    """binary16 pattern of x by Python's struct 'e' format (round half to even)."""
    try:
        return struct.unpack("<H", struct.pack("<e", x))[0]
    except OverflowError:
        return 0x7C00 if x > 0 else 0xFC00


def test_f16_format_against_libraries():
    """The oracle's binary16 decode and rounding, written from the format's
    definition, against numpy's float16 and Python's struct 'e' format:
    every bit pattern, random binary32 values, exact ties and the overflow
    boundary."""
    b = np.arange(65536, dtype=np.uint16)
    ref = b.view(np.float16).astype(np.float64)
    got = O.f16_bits_to_f64(b)
    assert np.all((got == ref) | (np.isnan(got) & np.isnan(ref)))
    rng = np.random.default_rng(40)
    u = rng.integers(0, 2 ** 32, size=200_000, dtype=np.uint64).astype(np.uint32)
    v = u.view(np.float32)
    v = v[~np.isnan(v)]
    with np.errstate(over="ignore"):
        assert np.array_equal(O.f16_rne_bits(v), v.astype(np.float16).view(np.uint16))
    # exact midpoints between neighbouring binary16 values (all exact in binary32)
    h = np.arange(0, 0x7BFF, dtype=np.uint16)
    lo = h.view(np.float16).astype(np.float64)
    hi = (h + 1).astype(np.uint16).view(np.float16).astype(np.float64)
    mid = ((lo + hi) / 2).astype(np.float32)
    want = np.where(h % 2 == 0, h, h + 1).astype(np.uint16)       # to the even pattern
    assert np.array_equal(O.f16_rne_bits(mid), want)
    assert np.array_equal(O.f16_rne_bits(-mid), want | np.uint16(0x8000))
    for x in (65504.0, 65519.99, 65520.0, 2.0 ** -25, 2.0 ** -25 * (1 + 2 ** -23), 3e-8, 1e-3, 0.1):
        x32 = float(np.float32(x))
        assert int(O.f16_rne_bits(np.float32(x32))) == py_f16_bits(x32), x


def _grid_layer(N, G, group, qmax, seed):
    """bf16 weights k * 2^-7 whose every group has range qmax * j * 2^-7
    (j in 1..8), so the fp32 step j * 2^-7 is a binary16 value."""
    rng = np.random.default_rng(seed)
    k = np.empty((N, G, group), np.int64)
    for n in range(N):
        for g in range(G):
            j = int(rng.integers(1, 9))
            lo = -int(rng.integers(0, qmax * j + 1))
            hi = lo + qmax * j
            k[n, g] = rng.integers(lo, hi + 1, size=group)
            k[n, g, rng.integers(0, group)] = lo
            k[n, g, rng.integers(0, group)] = hi
    return bits_of(k.reshape(N, G * group).astype(np.float32) * np.float32(2.0 ** -7))


def test_compact_worked_groups():
    """Hand-worked groups whose fp32 steps sit exactly between two binary16
    values (tests/golden/compact_worked.json): one tie goes down to an even
    fraction, the other up."""
    with open(os.path.join(GOLDEN, "compact_worked.json")) as f:
        g = json.load(f)
    K = g["K"]
    W = np.zeros((1, K), np.float32)
    for k, v in g["w_nonzero"]:
        W[0, k] = v
    s = np.ones(K, np.float32)
    for k, v in g["s_nonzero"]:
        s[k] = v
        assert float(np.float32(v)) == v
    q, z, st = O.quantize16(synth.to_bf16_bits(W), s, g["bits"], g["group"])
    sb, zb = O.pack_meta16(z, st)
    assert [hex(int(v)) for v in sb[0]] == g["expected_steps16_hex"]
    assert zb[0].tolist() == g["expected_zeros4"]
    nz = [[int(k), int(q[0, k])] for k in np.flatnonzero(q[0])]
    assert nz == g["expected_codes_nonzero"]


def test_quantize16_equals_quantize_when_steps_are_binary16():
    for bits in (3, 4):
        w = _grid_layer(6, 3, 128, (1 << bits) - 1, seed=41 + bits)
        q1, z1, st1 = O.quantize(w, None, bits, 128)
        q2, z2, st2 = O.quantize16(w, None, bits, 128)
        assert np.array_equal(q1, q2) and np.array_equal(z1, z2) and np.array_equal(st1, st2)


def test_quantize16_brute_force_nearest_level():
    """Each step is the binary16 nearest the fp32 step (struct 'e'), and each
    code is the nearest of the qmax+1 levels to f32(ws/step) + z (ties: even)."""
    x, w = synth.random_layer(32, 256, 6, seed=42, n_outlier=2)
    s = O.candidate_scales(O.act_stats(x)[1], 20)[0][11]
    W = synth.bf16_bits_to_f32(w).astype(np.float64)
    for bits in (3, 4):
        qmax = (1 << bits) - 1
        q, z, step = O.quantize16(w, s, bits, 128)
        _, _, step32 = O.quantize(w, s, bits, 128)
        for n in range(6):
            for g in range(2):
                st = float(step[n, g])
                assert py_f16_bits(st) == py_f16_bits(float(step32[n, g]))
                assert struct.unpack("<e", struct.pack("<e", st))[0] == st
                ws = [py_f32(W[n, k] * s[k]) for k in range(128 * g, 128 * g + 128)]
                mn = min(min(ws), 0.0)
                zz = min(max(round(py_f32(-mn / st)), 0), qmax)
                assert z[n, g] == zz
                for j, v in enumerate(ws):
                    t = py_f32(v / st)
                    best = min(range(qmax + 1), key=lambda c: (abs(t - (c - zz)), (c - zz) % 2))
                    assert q[n, 128 * g + j] == best


def test_quantize16_clamped_and_subnormal_steps():
    """Tiny ranges take the smallest binary16 step 2^-24 (codes and zero 0);
    ranges past 15 * 65504 take 65504 and saturate the codes; a zero group
    keeps step 1; binary16-subnormal steps are multiples of 2^-24 within
    2^-25 of the fp32 step."""
    vals = np.zeros((4, 128), np.float32)
    vals[0, :64], vals[0, 64:] = 1e-9, -1e-9
    vals[1, 0], vals[1, 1], vals[1, 2] = 2.0 ** 20, -(2.0 ** 20), 65536.0
    vals[3] = np.linspace(-3e-4, 2e-4, 128, dtype=np.float32)
    w = synth.to_bf16_bits(vals)
    q, z, step = O.quantize16(w, None, 4, 128)
    assert step[0, 0] == 2.0 ** -24 and z[0, 0] == 0 and np.all(q[0] == 0)
    assert step[1, 0] == 65504.0 and z[1, 0] == 15
    assert q[1, 0] == 15 and q[1, 1] == 0 and q[1, 2] == 15 and q[1, 3] == 15
    assert step[2, 0] == 1.0 and z[2, 0] == 0 and np.all(q[2] == 0)
    _, _, s32 = O.quantize(w, None, 4, 128)
    assert s32[3, 0] < 2.0 ** -14
    n = step[3, 0] / 2.0 ** -24
    assert n == int(n) and abs(step[3, 0] - s32[3, 0]) <= 2.0 ** -25


def test_meta16_pack_brute_force_and_roundtrip():
    rng = np.random.default_rng(43)
    for G in (1, 5, 8):
        z = rng.integers(0, 16, size=(3, G))
        st = np.array([[struct.unpack("<e", struct.pack("<e", float(v)))[0] for v in row]
                       for row in rng.uniform(1e-3, 2.0, size=(3, G))])
        sb, zb = O.pack_meta16(z, st)
        assert sb.dtype == np.uint16 and zb.dtype == np.uint8 and zb.shape == (3, (G + 1) // 2)
        for n in range(3):
            for g in range(G):
                assert int(sb[n, g]) == py_f16_bits(float(st[n, g]))
            for j in range((G + 1) // 2):
                lo = int(z[n, 2 * j])
                hi = int(z[n, 2 * j + 1]) if 2 * j + 1 < G else 0
                assert int(zb[n, j]) == lo + 16 * hi
        st2, z2 = O.unpack_meta16(sb, zb, G)
        assert np.array_equal(z2, z) and np.array_equal(st2, st)


def test_decode_gemm16_brute_force_from_bytes():
    """Codes, zeros and steps decoded from the stored words and bytes in pure
    Python (nibbles by shifting, steps by struct 'e'); the dequantized weight
    (q - z) * step is exact in binary64.  The dense INT3 container gives the
    same product."""
    M, N, K = 3, 6, 384
    x, w = synth.random_layer(M, K, N, seed=44)
    X = synth.bf16_bits_to_f32(x).astype(np.float64)
    for bits in (4, 3):
        q, z, st = O.quantize16(w, None, bits, 128)
        qw = O.pack(q, z, st)[0]
        sb, zb = O.pack_meta16(z, st)
        Y = O.decode_gemm16(x, qw, sb, zb, 128)
        words = qw.astype(np.uint64)
        for m in range(M):
            for n in range(N):
                terms = []
                for k in range(K):
                    g = k // 128
                    code = (int(words[n, k // 8]) >> (4 * (k % 8))) & 15
                    zero = (int(zb[n, g // 2]) >> (4 * (g % 2))) & 15
                    stv = struct.unpack("<e", struct.pack("<H", int(sb[n, g])))[0]
                    terms.append(X[m, k] * ((code - zero) * stv))
                assert Y[m, n] == pytest.approx(math.fsum(terms), rel=1e-13, abs=1e-300)
        if bits == 3:
            Y3 = O.decode_gemm16(x, O.pack3(q), sb, zb, 128, dense3=True)
            assert np.array_equal(Y3, Y)


def test_compact_storage_bytes():
    """4-bit codes + 2-byte step + half-byte zero per group of 128: 4.156
    bits per weight, 3.85 times smaller than bf16 (the pages' "about four
    times")."""
    N, K = 4096, 4096
    assert O.packed16_bytes(N, K, 128) == N * K // 2 + N * 32 * 2 + N * 16
    assert O.packed16_bytes(N, K, 128, code_bits=3) == N * K * 3 // 8 + N * 32 * 2 + N * 16
    ratio = 2 * N * K / O.packed16_bytes(N, K, 128)
    assert 3.8 < ratio < 3.9


# ------------------------------------------------- the synthetic block pipeline

def test_rmsnorm_closed_form_and_scaling():
    """A constant row c = +-2^p with eps = 0 normalises to exactly +-gamma;
    with eps = 0 scaling the row by 2^p changes nothing; the normalised
    row's mean square is ms / (ms + eps)."""
    gamma = np.array([0.75, 1.25, 1.0, 1.5] * 32, np.float32)
    for c in (4.0, -0.5, 2.0 ** -6):
        x = synth.to_bf16_bits(np.full((1, 128), c, np.float32))
        u, r = O.rmsnorm(x, gamma, 0.0)
        assert r[0] == 1.0 / abs(c)
        assert np.array_equal(O.bf16_bits_to_f64(u)[0], np.sign(c) * O.bf16_round(gamma))
    x, _ = synth.random_layer(9, 256, 8, seed=23, n_outlier=3)
    u0, _ = O.rmsnorm(x, gamma[:1].repeat(256), 0.0)
    x8 = synth.to_bf16_bits((O.bf16_bits_to_f64(x) * 8).astype(np.float32))
    u8, _ = O.rmsnorm(x8, gamma[:1].repeat(256), 0.0)
    assert np.array_equal(u0, u8)
    X = O.bf16_bits_to_f64(x)
    ms = (X * X).mean(axis=1)
    _, r = O.rmsnorm(x, np.ones(256, np.float32), 1e-2)
    np.testing.assert_allclose(ms * r.astype(np.float64) ** 2, ms / (ms + 1e-2), rtol=2e-7)


def test_silu_mul_against_torch_and_identities():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(29)
    F = 64
    y = (rng.standard_normal((5, 2 * F)) * 4).astype(np.float32)
    y[0, :4] = [0.0, 60.0, -60.0, -800.0]
    h = O.silu_mul(y, F)
    ref = torch.nn.functional.silu(torch.from_numpy(y[:, :F]).double()) * torch.from_numpy(y[:, F:]).double()
    assert np.array_equal(h, O.bf16_rne_bits(ref.float().numpy()))
    H = O.bf16_bits_to_f64(h)
    assert H[0, 0] == 0.0 and H[0, 3] == 0.0
    assert H[0, 1] == O.bf16_round(O.f32(60.0 * np.float64(y[0, F + 1])))


def test_divide_rows_and_residual_against_library():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(31)
    v = rng.uniform(1e-4, 1e-2, (12, 5)).astype(np.float32)
    s = rng.uniform(0.2, 5.0, 12).astype(np.float32)
    assert np.array_equal(O.divide_rows(v, s), v / s[:, None])
    assert np.array_equal(O.divide_rows(v[:, 0], s), v[:, 0] / s)
    x, _ = synth.random_layer(4, 128, 8, seed=31)
    y = rng.standard_normal((4, 128)).astype(np.float32)
    xt = torch.from_numpy(O.bf16_bits_to_f64(x).astype(np.float32))
    ref = (xt + torch.from_numpy(y)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(O.residual_add(x, y), ref)


def test_folds_move_the_scale_into_the_preceding_op():
    """The method's premise for the folds: dividing the preceding op's output
    by s and multiplying the weight by s leaves the product; after the
    roundings, rmsnorm with gamma / s times s is rmsnorm with gamma to within
    two bf16 steps, and silu(g) * (v / s) is silu(g) * v / s."""
    x, _ = synth.random_layer(16, 256, 8, seed=37, n_outlier=4)
    rng = np.random.default_rng(37)
    gamma = rng.uniform(0.5, 1.5, 256).astype(np.float32)
    s = np.exp(rng.uniform(-1, 1, 256)).astype(np.float32)
    u, _ = O.rmsnorm(x, gamma, 1e-5)
    uf, _ = O.rmsnorm(x, O.divide_rows(gamma, s), 1e-5)
    U, UF = O.bf16_bits_to_f64(u), O.bf16_bits_to_f64(uf) * s[None, :]
    assert np.all(np.abs(UF - U) <= 2 * 2.0 ** -8 * np.abs(U) + 1e-30)
    F = 256
    y = (rng.standard_normal((16, 2 * F)) * 3).astype(np.float32)
    yf = y.copy()
    yf[:, F:] = (y[:, F:].astype(np.float64) / s[None, :]).astype(np.float32)
    H = O.bf16_bits_to_f64(O.silu_mul(y, F))
    HF = O.bf16_bits_to_f64(O.silu_mul(yf, F)) * s[None, :]
    assert np.all(np.abs(HF - H) <= 3 * 2.0 ** -8 * np.abs(H) + 1e-30)


def test_mlp_block_steps_and_fold_of_the_up_rows():
    """One block: the searches are the plain search on the block's own
    activations, gamma and the up rows' steps carry 1/s, and the deployed
    up output equals the undeployed one divided by s2 (to the roundings)."""
    rng = np.random.default_rng(43)
    d, F = 256, 384
    x, _ = synth.random_layer(48, d, 8, seed=43, n_outlier=3)
    gamma = rng.uniform(0.5, 1.5, d).astype(np.float32)
    wgu = synth.to_bf16_bits((rng.standard_normal((2 * F, d)) * 0.02).astype(np.float32))
    wd = synth.to_bf16_bits((rng.standard_normal((d, F)) * 0.02).astype(np.float32))
    r = O.mlp_block(x, gamma, wgu, wd, n_grid=6)
    ref1 = O.search(r["u"], wgu, 4, 128, 6)
    assert np.array_equal(r["gate_up"]["losses"], ref1["losses"])
    assert np.array_equal(r["gamma_folded"], O.divide_rows(gamma, ref1["best_s"]))
    ref2 = O.search(r["h"], wd, 4, 128, 6)
    assert np.array_equal(r["down"]["losses"], ref2["losses"])
    s2 = ref2["best_s"].astype(np.float64)
    assert np.array_equal(r["scales_gu_folded"][:F], r["gate_up"]["scales"][:F])
    v1, v2 = r["y_gu"][:, F:], r["y_gu2"][:, F:]
    assert np.abs(v2 * s2[None, :] - v1).max() <= 2e-2 * np.abs(v1).max()
    assert r["x_next"].shape == x.shape and r["x_next"].dtype == np.uint16


def test_mlp_block_deployed_error_is_the_searched_loss():
    """The block against the fp64 block with unquantized weights.  Each
    layer's search scores candidate i by the MSE of X . B_i^T against
    X . W^T, with 1/s folded into B (robotsatlas.com "AWQ", How it works:
    the activation is divided by the factor that multiplies the weight, and
    the grid search minimises the layer's output error).  Once deployed
    (1/s1 folded into the RMSNorm gain, 1/s2 into the up rows' steps), each
    layer computes the same product up to bf16 roundings of the folded
    activation and weight, so its output error against the fp64 product
    with unquantized weights must equal the search's chosen loss to within
    those roundings (measured 0.1%; 2% allowed).  Deploying on the unfolded
    activation or skipping a fold multiplies the error several times over.
    End to end, the block's update error is at most the down layer's
    searched error plus the gate/up error carried through the down weights
    (triangle inequality)."""
    rng = np.random.default_rng(44)
    M, d, F = 128, 256, 256
    x, _ = synth.random_layer(M, d, 8, seed=44, n_outlier=4, outlier_factor=20.0)
    gamma = rng.uniform(0.5, 1.5, d).astype(np.float32)
    wgu = synth.to_bf16_bits((rng.standard_normal((2 * F, d)) * 0.02).astype(np.float32))
    wd = synth.to_bf16_bits((rng.standard_normal((d, F)) * 0.02).astype(np.float32))
    r = O.mlp_block(x, gamma, wgu, wd, n_grid=10)
    b1, b2 = r["gate_up"]["best_idx"], r["down"]["best_idx"]
    assert b1 > 0 and b2 > 0          # the folds are not identities here
    u = O.bf16_bits_to_f64(O.rmsnorm(x, gamma, 1e-5)[0])
    y_gu_fp = u @ O.bf16_bits_to_f64(wgu).T
    ratio_gu = np.mean((r["y_gu"] - y_gu_fp) ** 2) / r["gate_up"]["losses"][b1]
    assert abs(ratio_gu - 1.0) <= 2e-2, ratio_gu
    h = O.bf16_bits_to_f64(r["h"])
    Wd = O.bf16_bits_to_f64(wd)
    y_d_fp = h @ Wd.T
    ratio_d = np.mean((r["y_down"] - y_d_fp) ** 2) / r["down"]["losses"][b2]
    assert abs(ratio_d - 1.0) <= 2e-2, ratio_d
    # end to end against the unquantized block (fp64 throughout)
    g, v = y_gu_fp[:, :F], y_gu_fp[:, F:]
    H_fp = g / (1.0 + np.exp(-g)) * v
    Y_fp = H_fp @ Wd.T
    bound = 1.02 * np.sqrt(M * d * r["down"]["losses"][b2]) + np.linalg.norm((h - H_fp) @ Wd.T)
    err = np.linalg.norm(r["y_down"] - Y_fp)
    assert err <= bound, (err, bound)
    x_next_fp = O.bf16_bits_to_f64(x) + Y_fp
    assert np.linalg.norm(O.bf16_bits_to_f64(r["x_next"]) - x_next_fp) <= bound + 2e-2 * np.linalg.norm(x_next_fp)
