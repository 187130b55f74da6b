"""CPU fp64 oracle for the AWQ per-layer scale search and its W4A16 contraction.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  It shares no code
with the HIP library (no kernels, headers, helpers or constants); the two agree
only through the arithmetic contract written out below.

Pages (cited by title / address and section; nothing here is quoted):

  [P1] "AWQ (Activation-aware Weight Quantization)", builderai.tools/tool/awq
  [P3] "AWQ", robotsatlas.com/ai-technologies/awq
  [P4] AWQ project page, sourcepulse.org/projects/1842286
  [P5] "What is AWQ?", aquanode.io/gpu-glossary/awq

What the pages fix: a calibration pass measures how large the activations are
at each linear layer's input ([P3] "How it works", "Key mechanisms",
"Components"); each input channel gets a factor that multiplies the weight and
divides the activation, which leaves the product unchanged ([P3] "How it works",
"Components" / per-channel scaling; [P5] "The core idea"); the factor is picked
by a grid search that minimises the layer's output error ([P3] "How it works",
"Key mechanisms"); then weights are quantized group-wise (groups of 128) to 4 or
3 bits with a per-group scale ([P3] "Components" / group-wise 4-bit
quantization, "Hyperparameters"; [P4] opening paragraph) and written as real
packed INT4 ([P1] "About").

Where the pages are silent the following readings are used (each one is also a
contract the GPU library implements):

  statistic        a[k] = mean over tokens of |x[m,k]|
  grid             alpha_i = i / n_grid, i = 0..n_grid-1  (includes 0, excludes 1)
  candidate        r = max(a^alpha, 1e-4);  s = r / sqrt(max_k r * min_k r)
  quantizer        asymmetric, per (row, group of `group` input channels):
                   range extended to include 0; step = range / qmax
                   (1.0 when that is zero); zero z = rint(-min/step);
                   q = clamp(rint(ws/step) + z, 0, qmax); rint = half-to-even
  packing          qweight[n][t] = sum_i q[n, 8t+i] << 4i  (u32, sequential
                   nibbles along K; 3-bit codes use the same 4-bit containers)
                   scales f32 [N][K/group], zeros u8 [N][K/group]
  dense INT3       qweight3[n][3c .. 3c+2] = the 96-bit little-endian value
                   sum_i q[n, 32c+i] << 3i of each run of 32 codes
  compact format   for deployment: the fp32 step limited to [2^-24, 65504]
                   and rounded to binary16 (nearest, ties to even) before the
                   zero and the codes are computed; steps stored as binary16
                   [N][G], zeros two per byte (even group in the low nibble)
                   [N][ceil(G/2)]
  decode tiles     the codes of rows 16b..16b+15 and group g as tile b*G+g,
                   row r's piece for channels 32q.. at byte P*(r + 16q);
                   inside a piece channels 2p, 2p+1 form pair p, placed
                   for a one-mask lift into a 32-bit word's two halves
  dequantized B    B[n,k] = bf16( f32( f32((q - z) * step) * inv_s[k] ) )
                   (1/s folded into the weight operand; the activation operand
                   is the caller's bf16 X, unchanged)
  difference       D = bf16(f32(B - W)), the operand whose product with X is
                   the output error X.B^T - X.W^T; no rounding happens there:
                   a nonzero B has |W s| >= step/2, so B/W lies in [1/2, 2]
                   and by Sterbenz's lemma B - W is a bf16 value
  loss             MSE over all M*N outputs of X.B^T against X.W^T, fp64
  selection        first index of the minimum loss (NaN never wins; all-NaN
                   gives -1)
  block pipeline   a Llama-shaped feed-forward sublayer searched in order:
                   u = bf16(f32(f32(x * r) * gamma)), r = f32(1/sqrt(mean x^2 + eps));
                   H = bf16(f32(silu(g) * v)) in fp64; 1/s folds into gamma
                   (gate_up) and into the up rows' steps (down) as f32(v / s);
                   the residual x + y rounds to f32, then to bf16
  decode product   for the deployment contraction with few tokens, the
                   dequantized weight is the exact (q - z) * step (no bf16
                   rounding): Y = A . ((q - z) * step)^T

Every "f32(...)" marks one IEEE fp32 operation of the contract.  The oracle
evaluates the exact operation in fp64 and rounds the result to fp32; for +, -,
x and / this equals the correctly rounded fp32 result because 53 >= 2*24 + 2
(double rounding is innocuous; S. Figueroa, "When is double rounding
innocuous?", 1995).  Products of two fp32 values are exact in fp64.

Parity unpinned (convention only, no value on the pages can fix them): the
normalising constant sqrt(max*min), the 1e-4 floor, the nibble order of the
packed layout, the 4-bit container used for INT3 codes and the bit order of the
dense INT3 layout, the order of the decode tiles, and the compact format's
step range limits and zero nibble order.
"""

from __future__ import annotations

import numpy as np

# Floor applied after the power in the candidate scale (a reading: guards dead
# channels, whose 0^alpha would make 1/s infinite).
SCALE_FLOOR = 1e-4


# --------------------------------------------------------------------------
# Number formats.  bf16 is the top 16 bits of an IEEE binary32.
# --------------------------------------------------------------------------

def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bf16 bit patterns (uint16) as float64."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f32(x) -> np.ndarray:
    """Round float64 values to the nearest binary32 (ties to even); back as float64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_rne_bits(x) -> np.ndarray:
    """Round values that are already binary32 to bf16, nearest with ties to even.

    Written out as the definition: the two bf16 neighbours of x are the value
    with the low 16 bits cleared (towards zero) and the next one away from
    zero; the closer one wins and an exact tie goes to the one whose last
    kept mantissa bit is 0.  NaN maps to a quiet NaN.
    """
    v = np.asarray(x, dtype=np.float64).astype(np.float32)
    u = v.view(np.uint32)
    lo = u & np.uint32(0xFFFF0000)                     # towards zero
    hi = lo + np.uint32(0x10000)                       # away from zero
    vlo = lo.view(np.float32).astype(np.float64)
    vhi = hi.view(np.float32).astype(np.float64)
    # Past the largest finite bf16 the upper neighbour is 2^128 in an unbounded
    # exponent range (IEEE 754 overflow rule); it is stored as infinity.
    vhi = np.where(np.isinf(vhi), np.copysign(2.0 ** 128, vhi), vhi)
    vx = v.astype(np.float64)
    dlo = np.abs(vx - vlo)
    with np.errstate(invalid="ignore"):
        dhi = np.abs(vhi - vx)
    lo_even = ((lo >> np.uint32(16)) & np.uint32(1)) == 0
    take_lo = (dlo < dhi) | ((dlo == dhi) & lo_even)
    out = np.where(take_lo, lo, hi)
    exact = (u & np.uint32(0xFFFF)) == 0
    out = np.where(exact, u, out)
    nan = np.isnan(v)
    out = np.where(nan, (u | np.uint32(0x00400000)) & np.uint32(0xFFFF0000), out)
    return (out >> np.uint32(16)).astype(np.uint16)


def bf16_round(x) -> np.ndarray:
    """Value after RNE rounding of binary32 values to bf16, as float64."""
    return bf16_bits_to_f64(bf16_rne_bits(x))


# --------------------------------------------------------------------------
# Step 1: activation statistics.
# [P3] "How it works" and "Components" / activation saliency analysis: the
# calibration set is run through the model and activation magnitudes are
# measured at each linear layer's input.  Reading: mean |x| per input channel.
# --------------------------------------------------------------------------

def act_stats(x_bits, chunk_rows: int = 8192):
    """Per-input-channel mean |x| over all M calibration tokens.

    x_bits: uint16 bf16 patterns [M][K].  Returns (a64, a32): the fp64 mean and
    that mean rounded to fp32 (the value the scale step consumes).
    """
    x_bits = np.asarray(x_bits)
    M, K = x_bits.shape
    total = np.zeros(K, dtype=np.float64)
    for r0 in range(0, M, chunk_rows):
        total += np.abs(bf16_bits_to_f64(x_bits[r0:r0 + chunk_rows])).sum(axis=0)
    a64 = total / M
    return a64, f32(a64)


# --------------------------------------------------------------------------
# Step 2: candidate per-channel scales.
# [P3] "How it works": a factor per input channel, weight multiplied and
# activation divided by it; the factor comes from the activation statistic.
# Reading: s = a^alpha on an n_grid-point grid in [0, 1), floored, normalised.
# --------------------------------------------------------------------------

def alpha_grid(n_grid: int) -> np.ndarray:
    return np.arange(n_grid, dtype=np.float64) / float(n_grid)


def candidate_scales(a32, n_grid: int):
    """(s32, inv32), each [n_grid][K]: s rounded to fp32 and fp32(1 / s32)."""
    a32 = np.asarray(a32, dtype=np.float64)
    K = a32.shape[0]
    s32 = np.empty((n_grid, K), dtype=np.float64)
    inv32 = np.empty((n_grid, K), dtype=np.float64)
    for i, alpha in enumerate(alpha_grid(n_grid)):
        r = np.maximum(np.power(a32, alpha), SCALE_FLOOR)   # 0^0 = 1
        s = r / np.sqrt(r.max() * r.min())
        s32[i] = f32(s)
        inv32[i] = f32(1.0 / s32[i])
    return s32, inv32


# --------------------------------------------------------------------------
# Step 3: group-wise asymmetric quantization of W.diag(s).
# [P3] "How it works" (quantized group-wise after the scales are set),
# "Components" (groups of 128, per-group scale), "Hyperparameters" (4 or 3
# bits, group 128).  Reading: asymmetric, with a per-group integer zero.
# --------------------------------------------------------------------------

def quantize(w, s32, bits: int, group: int):
    """Quantize ws = f32(W * s) group-wise along K.

    w: bf16 bit patterns (uint16) or float64 values [N][K]; s32: [K] or None
    (None means s = 1).  Returns (q int64 [N][K], z int64 [N][K/group],
    step float64 [N][K/group] holding fp32 values).
    """
    return _quantize(w, s32, bits, group, half_steps=False)


def quantize16(w, s32, bits: int, group: int):
    """The quantizer for the compact deployment format (16-bit steps): as
    quantize, except that the fp32 step is first limited to the binary16
    range [2^-24, 65504] (fmax/fmin, so NaN becomes 2^-24) and rounded to
    binary16; the zero and the codes are then computed with that step, so
    the stored step is the one the codes were rounded against.  Returns
    (q, z, step) with step holding binary16 values."""
    return _quantize(w, s32, bits, group, half_steps=True)


def _quantize(w, s32, bits: int, group: int, half_steps: bool):
    W = bf16_bits_to_f64(w) if np.asarray(w).dtype == np.uint16 else np.asarray(w, np.float64)
    N, K = W.shape
    if K % group:
        raise ValueError("K must be a multiple of the group size")
    qmax = float((1 << bits) - 1)
    ws = f32(W * (1.0 if s32 is None else np.asarray(s32, np.float64)[None, :]))
    G = ws.reshape(N, K // group, group)
    mx = np.maximum(G.max(axis=2), 0.0)
    mn = np.minimum(G.min(axis=2), 0.0)
    rng = f32(mx - mn)
    step = f32(rng / qmax)
    step = np.where(step > 0.0, step, 1.0)
    if half_steps:
        step = f16_bits_to_f64(f16_rne_bits(np.fmin(np.fmax(step, F16_MIN), F16_MAX)))
    z = np.clip(np.rint(f32(-mn / step)), 0.0, qmax)
    q = np.clip(np.rint(f32(G / step[:, :, None])) + z[:, :, None], 0.0, qmax)
    return q.reshape(N, K).astype(np.int64), z.astype(np.int64), step


# IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
F16_MIN = 2.0 ** -24          # smallest positive (subnormal) value
F16_MAX = 65504.0             # largest finite value


def f16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of binary16 bit patterns (uint16), from the format's
    definition: (-1)^s * 2^(e-15) * (1 + f/1024) for 0 < e < 31,
    (-1)^s * 2^-14 * f/1024 for e = 0, infinity or NaN for e = 31."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(b >> 15, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    f = (b & 0x3FF).astype(np.float64)
    normal = (1.0 + f / 1024.0) * np.exp2(e.astype(np.float64) - 15.0)
    sub = f / 1024.0 * 2.0 ** -14
    mag = np.where(e == 0, sub, normal)
    mag = np.where(e == 31, np.where(f == 0, np.inf, np.nan), mag)
    return sign * mag


def f16_rne_bits(x) -> np.ndarray:
    """Round binary32 values to binary16, nearest with ties to even, as bit
    patterns.  Written out from the definition: in the binade of |x| (the
    subnormal binade below 2^-14) the spacing is u = 2^(E-10); |x| / u is
    rounded to the nearest integer, an exact half going to the even one, and
    the result re-encoded; a result above 65504 is infinity (IEEE 754
    overflow: |x| >= 65520).  NaN maps to a quiet NaN."""
    with np.errstate(invalid="ignore", over="ignore"):
        v = np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)
    neg = np.signbit(v)
    a = np.abs(v)
    finite = np.isfinite(a)
    af = np.where(finite & (a > 0), a, 1.0)
    _, ex = np.frexp(af)                        # af = m * 2^ex, m in [1/2, 1)
    E = np.maximum(ex - 1, -14)                 # binade exponent, floored at the subnormals
    u = np.exp2((E - 10).astype(np.float64))
    n = af / u                                  # exact: a power-of-two scaling
    lo = np.floor(n)
    frac = n - lo
    up = (frac > 0.5) | ((frac == 0.5) & (np.mod(lo, 2.0) == 1.0))
    m = (lo + up) * u                           # the rounded magnitude
    m = np.where(finite & (a > 0), m, np.where(finite, 0.0, np.inf))
    _, ex2 = np.frexp(np.where(m > 0, m, 1.0))
    e_field = np.where(m >= 2.0 ** -14, ex2 - 1 + 15, 0)
    frac_field = np.where(m >= 2.0 ** -14, (m / np.exp2((ex2 - 1).astype(np.float64)) - 1.0) * 1024.0,
                          m / 2.0 ** -24)
    out = (e_field.astype(np.int64) << 10) | np.rint(np.where(np.isfinite(frac_field), frac_field, 0.0)).astype(np.int64)
    out = np.where(m > F16_MAX, 0x7C00, out)
    out = np.where(np.isnan(v), 0x7E00, out)
    out = out | np.where(neg, 0x8000, 0)
    return out.astype(np.uint16)


# --------------------------------------------------------------------------
# Step 3b: packing ("writes real INT4 weights", [P1] "About").
# --------------------------------------------------------------------------

def pack(q, z, step):
    """(qweight u32 [N][K/8], scales f32 [N][K/g], zeros u8 [N][K/g])."""
    q = np.asarray(q, dtype=np.uint64)
    N, K = q.shape
    words = np.zeros((N, K // 8), dtype=np.uint64)
    for i in range(8):
        words |= q[:, i::8] << np.uint64(4 * i)
    return (words.astype(np.uint32), np.asarray(step, np.float64).astype(np.float32),
            np.asarray(z).astype(np.uint8))


def unpack(qweight):
    """Codes [N][K] from packed words (inverse of pack's nibble order)."""
    w = np.asarray(qweight, dtype=np.uint32)
    N, T = w.shape
    q = np.empty((N, T * 8), dtype=np.int64)
    for i in range(8):
        q[:, i::8] = (w >> np.uint32(4 * i)) & np.uint32(0xF)
    return q


def packed_bytes(N: int, K: int, group: int) -> int:
    """Storage of the packed form: 4-bit codes + fp32 scale + u8 zero per group."""
    return N * K // 2 + N * (K // group) * (4 + 1)


def pack_meta16(z, step16):
    """The compact per-group metadata of the deployment format: steps as
    binary16 bit patterns uint16 [N][G], and zeros two per byte, group 2j in
    the low nibble of byte j and group 2j+1 in the high nibble (a zero past
    the last group is 0), uint8 [N][ceil(G/2)]."""
    z = np.asarray(z, dtype=np.int64)
    N, G = z.shape
    if z.min(initial=0) < 0 or z.max(initial=0) > 15:
        raise ValueError("zeros must lie in [0, 15]")
    zp = np.zeros((N, 2 * ((G + 1) // 2)), dtype=np.int64)
    zp[:, :G] = z
    zeros4 = (zp[:, 0::2] | (zp[:, 1::2] << 4)).astype(np.uint8)
    return f16_rne_bits(step16), zeros4


def unpack_meta16(steps16, zeros4, G: int):
    """(step float64 [N][G], z int64 [N][G]) from the compact metadata."""
    zb = np.asarray(zeros4, dtype=np.int64)
    z = np.empty((zb.shape[0], 2 * zb.shape[1]), dtype=np.int64)
    z[:, 0::2] = zb & 0xF
    z[:, 1::2] = zb >> 4
    return f16_bits_to_f64(steps16), z[:, :G]


def packed16_bytes(N: int, K: int, group: int, code_bits: int = 4) -> int:
    """Storage of the compact form: codes + binary16 step + 4-bit zero per group."""
    G = K // group
    return N * code_bits * K // 8 + N * G * 2 + N * ((G + 1) // 2)


def pack3(q):
    """Dense INT3 codes ([P4] opening paragraph: 3- and 4-bit weights): each
    run of 32 codes along K is one 96-bit little-endian value with code i at
    bits 3i .. 3i+2, stored as three u32 words.  qweight3 u32 [N][3K/32]."""
    q = np.asarray(q, dtype=np.int64)
    N, K = q.shape
    if K % 32:
        raise ValueError("K must be a multiple of 32")
    if q.min(initial=0) < 0 or q.max(initial=0) > 7:
        raise ValueError("codes must lie in [0, 7]")
    bits = ((q.reshape(N, K // 32, 32, 1) >> np.arange(3)) & 1).astype(np.uint8)
    by = np.packbits(bits.reshape(N, K // 32, 96), axis=-1, bitorder="little")   # 12 bytes
    return np.ascontiguousarray(by).view("<u4").reshape(N, 3 * K // 32).astype(np.uint32)


def unpack3(qweight3):
    """Codes [N][K] from dense INT3 words (inverse of pack3)."""
    w = np.ascontiguousarray(np.asarray(qweight3, dtype="<u4"))
    N, T = w.shape
    bits = np.unpackbits(w.view(np.uint8).reshape(N, T // 3, 12), axis=-1, bitorder="little")
    b3 = bits.reshape(N, T // 3, 32, 3).astype(np.int64)
    return (b3[..., 0] | (b3[..., 1] << 1) | (b3[..., 2] << 2)).reshape(N, T // 3 * 32)


def decode_tiles(qweight, K: int, dense3: bool = False, group: int = 128) -> np.ndarray:
    """The packed codes rearranged for streaming by 16-row blocks (a layout of
    this library, for the deployment contraction): rows 16b .. 16b+15 (zero
    rows past N) and one group g form tile b*G + g; inside it the P-byte
    piece of row r covering the group's channels 32q .. 32q+31 sits at byte
    P*(r + 16q), with P = 16 for 4-bit containers and 12 for dense INT3.
    Inside a piece, channels 2p and 2p+1 form pair p (p = 0..15), placed so
    that one mask lifts a pair into the two halves of a 32-bit word:
      4-bit containers: u32 word j holds pairs 4j..4j+3, pair 4j+t's first
        code in nibble t and its second in nibble 4+t;
      dense INT3: pair p < 15 sits in u32 word p // 5, first code at bits
        3(p % 5), second at bits 16 + 3(p % 5); pair 15 is spread over the
        free bits: bit i of channel 30's code at bit 15 of word i, bit i of
        channel 31's code at bit 31 of word i.
    Returns bytes (little-endian words), uint8 [ceil(N/16) * G * 16 * 4P]."""
    codes = unpack3(qweight) if dense3 else unpack(qweight)
    N = codes.shape[0]
    G = K // group
    NB = -(-N // 16)
    c = np.zeros((NB * 16, K), dtype=np.uint64)
    c[:N] = codes
    pieces = c.reshape(NB, 16, G, 4, 32)                  # [b][r][g][q][channel]
    first, second = pieces[..., 0::2], pieces[..., 1::2]  # [b][r][g][q][pair]
    if dense3:
        words = np.zeros(pieces.shape[:4] + (3,), dtype=np.uint64)
        for p in range(15):
            sh = np.uint64(3 * (p % 5))
            words[..., p // 5] |= (first[..., p] << sh) | (second[..., p] << (sh + np.uint64(16)))
        for i in range(3):
            bit = np.uint64(i)
            words[..., i] |= (((first[..., 15] >> bit) & np.uint64(1)) << np.uint64(15)) | \
                             (((second[..., 15] >> bit) & np.uint64(1)) << np.uint64(31))
    else:
        words = np.zeros(pieces.shape[:4] + (4,), dtype=np.uint64)
        for j in range(4):
            for t in range(4):
                words[..., j] |= (first[..., 4 * j + t] << np.uint64(4 * t)) | \
                                 (second[..., 4 * j + t] << np.uint64(16 + 4 * t))
    t = words.transpose(0, 2, 3, 1, 4)                    # [b][g][q][r][word]
    return np.ascontiguousarray(t.astype("<u4")).reshape(-1).view(np.uint8)


def decode_meta(steps16, zeros4, K: int, group: int = 128) -> np.ndarray:
    """The compact metadata rearranged like decode_tiles (a layout of this
    library, for the deployment contraction): one u32 per row and group,
    the binary16 step bits in bits 0..15 and the 4-bit zero in bits 16..19;
    word r of tile b*G + g belongs to row 16b + r and group g, rows past N
    give 0.  Returns uint32 [ceil(N/16) * G * 16]."""
    G = K // group
    st = np.asarray(steps16, dtype=np.uint16).astype(np.uint64)
    N = st.shape[0]
    _, z = unpack_meta16(steps16, zeros4, G)
    NB = -(-N // 16)
    w = np.zeros((NB * 16, G), dtype=np.uint64)
    w[:N] = st | (z.astype(np.uint64) << np.uint64(16))
    return np.ascontiguousarray(w.reshape(NB, 16, G).transpose(0, 2, 1)).reshape(-1).astype(np.uint32)


def packed3_bytes(N: int, K: int, group: int) -> int:
    """Storage of the dense INT3 form: 3-bit codes + fp32 scale + u8 zero per group."""
    return N * 3 * K // 8 + N * (K // group) * (4 + 1)


# --------------------------------------------------------------------------
# Step 4: the weight operand of the contraction and the per-candidate loss.
# [P3] "How it works" / "Key mechanisms": the scale is chosen by a grid search
# that minimises the layer's output error.  The activation divided by s is the
# same product as the weight multiplied by 1/s ([P3] "Components" / per-channel
# scaling), so 1/s is applied to the dequantized weight.
# --------------------------------------------------------------------------

def dequant_operand(q, z, step, group: int, inv32=None) -> np.ndarray:
    """B[n,k] = bf16(f32(f32((q - z) * step) * inv_s[k])) as float64 values.

    With inv32 None the last multiply is skipped (deployment form, s folded
    upstream): B = bf16(f32((q - z) * step)).
    """
    q = np.asarray(q, np.float64)
    zz = np.repeat(np.asarray(z, np.float64), group, axis=1)
    st = np.repeat(np.asarray(step, np.float64), group, axis=1)
    d = f32((q - zz) * st)
    if inv32 is not None:
        d = f32(d * np.asarray(inv32, np.float64)[None, :])
    return bf16_round(d)


def diff_operand(w_bits, b_values) -> np.ndarray:
    """D[n,k] = bf16(f32(B[n,k] - W[n,k])) as float64 values (B from dequant_operand).

    B - W is exact in fp64 (two bf16 values); the f32 then bf16 roundings are
    the contract's, and for the quantizer's B they change nothing (Sterbenz).
    """
    return bf16_round(f32(np.asarray(b_values, np.float64) - bf16_bits_to_f64(w_bits)))


def gemm(x_bits, b_values) -> np.ndarray:
    """Y = X . B^T in fp64 (X given as bf16 patterns, B as float64 values)."""
    return bf16_bits_to_f64(x_bits) @ np.asarray(b_values, np.float64).T


def output_mse(x_bits, w_bits, b_values, chunk_rows: int = 4096) -> float:
    """mean over m, n of (X.B^T - X.W^T)^2, evaluated as ||X (B - W)^T||^2 / (M N).

    X.B^T - X.W^T = X.(B - W)^T by distributivity; B - W is exact in fp64
    because both are bf16 values.
    """
    x_bits = np.asarray(x_bits)
    M = x_bits.shape[0]
    D = np.asarray(b_values, np.float64) - bf16_bits_to_f64(w_bits)
    N = D.shape[0]
    sse = 0.0
    for r0 in range(0, M, chunk_rows):
        E = bf16_bits_to_f64(x_bits[r0:r0 + chunk_rows]) @ D.T
        sse += float(np.einsum("ij,ij->", E, E))
    return sse / (M * N)


def gram(x_bits, chunk_rows: int = 8192) -> np.ndarray:
    """G = X^T X in fp64."""
    x_bits = np.asarray(x_bits)
    M, K = x_bits.shape
    G = np.zeros((K, K), dtype=np.float64)
    for r0 in range(0, M, chunk_rows):
        Xc = bf16_bits_to_f64(x_bits[r0:r0 + chunk_rows])
        G += Xc.T @ Xc
    return G


def output_mse_gram(G, M: int, w_bits, b_values) -> float:
    """Same MSE from the Gram matrix: sum_n D_n G D_n^T / (M N), D = B - W."""
    D = np.asarray(b_values, np.float64) - bf16_bits_to_f64(w_bits)
    N = D.shape[0]
    return float(np.einsum("nk,nk->", D @ G, D)) / (M * N)


def first_argmin(losses) -> int:
    """First index of the smallest loss; NaN never wins; -1 if all are NaN."""
    losses = np.asarray(losses, np.float64)
    best, best_v = -1, None
    for i, v in enumerate(losses):
        if np.isnan(v):
            continue
        if best_v is None or v < best_v:
            best, best_v = i, v
    return best


# --------------------------------------------------------------------------
# The whole per-layer search.
# --------------------------------------------------------------------------

def search(x_bits, w_bits, bits: int = 4, group: int = 128, n_grid: int = 20,
           loss_form: str = "direct", timings: dict | None = None):
    """AWQ per-layer scale search.  Returns a dict with every intermediate.

    loss_form "direct" evaluates each loss over the tokens; "gram" forms
    G = X^T X once and evaluates sum_n D_n G D_n^T (same value).
    """
    import time
    t0 = time.perf_counter()
    x_bits = np.asarray(x_bits)
    w_bits = np.asarray(w_bits)
    M = x_bits.shape[0]
    a64, a32 = act_stats(x_bits)
    s32, inv32 = candidate_scales(a32, n_grid)
    t1 = time.perf_counter()
    G = gram(x_bits) if loss_form == "gram" else None
    losses = np.empty(n_grid, dtype=np.float64)
    t_quant = 0.0
    for i in range(n_grid):
        tq = time.perf_counter()
        q, z, step = quantize(w_bits, s32[i], bits, group)
        B = dequant_operand(q, z, step, group, inv32[i])
        t_quant += time.perf_counter() - tq
        if G is None:
            losses[i] = output_mse(x_bits, w_bits, B)
        else:
            losses[i] = output_mse_gram(G, M, w_bits, B)
    t2 = time.perf_counter()
    best = first_argmin(losses)
    sel = best if best >= 0 else 0
    q, z, step = quantize(w_bits, s32[sel], bits, group)
    qweight, scales, zeros = pack(q, z, step)
    t3 = time.perf_counter()
    if timings is not None:
        timings.update(stats_and_scales=t1 - t0, quantize=t_quant,
                       loss=(t2 - t1) - t_quant, final_pack=t3 - t2)
    return dict(mean_abs64=a64, mean_abs=a32, s=s32, inv_s=inv32, alphas=alpha_grid(n_grid),
                losses=losses, best_idx=best, best_s=s32[sel].copy(),
                q=q, z=z, step=step, qweight=qweight, scales=scales, zeros=zeros)


def deploy_gemm(a_bits, qweight, scales, zeros, group: int, inv32=None) -> np.ndarray:
    """Y = A . B^T with B dequantized from packed codes ([P4] "Highlighted
    Details": 4-bit linear layers; [P1] "About": W4A16 kernels)."""
    q = unpack(qweight)
    B = dequant_operand(q, np.asarray(zeros, np.int64), np.asarray(scales, np.float64),
                        group, inv32)
    return gemm(a_bits, B)


def decode_gemm3(a_bits, qweight3, scales, zeros, group: int) -> np.ndarray:
    """The deployment contraction on dense INT3 weights: decode_gemm's
    product with the codes read through unpack3."""
    q = unpack3(qweight3)
    return _decode_product(a_bits, q, scales, zeros, group)


def decode_gemm(a_bits, qweight, scales, zeros, group: int) -> np.ndarray:
    """Deployment contraction with packed weights ([P1] "About": 4-bit weights
    with 16-bit activations; [P3] "Implementation pitfalls": the packed form
    is read directly): Y = A . Wd^T with Wd = (q - z) * step exactly.  (q - z)
    is a small integer and step a binary32, so every Wd and every product with
    a bf16 activation is exact in fp64; only the K-sum rounds."""
    return _decode_product(a_bits, unpack(qweight), scales, zeros, group)


def decode_gemm16(a_bits, qweight, steps16, zeros4, group: int, dense3: bool = False) -> np.ndarray:
    """The deployment contraction on the compact format: decode_gemm's
    product with (step, zero) read from binary16 steps and 4-bit zeros
    (every binary16 value is a binary32 value, so Wd = (q - z) * step stays
    exact)."""
    q = unpack3(qweight) if dense3 else unpack(qweight)
    step, z = unpack_meta16(steps16, zeros4, q.shape[1] // group)
    return _decode_product(a_bits, q, step, z, group)


def _decode_product(a_bits, q, scales, zeros, group: int) -> np.ndarray:
    """A . ((q - z) * step)^T in fp64 from codes [N][K]."""
    q = np.asarray(q, np.float64)
    z = np.repeat(np.asarray(zeros, np.float64), group, axis=1)
    step = np.repeat(np.asarray(scales, np.float32).astype(np.float64), group, axis=1)
    wd = (q - z) * step
    return bf16_bits_to_f64(a_bits) @ wd.T


# --------------------------------------------------------------------------
# The synthetic block pipeline around the search: a Llama-shaped feed-forward
# sublayer, searched layer after layer with each scale folded into the op
# before it ([P3] "How it works": the activation is divided by the same
# per-channel factor that multiplies the weight, which a deployment folds
# into the preceding operation; "Computational complexity": one search per
# layer, over the layers in order).  Every "bf16(...)" and "f32(...)" is a
# rounding point of the contract.
# --------------------------------------------------------------------------

def rmsnorm(x_bits, gamma32, eps: float):
    """u[m,k] = bf16(f32(f32(x[m,k] * r_m) * gamma[k])) with
    r_m = f32(1 / sqrt(sum_k x[m,k]^2 / K + eps)) evaluated in fp64.
    Returns (u bf16 bit patterns, r32)."""
    X = bf16_bits_to_f64(x_bits)
    K = X.shape[1]
    r32 = f32(1.0 / np.sqrt((X * X).sum(axis=1) / K + eps))
    u = f32(f32(X * r32[:, None]) * np.asarray(gamma32, np.float64)[None, :])
    return bf16_rne_bits(u), r32


def silu_mul(y32, F: int):
    """H = bf16(f32(silu(g) * v)) for y = [g | v] ([M][2F] fp32), with
    silu(g) = g / (1 + exp(-g)) and the product in fp64."""
    Y = np.asarray(y32, np.float64)
    g, v = Y[:, :F], Y[:, F:2 * F]
    with np.errstate(over="ignore"):
        h = g / (1.0 + np.exp(-g)) * v
    return bf16_rne_bits(f32(h))


def divide_rows(v32, s32):
    """out[r][c] = f32(v[r][c] / s[r]): 1/s folded into a gain (C = 1) or into
    the per-group steps of a quantized layer's output rows."""
    v = np.asarray(v32, np.float64)
    s = np.asarray(s32, np.float64)
    return f32(v / s.reshape((-1,) + (1,) * (v.ndim - 1)))


def residual_add(x_bits, y32):
    """x_next = bf16(f32(x + y))."""
    return bf16_rne_bits(f32(bf16_bits_to_f64(x_bits) + np.asarray(y32, np.float64)))


def mlp_block(x_bits, gamma32, wgu_bits, wdown_bits, eps: float = 1e-5, bits: int = 4,
              group: int = 128, n_grid: int = 20, upstream=None):
    """One feed-forward sublayer through the search, in order:

      u = rmsnorm(x, gamma);  search gate_up on u -> s1, Q_gu;  gamma' = gamma / s1
      [g | v] = rmsnorm(x, gamma') . dequant(Q_gu)^T (the deployed product)
      H = silu_mul(g, v);  search down on H -> s2, Q_down
      up rows' steps /= s2;  H' = silu_mul(g, v / s2 as deployed)
      x_next = residual_add(x, H' . dequant(Q_down)^T)

    `upstream` may supply the GPU's own intermediates (keys "u", "y_gu", "h",
    "h2", "y_down") so each step can be checked on identical inputs; the
    returned dict holds every intermediate the oracle computed."""
    up = upstream or {}
    F = np.asarray(wgu_bits).shape[0] // 2
    u, _ = rmsnorm(x_bits, gamma32, eps)
    r1 = search(up.get("u", u), wgu_bits, bits, group, n_grid)
    gamma_f = divide_rows(gamma32, r1["best_s"])
    u_f, _ = rmsnorm(x_bits, gamma_f, eps)
    y_gu = deploy_gemm(up.get("u_f", u_f), r1["qweight"], r1["scales"], r1["zeros"], group)
    h = silu_mul(up.get("y_gu", y_gu), F)
    r2 = search(up.get("h", h), wdown_bits, bits, group, n_grid)
    scales_f = np.asarray(r1["scales"], np.float32).copy()
    scales_f[F:] = divide_rows(scales_f[F:], r2["best_s"])
    y_gu2 = deploy_gemm(up.get("u_f", u_f), r1["qweight"], scales_f, r1["zeros"], group)
    h2 = silu_mul(up.get("y_gu2", y_gu2), F)
    y_down = deploy_gemm(up.get("h2", h2), r2["qweight"], r2["scales"], r2["zeros"], group)
    x_next = residual_add(x_bits, up.get("y_down", y_down))
    return dict(u=u, gate_up=r1, gamma_folded=gamma_f, u_f=u_f, y_gu=y_gu, h=h, down=r2,
                scales_gu_folded=scales_f, y_gu2=y_gu2, h2=h2, y_down=y_down, x_next=x_next)
