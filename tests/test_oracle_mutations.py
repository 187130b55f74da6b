"""Plant plausible mistakes in the oracle (CPU only) and check that the pins
in test_oracle_pins catch every one of them."""

import numpy as np
import pytest

import oracle
import oracle.awq_oracle as OA
import test_oracle_pins as P


class _NumpyWith:
    """numpy, except for the attributes overridden."""

    def __init__(self, **over):
        self._over = over

    def __getattr__(self, name):
        return self._over.get(name, getattr(np, name))


def _mut_floor_instead_of_rint(mp):
    mp.setattr(OA, "np", _NumpyWith(rint=np.floor))


def _mut_drop_inv_s(mp):
    orig = OA.dequant_operand
    mp.setattr(OA, "dequant_operand", lambda q, z, st, g, inv32=None: orig(q, z, st, g, None))


def _mut_alpha_grid_closed(mp):
    mp.setattr(OA, "alpha_grid", lambda n: np.arange(n, dtype=np.float64) / max(n - 1, 1))


def _mut_scale_index_reversed(mp):
    orig = OA.quantize
    mp.setattr(OA, "quantize", lambda w, s, b, g: orig(w, None if s is None else np.asarray(s)[::-1], b, g))


def _mut_zero_added_before_rounding(mp):
    def q2(w, s32, bits, group):
        q, z, step = orig(w, s32, bits, group)
        W = OA.bf16_bits_to_f64(w) if np.asarray(w).dtype == np.uint16 else w
        ws = OA.f32(W * (1.0 if s32 is None else np.asarray(s32)[None, :]))
        N, K = ws.shape
        qmax = (1 << bits) - 1
        G = ws.reshape(N, K // group, group)
        qq = np.clip(np.floor(OA.f32(G / step[:, :, None]) + z[:, :, None] + 0.5), 0, qmax)
        return qq.reshape(N, K).astype(np.int64), z, step
    orig = OA.quantize
    mp.setattr(OA, "quantize", q2)


def _mut_loss_sign(mp):
    def mse(x_bits, w_bits, b_values, chunk_rows=4096):
        X = OA.bf16_bits_to_f64(x_bits)
        D = np.asarray(b_values) + OA.bf16_bits_to_f64(w_bits)
        E = X @ D.T
        return float((E * E).sum()) / E.size
    mp.setattr(OA, "output_mse", mse)


def _mut_no_range_extension(mp):
    mp.setattr(OA, "np", _NumpyWith(maximum=lambda a, b, *r: a if np.isscalar(b) else np.maximum(a, b, *r),
                                    minimum=lambda a, b, *r: a if np.isscalar(b) else np.minimum(a, b, *r)))


def _mut_stats_mean_without_abs(mp):
    mp.setattr(OA, "np", _NumpyWith(abs=lambda a: a))


def _mut_normaliser_max_only(mp):
    orig_sqrt = np.sqrt
    mp.setattr(OA, "np", _NumpyWith(sqrt=lambda v: orig_sqrt(v) * 1.5))


def _mut_decode_zero_of_first_group(mp):
    def dec(a_bits, qweight, scales, zeros, group):
        q = OA.unpack(qweight).astype(np.float64)
        z = np.asarray(zeros, np.float64)[:, :1]
        step = np.repeat(np.asarray(scales, np.float64), group, axis=1)
        return OA.bf16_bits_to_f64(a_bits) @ ((q - z) * step).T
    # The pins call the package's name for it.
    mp.setattr(oracle, "decode_gemm", dec)


def _mut_decode_rounds_weight_to_bf16(mp):
    mp.setattr(oracle, "decode_gemm", lambda a, qw, sc, ze, g: OA.deploy_gemm(a, qw, sc, ze, g))


def _mut_diff_sign(mp):
    orig = OA.diff_operand
    mp.setattr(oracle, "diff_operand", lambda w, b: -orig(w, b))


def _mut_diff_off_by_half_ulp(mp):
    # The difference left slightly off its bf16 value (a stray factor).
    mp.setattr(oracle, "diff_operand",
               lambda w, b: OA.f32(np.asarray(b, np.float64) - OA.bf16_bits_to_f64(w)) * (1 + 2.0 ** -9))


def _mut_pack3_code_bits_reversed(mp):
    orig = OA.pack3

    def p3(q):
        q = np.asarray(q, np.int64)
        rev = ((q & 1) << 2) | (q & 2) | ((q >> 2) & 1)      # bit order inside each code
        return orig(rev)
    mp.setattr(oracle, "pack3", p3)


def _mut_pack3_runs_of_16(mp):
    orig = OA.pack3

    def p3(q):
        q = np.asarray(q, np.int64)
        N, K = q.shape
        perm = np.arange(K).reshape(K // 32, 2, 16)[:, ::-1, :].reshape(K)   # halves swapped
        return orig(q[:, perm])
    mp.setattr(oracle, "pack3", p3)


def _mut_tiles_row_major_inside(mp):
    """Pieces inside a tile ordered row by row (r*4 + q) instead of lane order."""
    orig = OA.decode_tiles

    def tiles(qweight, K, dense3=False, group=128):
        t = orig(qweight, K, dense3, group)
        P = 12 if dense3 else 16
        return np.ascontiguousarray(t.reshape(-1, 4, 16, P).transpose(0, 2, 1, 3)).reshape(-1)
    mp.setattr(oracle, "decode_tiles", tiles)


def _mut_tiles_codes_in_pack_order(mp):
    """Pieces copied from the packed words unchanged (no pairing inside)."""
    def tiles(qweight, K, dense3=False, group=128):
        w = np.ascontiguousarray(np.asarray(qweight, dtype="<u4"))
        N = w.shape[0]
        G, P = K // group, (12 if dense3 else 16)
        rows = w.view(np.uint8).reshape(N, G, 4, P)
        NB = -(-N // 16)
        padded = np.zeros((NB * 16, G, 4, P), dtype=np.uint8)
        padded[:N] = rows
        return np.ascontiguousarray(padded.reshape(NB, 16, G, 4, P).transpose(0, 2, 3, 1, 4)).reshape(-1)
    mp.setattr(oracle, "decode_tiles", tiles)


def _mut_rmsnorm_without_mean(mp):
    def rms(x_bits, gamma32, eps):
        X = OA.bf16_bits_to_f64(x_bits)
        r32 = OA.f32(1.0 / np.sqrt((X * X).sum(axis=1) + eps))       # sum, not mean
        u = OA.f32(OA.f32(X * r32[:, None]) * np.asarray(gamma32, np.float64)[None, :])
        return OA.bf16_rne_bits(u), r32
    mp.setattr(oracle, "rmsnorm", rms)


def _mut_silu_is_sigmoid(mp):
    def sm(y32, F):
        Y = np.asarray(y32, np.float64)
        with np.errstate(over="ignore"):
            h = 1.0 / (1.0 + np.exp(-Y[:, :F])) * Y[:, F:2 * F]
        return OA.bf16_rne_bits(OA.f32(h))
    mp.setattr(oracle, "silu_mul", sm)


def _mut_fold_multiplies(mp):
    mp.setattr(oracle, "divide_rows",
               lambda v, s: OA.f32(np.asarray(v, np.float64) *
                                   np.asarray(s, np.float64).reshape((-1,) + (1,) * (np.ndim(v) - 1))))


def _mut_f16_ties_away(mp):
    orig = OA.f16_rne_bits

    def ties_away(x):
        # one binary32 ulp away from zero first: exact ties round away from zero
        v = np.asarray(x, np.float64).astype(np.float32)
        return orig(np.nextafter(v, np.copysign(np.float32(np.inf), v)))
    mp.setattr(OA, "f16_rne_bits", ties_away)
    mp.setattr(oracle, "f16_rne_bits", ties_away)


def _mut_quantize16_codes_with_fp32_step(mp):
    def q16(w, s32, bits, group):
        q, z, _ = OA._quantize(w, s32, bits, group, half_steps=False)
        _, _, step = OA._quantize(w, s32, bits, group, half_steps=True)
        return q, z, step
    mp.setattr(OA, "quantize16", q16)
    mp.setattr(oracle, "quantize16", q16)


def _mut_zero_nibbles_swapped(mp):
    orig = OA.pack_meta16

    def swapped(z, step16):
        sb, zb = orig(z, step16)
        return sb, ((zb >> 4) | (zb << 4)).astype(np.uint8)
    mp.setattr(OA, "pack_meta16", swapped)
    mp.setattr(oracle, "pack_meta16", swapped)


def _mut_half_step_no_clamp(mp):
    mp.setattr(OA, "F16_MIN", 0.0)


def _mut_block_deploys_on_unfolded_u(mp):
    """gate/up deployed on u instead of u_f: the gain fold 1/s1 is dropped."""
    orig = OA.divide_rows
    mp.setattr(OA, "divide_rows", lambda v, s: np.asarray(v, np.float64) if np.ndim(v) == 1 else orig(v, s))


def _mut_meta_zero_at_bit_20(mp):
    """Metadata tiles with the zero one nibble too high (bits 20..23)."""
    orig = OA.decode_meta

    def meta(steps16, zeros4, K, group=128):
        m = orig(steps16, zeros4, K, group).astype(np.uint64)
        return ((m & np.uint64(0xFFFF)) | ((m >> np.uint64(16)) << np.uint64(20))).astype(np.uint32)
    mp.setattr(oracle, "decode_meta", meta)


def _mut_meta_row_major(mp):
    """Metadata in row-major order [row][group] instead of tile order."""
    def meta(steps16, zeros4, K, group=128):
        G = K // group
        st = np.asarray(steps16, dtype=np.uint16).astype(np.uint64)
        N = st.shape[0]
        _, z = OA.unpack_meta16(steps16, zeros4, G)
        w = np.zeros((-(-N // 16) * 16, G), dtype=np.uint64)
        w[:N] = st | (z.astype(np.uint64) << np.uint64(16))
        return w.reshape(-1).astype(np.uint32)
    mp.setattr(oracle, "decode_meta", meta)


def _mut_block_up_rows_not_folded(mp):
    """The up rows' steps keep their unfolded values (1/s2 dropped)."""
    orig = OA.divide_rows
    mp.setattr(OA, "divide_rows", lambda v, s: np.asarray(v, np.float64) if np.ndim(v) == 2 else orig(v, s))


MUTATIONS = [_mut_floor_instead_of_rint, _mut_drop_inv_s, _mut_alpha_grid_closed,
             _mut_scale_index_reversed, _mut_zero_added_before_rounding, _mut_loss_sign,
             _mut_no_range_extension, _mut_stats_mean_without_abs, _mut_normaliser_max_only,
             _mut_decode_zero_of_first_group, _mut_decode_rounds_weight_to_bf16, _mut_diff_sign,
             _mut_diff_off_by_half_ulp, _mut_pack3_code_bits_reversed, _mut_pack3_runs_of_16,
             _mut_tiles_row_major_inside, _mut_tiles_codes_in_pack_order, _mut_rmsnorm_without_mean, _mut_silu_is_sigmoid,
             _mut_fold_multiplies, _mut_f16_ties_away, _mut_quantize16_codes_with_fp32_step,
             _mut_zero_nibbles_swapped, _mut_half_step_no_clamp, _mut_block_deploys_on_unfolded_u,
             _mut_block_up_rows_not_folded, _mut_meta_zero_at_bit_20, _mut_meta_row_major]

PINS = [
    P.test_quantizer_worked_group,
    P.test_quantizer_special_groups,
    P.test_stats_closed_form_constant_columns,
    P.test_alpha_grid_and_alpha0_is_identity,
    P.test_candidates_closed_form,
    P.test_candidates_floor_on_dead_channel,
    lambda: P.test_alpha0_loss_is_plain_rtn(4),
    lambda: P.test_whole_search_brute_force_tiny(24, 8, 128, 4, 20),
    lambda: P.test_whole_search_brute_force_tiny(16, 6, 256, 3, 21),
    P.test_decode_gemm_brute_force_from_words,
    P.test_decode_gemm_unit_codes_closed_form,
    lambda: P.test_difference_operand_is_exact(4),
    P.test_pack3_worked_words,
    P.test_pack3_big_integer_brute_force,
    lambda: P.test_decode_tiles_brute_force(False),
    lambda: P.test_decode_tiles_brute_force(True),
    P.test_decode_meta_brute_force,
    P.test_rmsnorm_closed_form_and_scaling,
    P.test_silu_mul_against_torch_and_identities,
    P.test_divide_rows_and_residual_against_library,
    P.test_f16_format_against_libraries,
    P.test_compact_worked_groups,
    P.test_quantize16_brute_force_nearest_level,
    P.test_quantize16_clamped_and_subnormal_steps,
    P.test_meta16_pack_brute_force_and_roundtrip,
    P.test_mlp_block_deployed_error_is_the_searched_loss,
]


@pytest.mark.parametrize("mutation", MUTATIONS, ids=lambda f: f.__name__[5:])
def test_pins_catch_planted_mistake(mutation, monkeypatch):
    # The unmutated oracle passes every pin here.
    mutation(monkeypatch)
    caught = 0
    for pin in PINS:
        try:
            pin()
        except (AssertionError, ValueError, FloatingPointError, IndexError):
            caught += 1
    assert caught >= 1, f"no pin caught {mutation.__name__}"
