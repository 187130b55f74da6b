"""CPU fp64 oracle (test infrastructure only; see awq_oracle's header)."""
from .awq_oracle import *  # noqa: F401,F403
from .awq_oracle import (SCALE_FLOOR, F16_MAX, F16_MIN, decode_gemm16, f16_bits_to_f64, f16_rne_bits, pack_meta16, packed16_bytes, quantize16, unpack_meta16, act_stats, alpha_grid, bf16_bits_to_f64,
                         bf16_rne_bits, bf16_round, candidate_scales, decode_gemm, decode_gemm3, decode_meta, decode_tiles, deploy_gemm,
                         dequant_operand, diff_operand, f32, first_argmin, gemm, gram,
                         output_mse, output_mse_gram, pack, pack3, packed3_bytes, packed_bytes, quantize,
                         search, unpack, unpack3, rmsnorm, silu_mul, divide_rows,
                         residual_add, mlp_block)
