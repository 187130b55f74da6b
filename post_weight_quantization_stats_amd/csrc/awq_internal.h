// Internal declarations shared by the host API and the kernel translation
// units of libawq_mi355x.  Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace awq {

// Only group size supported by the kernels (K is tiled in 128-wide groups).
constexpr int kGroup = 128;

// ---- W4A16 / reference GEMM tiling (also used to size SSE partials) ----
constexpr int kGemmBM = 256;
constexpr int kGemmBN = 256;

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }

inline int64_t gemm_tiles(int64_t M, int64_t N) {
  return ceil_div(M, kGemmBM) * ceil_div(N, kGemmBN);
}

// ---- activation statistics partition: R row chunks x K fp64 partials ----
struct StatsPlan {
  int64_t rows_per_block;
  int64_t row_blocks;
};
StatsPlan stats_plan(int64_t M, int64_t K);
inline size_t stats_ws_bytes(int64_t M, int64_t K) {
  return align_up((size_t)stats_plan(M, K).row_blocks * (size_t)K * sizeof(double));
}

// ---- candidate scales: r (fp64) + per-block min/max partials ----
constexpr int kScaleThreads = 256;
inline size_t scales_ws_bytes(int64_t K, int n_grid) {
  const int64_t nb = ceil_div(K, kScaleThreads);
  return align_up((size_t)n_grid * K * sizeof(double)) +
         align_up((size_t)n_grid * nb * 2 * sizeof(double));
}

// ---- launchers (each returns the launch's hipError_t) ----
hipError_t launch_act_stats(const uint16_t* x, int64_t M, int64_t K, float* mean_abs,
                            double* partial, hipStream_t stream);

hipError_t launch_candidate_scales(const float* mean_abs, int64_t K, int n_grid, float* s,
                                   float* inv_s, void* ws, hipStream_t stream);

// s_sel: when non-NULL, the scale row used is s + max(*s_sel, 0) * K.
hipError_t launch_quantize_pack(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                const int32_t* s_sel, int bits, uint32_t* qweight,
                                float* scales, uint8_t* zeros, hipStream_t stream);

// INT3 codes of W . diag(s) in the dense layout (32 codes in three u32 words).
hipError_t launch_quantize_pack3(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                 uint32_t* qweight3, float* scales, uint8_t* zeros,
                                 hipStream_t stream);

// Compact deployment format: the fp32 step limited to [2^-24, 65504] and
// rounded to binary16 before zero and codes; steps16 [N][G] binary16, zeros4
// [N][ceil(G/2)] two per byte (even group low).  Codes as launch_quantize_pack
// (4-bit containers, bits 3 or 4) or, int3_dense, as launch_quantize_pack3.
hipError_t launch_quantize_pack16(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                  int bits, bool int3_dense, uint32_t* qweight, uint16_t* steps16,
                                  uint8_t* zeros4, hipStream_t stream);
// Compact metadata -> fp32 steps and u8 zeros [N][G] (exact).
hipError_t launch_expand_meta16(const uint16_t* steps16, const uint8_t* zeros4, int64_t N,
                                int64_t G, float* scales, uint8_t* zeros, hipStream_t stream);

// The search's bf16 weight operand for one candidate:
// b_out[n][k] = bf16(f32(f32((q - z) * step) * inv_s[k])) (inv_s NULL: no factor).
hipError_t launch_quantize_dequant(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                   const float* inv_s, int bits, uint16_t* b_out,
                                   hipStream_t stream);

// bf16(B - W) as bf16 [N][K] (exact: see quantize_pack.hip).
hipError_t launch_quantize_diff_operand(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                        const float* inv_s, int bits, uint16_t* d_out,
                                        hipStream_t stream);
// Candidate difference for the Gram-form loss: d32[n][k] = B - W (fp32) and
// a_split[n] = [D | D] (bf16 [N][2K]).
hipError_t launch_quantize_diff(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                const float* inv_s, int bits, uint16_t* a_split, float* d32,
                                hipStream_t stream);

// Packed codes (4-bit containers [N][K/8], or dense INT3 [N][3K/32]) -> the
// bf16 operand b[n][k] = bf16(f32(f32((q - z) * step) * inv_s[k])) (inv_s
// NULL: no factor), as the fused W4A16 kernel dequantizes it.
hipError_t launch_dequant_packed(const uint32_t* qweight, const float* scales,
                                 const uint8_t* zeros, const float* inv_s, int64_t N, int64_t K,
                                 bool int3_dense, uint16_t* b, hipStream_t stream);

// ---- Gram form: X^T (bf16 [K][Mp], zero-padded) and the split G operand ----
int64_t gram_padded_m(int64_t M);
hipError_t launch_transpose_pad(const uint16_t* x, int64_t M, int64_t K, uint16_t* xt,
                                hipStream_t stream);
hipError_t launch_gram_split(const float* g, int64_t K, uint16_t* out, hipStream_t stream);

// ---- ops of the synthetic feed-forward block around the search ----
hipError_t launch_rmsnorm(const uint16_t* x, int64_t M, int64_t K, const float* gamma,
                          double eps, uint16_t* u, float* r, hipStream_t stream);
hipError_t launch_silu_mul(const float* y, int64_t M, int64_t F, uint16_t* h, hipStream_t stream);
hipError_t launch_divide_rows(const float* v, int64_t R, int64_t C, const float* s, float* out,
                              hipStream_t stream);
hipError_t launch_residual_add(const uint16_t* x, const float* y, int64_t n, uint16_t* out,
                               hipStream_t stream);

struct GemmOperands {
  const uint16_t* x;        // bf16 [M][K]
  int64_t M, N, K;
  // exactly one of: w (bf16 [N][K]) or the packed triple
  const uint16_t* w;
  const uint32_t* qweight;   // u32 [N][K/8], or with int3_dense u32 [N][3K/32]
  const float* scales;
  const uint8_t* zeros;
  bool int3_dense;          // packed codes in the dense INT3 layout
  const float* inv_s;       // [K] or NULL
  const float* y_ref;       // [M][N] or NULL
  float* y;                 // [M][N] or NULL
  double* partials;         // [tiles] fp64 SSE per tile, or NULL
  bool dot;                 // bf16 operand: partials hold sum(Y * y_ref) instead
  bool sq;                  // bf16 operand: partials hold sum(Y^2); y_ref unused
};
hipError_t launch_gemm(const GemmOperands& op, hipStream_t stream);

// ---- decode-shaped W4A16 contraction (M <= 64) ----
constexpr int64_t kDecodeMaxM = 64;
struct DecodePlan {
  int64_t groups_per_split;
  int64_t splits;
  bool cols;                // the column-split kernel (waves split columns, not K)
  int col_blocks;           // 16-column blocks per workgroup (1, 2 or 4), or per wave (cols: 2)
  int token_blocks;         // 16-token blocks per workgroup: 1 or 2 (cols: 2 or 4)
  size_t ws_bytes;          // fp32 partials [splits][M][N] when splits > 1
};
DecodePlan decode_plan(int64_t M, int64_t N, int64_t K);
// int3_dense: qweight holds dense INT3 words [N][3K/32] instead of 4-bit
// containers [N][K/8].
// tiled: qweight holds decode tiles (launch_decode_tiles) instead of row-major words.
hipError_t launch_decode_gemm(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                              const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                              float* y, void* ws, hipStream_t stream, bool int3_dense = false,
                              bool tiled = false);
// The decode contraction on decode tiles with the compact metadata.
hipError_t launch_decode_gemm16(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                const uint32_t* tiles, const uint16_t* steps16,
                                const uint8_t* zeros4, float* y, void* ws, hipStream_t stream,
                                bool int3_dense);
// The decode contraction on decode tiles with metadata tiles (launch_decode_meta).
hipError_t launch_decode_gemm_meta(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                   const uint32_t* tiles, const uint32_t* meta, float* y, void* ws,
                                   hipStream_t stream, bool int3_dense);
// Metadata tiles: u32 [ceil(N/16)][G][16], word r of tile b*G + g = binary16
// step of row 16b + r, group g, in bits 0..15 and its zero in bits 16..19
// (0 past N), from the compact metadata.
size_t decode_meta_bytes(int64_t N, int64_t K);
hipError_t launch_decode_meta(const uint16_t* steps16, const uint8_t* zeros4, int64_t N,
                              int64_t K, uint32_t* meta, hipStream_t stream);
// Decode tiles: rows 16b .. 16b+15 (zero past N) x group g as tile b*G + g,
// row r's piece for channels 32q .. 32q+31 at byte P*(r + 16q) (P = 16 or 12).
size_t decode_tiles_bytes(int64_t N, int64_t K, bool int3_dense);
hipError_t launch_decode_tiles(const uint32_t* qweight, int64_t N, int64_t K, bool int3_dense,
                               uint32_t* tiles, hipStream_t stream);

// Measured ceilings (ceilings.hip): matrix cores fed from registers, and
// streaming copy (mode 0), read (1) and write (2) kernels.
hipError_t launch_mfma_ceiling(int blocks, int iters, bool zero, float* sink, hipStream_t stream);
int64_t mfma_ceiling_flops(int blocks, int iters);
hipError_t launch_stream_ceiling(int mode, const void* src, void* dst, size_t bytes, int blocks,
                                 hipStream_t stream);

// Static scratch of the entry point that allocates nothing: its size, and
// the device address of the current device's copy (looked up once per device
// with hipGetSymbolAddress; see noalloc.hip).
constexpr size_t kNoallocScratchBytes = size_t(16) << 20;
hipError_t noalloc_scratch(void** ptr);

// losses[i] = (sum_t partials[i*T + t]) / divisor, fixed summation order.
hipError_t launch_loss_reduce(const double* partials, int64_t T, int n_grid, double divisor,
                              double* losses, hipStream_t stream);
hipError_t launch_argmin(const double* losses, int n_grid, int32_t* best, hipStream_t stream);
hipError_t launch_select_row(const float* s, const int32_t* sel, int64_t K, float* out,
                             hipStream_t stream);
hipError_t launch_fill_f64(double* p, int64_t n, double v, hipStream_t stream);

}  // namespace awq
