/*
 * awq_mi355x.h -- C ABI of the AWQ per-layer scale search on AMD Instinct
 * MI355X (gfx950).
 *
 * AWQ (activation-aware weight quantization) picks, for each linear layer, a
 * per-input-channel scale s from calibration activation statistics, multiplies
 * the weight by s and divides the activation by it (the product is unchanged),
 * chooses s by a grid search that minimises the layer's output error, then
 * quantizes the scaled weight group-wise to 4 (or 3) bits and writes the
 * packed integers.  Sources, by page and section:
 *   robotsatlas.com AWQ page: "How it works", "Key mechanisms", "Components",
 *     "Hyperparameters", "Computational complexity";
 *   builderai.tools AWQ page: "About" (real INT4 weights, W4A16 kernels);
 *   aquanode.io "What is AWQ?": "The core idea".
 *
 * Conventions for every call
 *   - bf16 tensors are passed as uint16_t bit patterns; all tensors are dense,
 *     row-major, contiguous.  X is [M][K] (tokens x input channels), W is
 *     [N][K] (output channels x input channels, so Y = X . W^T).
 *   - Every pointer except `stream` is a DEVICE pointer.  `stream` is a
 *     hipStream_t passed as void* (NULL = the default stream).
 *   - The caller owns all memory: inputs, outputs and the workspace.  The
 *     library never allocates, frees or synchronises.  A call validates its
 *     arguments on the host, enqueues kernels on `stream` and returns; outputs
 *     are valid once the stream has completed; inputs must stay unchanged
 *     until then.  Calls on different streams that share an output race.
 *   - On any validation error nothing is enqueued and no HIP call is made.
 *   - Pointers to bf16/f32/u32 tensors with more than one element must be
 *     16-byte aligned (AWQ_ERR_ALIGN otherwise), except where a call states
 *     a weaker requirement (dense INT3 words, scales, sse).
 *   - group must be 128 and bits 3 or 4 (AWQ_ERR_UNSUPPORTED otherwise); K must
 *     be a positive multiple of group, at most 2^22, and the contractions
 *     take N <= 2^22 (AWQ_ERR_SHAPE otherwise: tiles are addressed with 32-bit
 *     byte offsets).
 *   - Inputs must be finite; NaN/Inf in X or W give unspecified codes and
 *     non-finite losses (the search then never selects a NaN loss).
 *   - No C++ exception crosses this boundary.  awq_last_error() returns a
 *     thread-local message for the last failing call on this thread.
 *
 * Packed weight format (the "real INT4 weights")
 *   qweight u32 [N][K/8]: code of (n, k) in word k/8 at bits 4*(k%8);
 *                         3-bit codes use the same 4-bit containers.
 *   scales  f32 [N][K/group]: quantization step of each group.
 *   zeros   u8  [N][K/group]: integer zero point of each group.
 *   Dequantized weight: (code - zero) * step.
 *   Dense INT3 (awq_quantize_pack3; sourcepulse AWQ project page: 3-bit
 *   weights): qweight3 u32 [N][3K/32], each run of 32 codes along K one
 *   96-bit little-endian value with code i at bits 3i, in three words.
 *   Compact deployment metadata (awq_quantize_pack16): binary16 steps and
 *   two 4-bit zeros per byte.
 */
#ifndef AWQ_MI355X_H
#define AWQ_MI355X_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AWQ_ABI_VERSION 1

typedef enum awq_status {
  AWQ_OK = 0,
  AWQ_ERR_NULL = 1,         /* a required pointer is NULL                          */
  AWQ_ERR_SHAPE = 2,        /* a size is out of range or inconsistent              */
  AWQ_ERR_UNSUPPORTED = 3,  /* bits, group or n_grid outside the supported set     */
  AWQ_ERR_ALIGN = 4,        /* a tensor pointer is not 16-byte aligned             */
  AWQ_ERR_WORKSPACE = 5,    /* workspace missing or smaller than awq_workspace_size */
  AWQ_ERR_LAUNCH = 6,       /* the HIP runtime reported an error (see awq_last_error) */
} awq_status;

typedef enum awq_op {
  AWQ_OP_ACT_STATS = 0,
  AWQ_OP_W4A16_GEMM = 1,
  AWQ_OP_SEARCH_SCALE = 2,
  AWQ_OP_CANDIDATE_SCALES = 3,
  AWQ_OP_DECODE_GEMM = 4,
  AWQ_OP_CANDIDATE_SSE = 5,
  AWQ_OP_SEARCH_SCALE_GRAM = 6,
  AWQ_OP_W4A16_GEMM_STAGED = 7,
} awq_op;

/* Packed code layouts of the deployment contraction. */
typedef enum {
  AWQ_LAYOUT_NIBBLE = 0,      /* awq_quantize_pack: codes in 4-bit fields, [N][K/8] words */
  AWQ_LAYOUT_INT3_DENSE = 1,  /* awq_quantize_pack3: 32 codes in 3 words, [N][3K/32] words */
} awq_layout;

/* Version of this ABI (AWQ_ABI_VERSION). */
int32_t awq_abi_version(void);

/* Static, human-readable name of a status code. */
const char* awq_status_string(int32_t status);

/* Message for the last failing call on the calling thread ("" if none). */
const char* awq_last_error(void);

/*
 * Bytes of device workspace a call needs (0 means ws may be NULL).
 *   op AWQ_OP_ACT_STATS:    uses M, K.
 *   op AWQ_OP_W4A16_GEMM:   uses M, N, K (needed only when sse is requested).
 *   op AWQ_OP_SEARCH_SCALE: uses M, N, K, bits, group, n_grid.
 *   op AWQ_OP_CANDIDATE_SCALES: uses K, n_grid.
 *   op AWQ_OP_DECODE_GEMM:  uses M, N, K, bits, group (0 bytes when K is not
 *                           split across workgroups).
 *   op AWQ_OP_CANDIDATE_SSE: uses M, N.
 *   op AWQ_OP_SEARCH_SCALE_GRAM: uses M, N, K, bits, group, n_grid.
 *   op AWQ_OP_W4A16_GEMM_STAGED: uses M, N, K, bits, group (2*N*K bytes of
 *                           dequantized operand plus per-tile partials).
 * Errors: AWQ_ERR_NULL (bytes NULL), AWQ_ERR_SHAPE, AWQ_ERR_UNSUPPORTED.
 */
awq_status awq_workspace_size(int32_t op, int64_t M, int64_t N, int64_t K, int32_t bits,
                              int32_t group, int32_t n_grid, size_t* bytes);

/*
 * Activation statistics (robotsatlas "How it works", "Components" / activation
 * saliency analysis: activation magnitudes measured at the layer input over a
 * calibration set).  Statistic: mean_abs[k] = (1/M) sum_m |x[m,k]|, summed in
 * fp64 in a fixed order, returned rounded to fp32.
 *   x        bf16 [M][K]  calibration activations (M >= 1, K % 8 == 0)
 *   mean_abs f32  [K]     output
 *   ws       device workspace of awq_workspace_size(AWQ_OP_ACT_STATS) bytes
 */
awq_status awq_act_stats(const uint16_t* x, int64_t M, int64_t K, float* mean_abs, void* ws,
                         size_t ws_bytes, void* stream);

/*
 * Candidate scales of the grid search (robotsatlas "How it works": a scaling
 * factor per input channel derived from the activation statistic; "Key
 * mechanisms": grid search over scales).  For i = 0..n_grid-1, alpha = i/n_grid:
 *   r[k] = max(mean_abs[k]^alpha, 1e-4)        (fp64; 0^0 = 1)
 *   s[i][k] = fp32(r[k] / sqrt(max_k r * min_k r))
 *   inv_s[i][k] = fp32(1 / s[i][k])
 *   mean_abs f32 [K] (non-negative); s, inv_s f32 [n_grid][K] outputs.
 *   1 <= n_grid <= 64.  ws: awq_workspace_size(AWQ_OP_CANDIDATE_SCALES) bytes.
 */
awq_status awq_candidate_scales(const float* mean_abs, int64_t K, int32_t n_grid, float* s,
                                float* inv_s, void* ws, size_t ws_bytes, void* stream);

/*
 * Group-wise asymmetric quantization and packing of W . diag(s) (robotsatlas
 * "How it works": weights quantized group-wise after the scales are set;
 * "Components": groups of 128 with a per-group scale; "Hyperparameters": 4 or
 * 3 bits; builderai "About": real INT4 weights are written).  Per row n and
 * group j (input channels j*group .. j*group+group-1), each step one IEEE
 * fp32 operation:
 *   ws   = w[n,k] * s[k]                     (s NULL means s = 1)
 *   mx   = max(max ws, 0);  mn = min(min ws, 0)
 *   step = (mx - mn) / qmax, replaced by 1 when it is 0   (qmax = 2^bits - 1)
 *   z    = clamp(rint(-mn / step), 0, qmax)
 *   q    = clamp(rint(ws / step) + z, 0, qmax)     (rint: ties to even)
 *   w     bf16 [N][K];  s f32 [K] or NULL
 *   qweight u32 [N][K/8], scales f32 [N][K/group], zeros u8 [N][K/group]
 * N == 0 is a no-op (pointers are then ignored).
 */
awq_status awq_quantize_pack(const uint16_t* w, int64_t N, int64_t K, const float* s, int32_t bits,
                             int32_t group, uint32_t* qweight, float* scales, uint8_t* zeros,
                             void* stream);

/*
 * The same quantization with 3-bit codes written densely (sourcepulse AWQ
 * project page, opening paragraph: 3- and 4-bit weights), so the codes take
 * 3 bits per weight instead of a 4-bit container: each run of 32 codes along
 * K is one 96-bit little-endian value, code i at bits 3i .. 3i+2, stored as
 * three u32 words.  Steps and zeros as awq_quantize_pack with bits = 3.
 *   w bf16 [N][K], s f32 [K] or NULL (s = 1)
 *   qweight3 u32 [N][3K/32] (4-byte aligned), scales f32 [N][K/group],
 *   zeros u8 [N][K/group].  N == 0 is a no-op.
 */
awq_status awq_quantize_pack3(const uint16_t* w, int64_t N, int64_t K, const float* s,
                              int32_t group, uint32_t* qweight3, float* scales, uint8_t* zeros,
                              void* stream);

/*
 * Dequantized weight operand of one candidate scale, the search's inner step
 * (robotsatlas "How it works": the weight is scaled by s, quantized
 * group-wise, and the activation divided by s; here 1/s is folded into the
 * dequantized weight, which leaves the product unchanged).  Quantizes
 * W . diag(s) exactly as awq_quantize_pack does and writes
 *   b[n][k] = bf16( f32( f32((q - z) * step) * inv_s[k] ) )   (RNE to bf16)
 * (inv_s NULL: no factor).  w bf16 [N][K]; s, inv_s f32 [K] (s NULL means 1);
 * b bf16 [N][K] output.  N == 0 is a no-op (pointers are then ignored).
 */
awq_status awq_dequant_operand(const uint16_t* w, int64_t N, int64_t K, const float* s,
                               const float* inv_s, int32_t bits, int32_t group, uint16_t* b,
                               void* stream);

/*
 * Difference operand of one candidate scale: the search's weight operand
 * minus the original weight, so that X . D^T is the candidate's output error
 * X . B^T - X . W^T directly (robotsatlas "How it works": the scale minimises
 * the error between the quantized and the original layer outputs).
 *   d[n][k] = bf16( f32(b[n][k] - w[n][k]) )   (RNE to bf16)
 * with b exactly as awq_dequant_operand writes it.  The rounding is exact: a
 * nonzero b has |w s| >= step / 2, so b and w share a sign and b / w lies in
 * [1/2, 2] (up to the roundings of s and 1/s); by Sterbenz's lemma their
 * difference is a bf16 value.  Arguments as for awq_dequant_operand; d bf16
 * [N][K] output.  N == 0 is a no-op (pointers are then ignored).
 */
awq_status awq_diff_operand(const uint16_t* w, int64_t N, int64_t K, const float* s,
                            const float* inv_s, int32_t bits, int32_t group, uint16_t* d,
                            void* stream);

/*
 * Dense reference product Y = X . W^T (robotsatlas "How it works": the output
 * error is measured against the layer's unquantized output).  bf16 operands,
 * fp32 accumulation on the matrix cores, fp32 output.
 *   x bf16 [M][K], w bf16 [N][K], y f32 [M][N].  M == 0 or N == 0 is a no-op
 *   (pointers are then ignored).
 */
awq_status awq_reference_gemm(const uint16_t* x, int64_t M, int64_t N, int64_t K,
                              const uint16_t* w, float* y, void* stream);

/*
 * Squared output error of one candidate (robotsatlas "How it works": the
 * scale is chosen by a grid search that minimises the layer's output error):
 *   sse = sum over m, n of ( (X . B^T)[m, n] - y_ref[m, n] )^2
 * with bf16 X [M][K] and B [N][K] (a candidate's operand from
 * awq_dequant_operand), fp32 accumulation on the matrix cores, and the error
 * reduced in fp64 in a fixed order (bit-reproducible).  The product is never
 * written to memory.  y_ref f32 [M][N], or NULL for sse = sum (X . B^T)^2
 * (B then a difference operand from awq_diff_operand: the search's form);
 * sse f64 [1];
 * ws: awq_workspace_size(AWQ_OP_CANDIDATE_SSE) bytes.  M == 0 or N == 0 sets
 * sse to 0.
 */
awq_status awq_candidate_sse(const uint16_t* x, int64_t M, int64_t N, int64_t K, const uint16_t* b,
                             const float* y_ref, double* sse, void* ws, size_t ws_bytes,
                             void* stream);

/*
 * W4A16 contraction with the packed weights (builderai "About": kernels for
 * 4-bit weights with 16-bit activations; robotsatlas "Implementation
 * pitfalls": dequantization stays inside the kernel).  The weight operand is
 *   B[n,k] = bf16( fp32( fp32((q - z) * step) * inv_s[k] ) )
 * (inv_s NULL: B = bf16(fp32((q - z) * step))), dequantized on chip and never
 * written to memory; Y = X . B^T with bf16 inputs and fp32 accumulation.
 *   x       bf16 [M][K];  qweight/scales/zeros as from awq_quantize_pack
 *   inv_s   f32 [K] or NULL
 *   y       f32 [M][N] output, or NULL
 *   y_ref   f32 [M][N] or NULL;  sse f64 [1] or NULL.  If sse is given, y_ref
 *           is required and sse = sum over m,n of (Y[m,n] - y_ref[m,n])^2,
 *           reduced in fp64 in a fixed order (bit-reproducible).
 *   ws      workspace of awq_workspace_size(AWQ_OP_W4A16_GEMM) bytes when sse
 *           is requested, else may be NULL.
 * At least one of y and sse must be non-NULL.  When M or N is 0 every pointer
 * but sse is ignored and sse (if given) is set to 0.
 */
awq_status awq_w4a16_gemm(const uint16_t* x, int64_t M, int64_t N, int64_t K,
                          const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                          int32_t bits, int32_t group, const float* inv_s, const float* y_ref,
                          float* y, double* sse, void* ws, size_t ws_bytes, void* stream);

/*
 * The same fused contraction on dense INT3 codes (sourcepulse AWQ project
 * page, opening paragraph: 3- and 4-bit weights; robotsatlas "Implementation
 * pitfalls": dequantization stays inside the kernel).  Each k-step's 32 codes
 * of a weight row come as one 12-byte run and are widened on chip to the
 * 4-bit fields the dequantization reads, so for the same codes Y and sse are
 * bit-identical to awq_w4a16_gemm on the 4-bit containers.
 *   qweight3  u32 [N][3K/32] as from awq_quantize_pack3 (each run of 32 codes
 *             along K one 96-bit little-endian value, code i at bits 3i),
 *             4-byte aligned; scales/zeros f32/u8 [N][K/group]
 *   other arguments, outputs, workspace (awq_workspace_size(AWQ_OP_W4A16_GEMM))
 *   and the M == 0 / N == 0 rule as awq_w4a16_gemm with bits = 3
 */
awq_status awq_w3a16_gemm(const uint16_t* x, int64_t M, int64_t N, int64_t K,
                          const uint32_t* qweight3, const float* scales, const uint8_t* zeros,
                          int32_t group, const float* inv_s, const float* y_ref, float* y,
                          double* sse, void* ws, size_t ws_bytes, void* stream);

/*
 * The same W4A16 product for many tokens, from codes in either packed layout
 * (builderai "About": 4-bit weights with 16-bit activations; sourcepulse AWQ
 * project page, opening paragraph: 3- and 4-bit weights).  The operand
 *   B[n,k] = bf16( fp32( fp32((q - z) * step) * inv_s[k] ) )
 * (the one awq_w4a16_gemm forms in LDS) is written once per call into the
 * workspace by a streaming kernel, then contracted on the bf16 matrix cores:
 * each weight is dequantized once instead of once per 256-row tile of X,
 * which pays once X has more than a few hundred rows.  Same operand as
 * awq_w4a16_gemm, contracted on the 16x16x32 matrix-core form (that one
 * uses 32x32x16): Y agrees with it to fp32 rounding of the sums, not bit
 * for bit; dense INT3 and the same codes in 4-bit containers give the same
 * Y bit for bit.
 *   layout  AWQ_LAYOUT_NIBBLE: qweight u32 [N][K/8] (awq_quantize_pack, bits
 *           3 or 4); AWQ_LAYOUT_INT3_DENSE: qweight u32 [N][3K/32]
 *           (awq_quantize_pack3, bits 3); 4-byte aligned.
 *   other arguments, outputs and the M == 0 / N == 0 rule as awq_w4a16_gemm
 *   ws      awq_workspace_size(AWQ_OP_W4A16_GEMM_STAGED) bytes, always
 *           required (it holds the 2*N*K-byte operand).
 */
awq_status awq_w4a16_gemm_staged(const uint16_t* x, int64_t M, int64_t N, int64_t K,
                                 const uint32_t* qweight, const float* scales,
                                 const uint8_t* zeros, int32_t bits, int32_t group,
                                 int32_t layout, const float* inv_s, const float* y_ref, float* y,
                                 double* sse, void* ws, size_t ws_bytes, void* stream);

/*
 * Decode-shaped W4A16 contraction for 1 <= M <= 64 tokens, the deployment
 * case (builderai "About": kernels for 4-bit weights with 16-bit activations;
 * robotsatlas "Implementation pitfalls": the speedup needs a kernel that reads
 * the packed weights directly; "Limitations": the benefit depends on matched
 * INT4 kernels).  Streams the packed weights once:
 *   y[m][n] = sum_k a[m][k] * (q[n][k] - zeros[n][k/group]) * scales[n][k/group]
 * The dequantized weight is the exact product (q - z) * step (not rounded to
 * bf16); products are exact and sums are fp32.
 *   a       bf16 [M][K] activations (already divided by the search's s, as
 *           the caller folds it)
 *   qweight/scales/zeros as from awq_quantize_pack, bits 3 or 4
 *   y       f32 [M][N] output
 *   ws      awq_workspace_size(AWQ_OP_DECODE_GEMM) bytes (fp32 partials
 *           when K is split across workgroups: up to 8 tokens when
 *           K > 8192, or K > 16384 for M <= 6; above 8 tokens when K > 8192
 *           or the layer is too narrow to fill the chip without a split;
 *           0 otherwise, and ws may then be NULL).
 * M > 64 gives AWQ_ERR_SHAPE (use awq_w4a16_gemm).  M == 0 or N == 0 is a
 * no-op.  Results are bit-reproducible for a given (M, N, K).
 */
awq_status awq_w4a16_decode_gemm(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                 const uint32_t* qweight, const float* scales,
                                 const uint8_t* zeros, int32_t bits, int32_t group, float* y,
                                 void* ws, size_t ws_bytes, void* stream);

/*
 * The same decode-shaped contraction on dense INT3 weights (the layout of
 * awq_quantize_pack3): 0.375 bytes of codes per weight instead of 0.5.
 * Arguments, limits, workspace (awq_workspace_size(AWQ_OP_DECODE_GEMM)) and
 * results as awq_w4a16_decode_gemm with bits = 3; qweight3 u32 [N][3K/32],
 * 4-byte aligned.  For the same codes the result is bit-identical to
 * awq_w4a16_decode_gemm on the 4-bit containers.
 */
awq_status awq_w3a16_decode_gemm(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                 const uint32_t* qweight3, const float* scales,
                                 const uint8_t* zeros, int32_t group, float* y, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * Decode tiles: the packed words rearranged once, at load time, for the
 * deployment contraction (robotsatlas "Limitations": the benefit depends on
 * matched INT4 kernels).  Rows 16b .. 16b+15 of group g (rows past N are
 * zero) form tile b*G + g; inside it, row r's piece covering the group's
 * channels 32q .. 32q+31 (P = 16 bytes for AWQ_LAYOUT_NIBBLE, 12 for
 * AWQ_LAYOUT_INT3_DENSE) sits at byte P*(r + 16q), so one wave's load of a
 * tile is one contiguous piece in lane order.  Inside a piece channels 2p
 * and 2p+1 form pair p: AWQ_LAYOUT_NIBBLE puts pair 4j+t in nibbles t and
 * 4+t of u32 word j; AWQ_LAYOUT_INT3_DENSE puts pair p < 15 at bits 3(p%5)
 * and 16+3(p%5) of word p/5, and bit i of channel 30's and 31's codes at
 * bits 15 and 31 of word i.
 *   awq_decode_tiles_size: *bytes = ceil(N/16) * 16 * (K/2 or 3K/8).
 *   awq_decode_tiles: qweight as written by awq_quantize_pack (layout
 *     NIBBLE, any bits) or awq_quantize_pack3 (INT3_DENSE), 4-byte aligned;
 *     tiles output of that size, 16-byte aligned.  N == 0 is a no-op.
 */
awq_status awq_decode_tiles_size(int64_t N, int64_t K, int32_t layout, int32_t group,
                                 size_t* bytes);
awq_status awq_decode_tiles(const uint32_t* qweight, int64_t N, int64_t K, int32_t layout,
                            int32_t group, uint32_t* tiles, void* stream);

/*
 * The decode-shaped contraction reading decode tiles: arguments, limits,
 * workspace and results as awq_w4a16_decode_gemm (layout NIBBLE) or
 * awq_w3a16_decode_gemm (INT3_DENSE), bit-identical to them for the same
 * codes.  The tiles must be at most 4 GiB (32-bit offsets); larger gives
 * AWQ_ERR_SHAPE.
 */
awq_status awq_decode_gemm_tiled(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                 const uint32_t* tiles, const float* scales, const uint8_t* zeros,
                                 int32_t layout, int32_t group, float* y, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * awq_decode_gemm_tiled for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  Arguments, limits and results as awq_decode_gemm_tiled
 * (bit-identical to it), without the workspace: the K-split partials go to a
 * scratch array owned by the library, 16 MiB per GPU (a static device array,
 * held by each GPU the library runs on until the process ends).  The call
 * itself allocates and frees nothing.  The partials take
 * awq_workspace_size(AWQ_OP_DECODE_GEMM) bytes (splits x M x N x 4); a shape
 * that needs more than 16 MiB gives AWQ_ERR_WORKSPACE (the Llama-2-70B down
 * projection at 64 tokens, 8192 x 28672, needs 8 MiB).  Every call
 * on one GPU shares that GPU's scratch: calls that overlap in time on one GPU
 * (two streams, two threads) race and must be serialised by the caller.
 * Nothing in the scratch needs clearing: each call overwrites every partial
 * it reads.
 */
awq_status awq_decode_gemm_tiled_noalloc(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                         const uint32_t* tiles, const float* scales,
                                         const uint8_t* zeros, int32_t layout, int32_t group,
                                         float* y, void* stream);

/*
 * Compact deployment format: 16-bit steps and 4-bit zeros (2.5 bytes of
 * metadata per group instead of 5; robotsatlas "Components": a scale per
 * group of 128; builderai "About": real low-bit weights are written).  The
 * final pack at the chosen s, with the step rounded before the codes:
 *   step  = as awq_quantize_pack, then limited to [2^-24, 65504] (a NaN step
 *           becomes 2^-24) and rounded to IEEE binary16 (nearest, ties to
 *           even)
 *   z, q  = as awq_quantize_pack, computed with that step
 *   w bf16 [N][K]; s f32 [K] or NULL (s = 1); bits 3 or 4
 *   layout AWQ_LAYOUT_NIBBLE: qweight u32 [N][K/8] (16-byte aligned) as
 *     awq_quantize_pack; AWQ_LAYOUT_INT3_DENSE (bits 3): qweight u32
 *     [N][3K/32] (4-byte aligned) as awq_quantize_pack3
 *   steps16 binary16 bit patterns [N][K/group] (2-byte aligned)
 *   zeros4  u8 [N][ceil(G/2)], G = K/group: group 2j in the low nibble of
 *     byte j, group 2j+1 in the high nibble (0 past the last group)
 * N == 0 is a no-op.
 */
awq_status awq_quantize_pack16(const uint16_t* w, int64_t N, int64_t K, const float* s,
                               int32_t bits, int32_t group, int32_t layout, uint32_t* qweight,
                               uint16_t* steps16, uint8_t* zeros4, void* stream);

/*
 * Compact metadata -> scales f32 [N][K/group] and zeros u8 [N][K/group]
 * (exact), for the contractions that take those (awq_w4a16_gemm with many
 * tokens).  N == 0 is a no-op.
 */
awq_status awq_expand_meta16(const uint16_t* steps16, const uint8_t* zeros4, int64_t N, int64_t K,
                             int32_t group, float* scales, uint8_t* zeros, void* stream);

/*
 * The decode-shaped contraction on decode tiles with the compact metadata
 * (awq_quantize_pack16): arguments, limits, workspace and results as
 * awq_decode_gemm_tiled, with steps16 (2-byte aligned) and zeros4 in place
 * of scales and zeros.  Bit-identical to awq_decode_gemm_tiled on the
 * expanded metadata.
 */
awq_status awq_decode_gemm_tiled16(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                   const uint32_t* tiles, const uint16_t* steps16,
                                   const uint8_t* zeros4, int32_t layout, int32_t group, float* y,
                                   void* ws, size_t ws_bytes, void* stream);

/*
 * Metadata tiles: the compact metadata (awq_quantize_pack16) rearranged like
 * the decode tiles, so that the decode contraction reads each row's step and
 * zero with its codes (robotsatlas "Implementation pitfalls": the benefit
 * needs matched INT4 kernels).  u32 [ceil(N/16)][K/group][16]: word r of
 * tile b*G + g holds the binary16 step of row 16b + r and group g in bits
 * 0..15 and its zero in bits 16..19, bits 20..31 clear; rows past N are 0.
 *   awq_decode_meta_size: *bytes = ceil(N/16) * 16 * (K/group) * 4.
 *   awq_decode_meta: steps16 (2-byte aligned) and zeros4 as written by
 *     awq_quantize_pack16; meta output of that size, 4-byte aligned.
 *     N == 0 is a no-op.
 */
awq_status awq_decode_meta_size(int64_t N, int64_t K, int32_t group, size_t* bytes);
awq_status awq_decode_meta(const uint16_t* steps16, const uint8_t* zeros4, int64_t N, int64_t K,
                           int32_t group, uint32_t* meta, void* stream);

/*
 * The decode-shaped contraction on decode tiles and metadata tiles:
 * arguments, limits, workspace and results as awq_decode_gemm_tiled16, with
 * meta (awq_decode_meta, 4-byte aligned) in place of steps16 and zeros4.
 * Bit-identical to awq_decode_gemm_tiled16 on the compact metadata the tiles
 * were made from.
 */
awq_status awq_decode_gemm_tiled_meta(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                      const uint32_t* tiles, const uint32_t* meta, int32_t layout,
                                      int32_t group, float* y, void* ws, size_t ws_bytes,
                                      void* stream);

/*
 * Measured ceilings of the GPU, so that each kernel can be reported as a
 * fraction of what the part sustains as well as of its spec (the
 * measurement of the path: GEMM TFLOP/s against the matrix cores' peak,
 * streaming kernels against the copy ceiling).  Not steps of the method;
 * time them with events on the given stream.
 *   awq_ceiling_mfma: `blocks` workgroups of 8 waves, each wave issuing
 *     iters x 32 v_mfma_f32_16x16x32_bf16 on operands held in registers (the
 *     search contraction's 128x64 wave tile), pseudo-random bf16 operands
 *     of magnitude 1..2, or zeros when zero_operands != 0 (the part is
 *     power-limited, so data sets the clock).  *flops (host) receives the
 *     flops of the launch.  sink: a device float, never written in
 *     practice.  1 <= blocks <= 65536, 1 <= iters <= 2^20.
 *   awq_ceiling_stream: mode AWQ_CEILING_COPY copies `bytes` from src to
 *     dst; AWQ_CEILING_READ reads src (dst: a device u32 sink, never written
 *     in practice); AWQ_CEILING_WRITE writes dst (16-byte element i gets the
 *     u32 values i, i^1, i^2, i^3 of its low 32 bits; src unused).  16 bytes
 *     per lane in a grid-stride loop over `blocks` workgroups of 256 threads
 *     (1 <= blocks <= 2^24; the fastest grid differs by mode and part, up to
 *     one pass over the bytes, so sweep it).  bytes: a positive multiple of 16; the buffers used 16-byte
 *     aligned.
 */
typedef enum {
  AWQ_CEILING_COPY = 0,
  AWQ_CEILING_READ = 1,
  AWQ_CEILING_WRITE = 2
} awq_ceiling_mode;
awq_status awq_ceiling_mfma(int32_t blocks, int32_t iters, int32_t zero_operands, float* sink,
                            int64_t* flops, void* stream);
awq_status awq_ceiling_stream(int32_t mode, const void* src, void* dst, size_t bytes,
                              int32_t blocks, void* stream);

/*
 * The whole per-layer search (robotsatlas "How it works", "Key mechanisms";
 * "Computational complexity": cost grows with layers x grid points x
 * calibration tokens).  Steps, all on `stream` with no host synchronisation:
 *   1. mean_abs = awq_act_stats(x)
 *   2. s, inv_s = awq_candidate_scales(mean_abs, n_grid)
 *   3. for each candidate i: quantize W . diag(s_i), write the difference
 *      operand D_i = B_i - W (awq_diff_operand; exact in bf16), then
 *      loss[i] = sum (X . D_i^T)^2 / (M N)   (fp64, fixed order)
 *      X . D_i^T equals X . B_i^T - X . W^T, the output error against the
 *      unquantized layer, so no reference output is formed.
 *   5. best = first index of the smallest loss (NaN never wins; -1 if every
 *      loss is NaN, in which case candidate 0 is written below)
 *   6. best_s = s[best]; qweight/scales/zeros = quantize_pack(w, best_s)
 *   x bf16 [M][K] (M >= 1), w bf16 [N][K] (N >= 1)
 *   mean_abs f32 [K], losses f64 [n_grid], best_idx i32 [1], best_s f32 [K],
 *   qweight u32 [N][K/8], scales f32 [N][K/group], zeros u8 [N][K/group]
 *   ws: awq_workspace_size(AWQ_OP_SEARCH_SCALE) bytes (it holds one
 *       candidate's bf16 difference operand, 2*N*K, and per-tile partials).
 */
awq_status awq_search_scale(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w, int64_t N,
                            int32_t bits, int32_t group, int32_t n_grid, float* mean_abs,
                            double* losses, int32_t* best_idx, float* best_s, uint32_t* qweight,
                            float* scales, uint8_t* zeros, void* ws, size_t ws_bytes,
                            void* stream);

/*
 * The same search with the losses in Gram form (an exact identity under the
 * fold of 1/s into the weight operand):
 *   loss_i = sum_n D_n G D_n^T / (M N),  D = B_i - W,  G = X^T X,
 * with G formed once per layer (fp32 sums of exact bf16 products) and D G
 * evaluated on the matrix cores against a two-term split of G ([D | D] .
 * [hi G | lo G]^T; D is exact in bf16 as in awq_diff_operand; about 2^-16
 * relative).  Per candidate it costs 4 N K^2 flops instead of 2 M N K, so it
 * pays when 2 K < M (many calibration tokens); G costs 2 M K^2 once.  Arguments and outputs as in
 * awq_search_scale (losses agree with it to about 1e-5 relative; the chosen
 * index can differ only between candidates whose losses tie to that
 * precision).  Limits: M rounded up to 128 and 2 K at most 2^22.
 *   ws: awq_workspace_size(AWQ_OP_SEARCH_SCALE_GRAM) bytes (X^T, G and its
 *       split, one candidate's split difference and D in fp32).
 */
awq_status awq_search_scale_gram(const uint16_t* x, int64_t M, int64_t K, const uint16_t* w,
                                 int64_t N, int32_t bits, int32_t group, int32_t n_grid,
                                 float* mean_abs, double* losses, int32_t* best_idx, float* best_s,
                                 uint32_t* qweight, float* scales, uint8_t* zeros, void* ws,
                                 size_t ws_bytes, void* stream);

/*
 * Ops of the synthetic feed-forward block around the search: a Llama-shaped
 * sublayer x -> x + down(silu(gate(u)) * up(u)), u = RMSNorm(x), searched
 * layer after layer with each 1/s folded into the op before the layer
 * (robotsatlas "How it works": the activation is divided by the same
 * per-channel factor that multiplies the weight; a deployment folds it into
 * the preceding operation).  Streams on `stream`; no host synchronisation.
 *
 * awq_rmsnorm: u[m][k] = bf16(f32(f32(x[m][k] * r_m) * gamma[k])),
 *   r_m = f32(1 / sqrt(sum_k x[m][k]^2 / K + eps)) in fp64 (sum in a fixed
 *   order).  x, u bf16 [M][K] (K a multiple of 8), gamma f32 [K], r f32 [M]
 *   output or NULL; eps >= 0.
 * awq_silu_mul: h[m][f] = bf16(f32(silu(g) * v)) with g = y[m][f],
 *   v = y[m][F + f], silu(g) = g / (1 + exp(-g)), in fp64.  y f32 [M][2F]
 *   (the fused gate/up output), h bf16 [M][F], F a multiple of 4.
 * awq_divide_rows: out[r][c] = f32(v[r][c] / s[r]) (IEEE division): 1/s
 *   folded into a gain (C = 1) or into the steps of a quantized layer's
 *   output rows (v = its scales [R][K/group]).  out may equal v.
 * awq_residual_add: out = bf16(f32(x + y)), x bf16 [M][K], y f32 [M][K],
 *   out bf16 [M][K], K a multiple of 8.
 * M == 0 (or F, C == 0) is a no-op.
 */
awq_status awq_rmsnorm(const uint16_t* x, int64_t M, int64_t K, const float* gamma, double eps,
                       uint16_t* u, float* r, void* stream);
awq_status awq_silu_mul(const float* y, int64_t M, int64_t F, uint16_t* h, void* stream);
awq_status awq_divide_rows(const float* v, int64_t R, int64_t C, const float* s, float* out,
                           void* stream);
awq_status awq_residual_add(const uint16_t* x, const float* y, int64_t M, int64_t K,
                            uint16_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* AWQ_MI355X_H */
