// Decode-shaped W4A16 contraction: Y[M][N] = A . Wd^T for M <= 64 tokens, with
// Wd[n][k] = (q[n][k] - z[n][g]) * step[n][g] taken from the packed weights
// (builderai AWQ page, "About": kernels for 4-bit weights and 16-bit
// activations; robotsatlas AWQ page, "Implementation pitfalls": without a
// matched INT4 kernel, dequantizing first throws the speedup away).
//
// At M <= 64 the contraction streams the packed weights once (0.54 bytes per
// weight) and does 2*M flops per weight, so it is bound by HBM, and the VALU
// work per weight has to stay near one instruction.  The kernel never forms
// (q - z) * step per weight:
//   * A code becomes the bf16 value 128 + q by OR-ing it into the mantissa of
//     bf16(128) (exact: 128..143).  One v_and_or_b32 builds two of them, which
//     takes codes k and k+4 of a packed word; the activation operand is
//     permuted the same way (slot order 0,4,1,5,2,6,3,7 within each 8 codes).
//   * v_mfma_f32_16x16x32_bf16 sums S = sum_k A[m][k] * (128 + q) over one
//     128-channel group (four MFMAs per 16 output channels), and the same four
//     MFMAs against an all-ones operand give sum_k A[m][k] in the same
//     accumulator layout.
//   * The group is then folded once per output: y += step * (S - (128 + z) *
//     sum A).  The products are exact in fp32, so the result is the
//     fp32-accumulated value of sum_k A * (q - z) * step.
//
// Up to 64 tokens: MB (1 or 2) 16-row blocks of A per workgroup; each
// group's codes are turned into bf16 once and feed every row block.  More
// tokens than that go to further workgroups along the grid's z, each
// re-reading the same codes (from L2 once the first has fetched them).
//
// Work split.  At these sizes a call is dominated by fixed latency (a kernel
// costs several microseconds before it streams a byte), so the layer should be
// in flight at once, in as few kernels as possible.  A workgroup owns 16, 32
// or 64 output channels and a range of at most 64 groups along K (128 at up
// to 6 tokens when K exceeds 64 groups, with 8 waves instead of 4); its waves
// split that range, and each wave streams its columns' codes through a ring
// of groups.  The waves' partial outputs are summed through LDS in wave
// order, so results do not depend on timing.  Layers whose K exceeds that
// range, and above 8 tokens layers too narrow to fill the chip otherwise,
// also split K across workgroups; those write fp32 partials that a second
// kernel sums in split order.  More columns per workgroup let one activation
// fragment feed more codes: up to 8 tokens that pays when the layer is wide
// enough to keep every CU busy anyway (decode_blocks_per_group); above 8
// tokens the activation traffic dominates and the plan takes the fewest
// workgroups that still fill the chip (many_token_shape).  Both rules were
// measured on the Llama-3-8B block's layers.  Above 32 tokens on layers of
// 96 Mi weights or more, decode_cols_kernel instead splits a workgroup's
// columns across its waves and stages each group's activations once in LDS
// for all of them.
// Tiled weights (TL): the packed codes rearranged once so that a wave's
// code load for one 16-column block and one group is a single contiguous
// 1 KiB (768 B for dense INT3) piece in lane order: tile b*G + g holds rows
// 16b .. 16b+15 of group g, row r's piece for channels 32q .. 32q+31 at byte
// P*(r + 16q).  Row-strided loads touch 16 cache lines for 64 useful bytes
// each; the tiles stream whole lines in order (10-27% faster from HBM on the
// largest layers).  Inside a piece channels 2p and 2p+1 (pair p) sit where
// one mask lifts them into the two bf16 halves of a word (nibbles t and 4+t
// of word p/4; dense INT3: bits 3t and 16+3t of word p/5, t = p%5, pair 15
// in bits 15 and 31 of the three words), so the MFMA slots hold channels in
// their natural order and the activations are used as loaded.
// The activations come from L2 (every workgroup reads the same few KiB); the
// codes are read once, with the non-temporal hint (3-7% faster on the
// Llama-3-8B layers).  The (step, 128 + zero) pairs of a wave's rows and
// groups come one of two ways:
//   * From the row-major metadata (fp32 steps and u8 zeros, or the compact
//     binary16 steps and 4-bit zeros): loaded into an LDS table up front, one
//     distinct element per lane (loaded per group they would touch 16 cache
//     lines for 64 useful bytes per instruction).
//   * From metadata tiles (META == kMetaTiles): the compact metadata
//     rearranged like the code tiles, one u32 per row and group (binary16
//     step in bits 0..15, zero in bits 16..19), the 16 rows of tile b*G + g
//     in 64 contiguous bytes.  Each lane then loads its row's word with the
//     group's codes, in the same ring: no table, no barrier before the loop,
//     one load per group and column block (7-19% faster at M = 1 than the
//     table on the Llama-3-8B layers).  Values equal the compact table's, so
//     the results are bit-identical to it.
#include <algorithm>
#include <type_traits>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kWaves = 4;                     // waves per workgroup (kWavesWide: see decode_plan)
constexpr int kWavesWide = 8;
constexpr int kDepth = 2;                     // groups of codes in flight per wave
// At one to eight tokens (A1, A4, A8) a ring slot holds one or two activation
// loads instead of four, and a ring of 4 groups measured fastest (Llama-3-8B layers at M = 1: qkv
// 6.72 -> 5.99 us, o_proj 4.74 -> 4.62, gate_up 15.9 -> 14.9, down 11.6 ->
// 8.8; 6 and 8 were slower).  With four activation loads per group deeper
// rings were slower at every M.
constexpr int kDepthOne = 4;
constexpr int kWaveGroups = 16;               // most groups per wave
constexpr int kBlockGroups = kWaves * kWaveGroups;   // 64 groups = 8192 channels
// Token blocks of 16 per workgroup: more tokens go to more workgroups along
// the grid's z (measured on the Llama-3-8B layers at 48 and 64 tokens: two
// blocks per workgroup beat four by up to 9%, and one block was slower on
// the wide layers).
constexpr int kMaxTokenBlocks = 2;
// Code ring of the column-split kernel (groups in flight per wave).
constexpr int kColsDepth = 4;

// Where the steps and zeros come from.
enum MetaSource { kMetaF32 = 0, kMetaH16 = 1, kMetaTiles = 2 };

typedef __amdgpu_buffer_rsrc_t rsrc_t;

struct DecodeParams {
  const uint16_t* a;
  const uint32_t* qweight;
  const float* scales;        // fp32 steps [N][G] (kMetaF32)
  const uint16_t* steps16;    // kMetaH16: binary16 steps [N][G]
  const uint8_t* zeros;       // u8 [N][G], or kMetaH16: two per byte [N][ceil(G/2)]
  const uint32_t* meta;       // kMetaTiles: u32 [ceil(N/16)][G][16]
  float* out;                 // y, or partials [splits][M][N]
  int64_t M, N, K;
  int64_t groups_per_split;
};

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t voff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Lane n of each 16-lane row, broadcast to the whole row (DPP row_newbcast).
template <int n>
__device__ __forceinline__ uint4 row_bcast(uint4 v) {
  constexpr int ctl = 0x150 + n;
  return make_uint4((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, ctl, 0xF, 0xF, false));
}

// The value of lane i + n of the lane's 16-lane row (DPP row_shl); lanes
// past the row's end get 0.
template <int n>
__device__ __forceinline__ uint4 row_shl(uint4 v) {
  constexpr int ctl = 0x100 + n;
  return make_uint4((uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.x, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.y, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.z, ctl, 0xF, 0xF, false),
                    (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v.w, ctl, 0xF, 0xF, false));
}

// Cache-policy bit of a buffer load: non-temporal (streamed once).
constexpr int kNonTemporal = 2;

// Codes: 16 bytes (4-bit containers) or 12 (dense INT3), read once.
__device__ __forceinline__ uint4 ld_codes16(rsrc_t r, uint32_t voff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kNonTemporal);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Eight activations a0..a7 (bf16 pairs in d) -> MFMA slots a0,a4,a1,a5,a2,a6,a3,a7.
__device__ __forceinline__ bf16x8 permute_a(uint4 d) {
  u32x4 r;
  r.x = (d.x & 0xFFFFu) | (d.z << 16);
  r.y = (d.x >> 16) | (d.z & 0xFFFF0000u);
  r.z = (d.y & 0xFFFFu) | (d.w << 16);
  r.w = (d.y >> 16) | (d.w & 0xFFFF0000u);
  return __builtin_bit_cast(bf16x8, r);
}

// Eight codes (code i at bits 4i) -> bf16 128 + code in slots 0,4,1,5,2,6,3,7.
// kc = 0x43004300 (bf16 128 in both halves), held in a VGPR: with the mask
// in an SGPR each mask-and-or is then one v_and_or_b32 (a VOP3 takes no
// literal here, and only one scalar operand).
__device__ __forceinline__ bf16x8 codes_b(uint32_t w, uint32_t kc) {
  u32x4 r;
  r.x = (w & 0x000F000Fu) | kc;
  r.y = ((w >> 4) & 0x000F000Fu) | kc;
  r.z = ((w >> 8) & 0x000F000Fu) | kc;
  r.w = ((w >> 12) & 0x000F000Fu) | kc;
  return __builtin_bit_cast(bf16x8, r);
}

// Dense INT3 (32 codes in three u32 words): the lane's 32 codes of a group
// come as 12 bytes and are widened to 4-bit fields (nibbles_from_int3) so the
// 4-bit path below applies unchanged.

// A dense-INT3 tile piece (three words) -> the four bf16x8 operands of its
// 32 channels in natural order: pair p as bf16 (128 + code) halves.
__device__ __forceinline__ void lift_pairs3(uint4 v, bf16x8 (&out)[4], uint32_t kc) {
  const uint32_t w[3] = {v.x, v.y, v.z};
  uint32_t r[16];
#pragma unroll
  for (int p = 0; p < 15; ++p) r[p] = ((w[p / 5] >> (3 * (p % 5))) & 0x00070007u) | kc;
  r[15] = ((w[0] >> 15) & 0x00010001u) | ((w[1] >> 14) & 0x00020002u) |
          ((w[2] >> 13) & 0x00040004u) | kc;
#pragma unroll
  for (int j = 0; j < 4; ++j)
    out[j] = __builtin_bit_cast(bf16x8, u32x4{r[4 * j], r[4 * j + 1], r[4 * j + 2], r[4 * j + 3]});
}

__device__ __forceinline__ uint4 ld_codes12(rsrc_t r, uint32_t voff) {
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, 0, kNonTemporal);
  return make_uint4(v.x, v.y, v.z, 0u);
}

// One group's loads for one lane: its 16 bytes of codes per 16-column block
// and, per 16-row block of tokens, its 64 bytes of activations (channels
// 32*g4 .. 32*g4+31 of the group).
template <int NB, int MB>
struct GroupLoads {
  uint32_t m[NB];       // kMetaTiles: the lane's (step, zero) word per column block
  uint4 q[NB];
  uint4 a[MB][4];
};

// NB 16-column blocks per workgroup (all of its waves work on them) and MB
// 16-row blocks of tokens (M <= 16 * MB); I3: dense INT3 codes; TL: tiled;
// META: where the steps and zeros come from (MetaSource; the compact
// metadata and its tiles go with tiled codes only).  W waves per workgroup.
// A1: exactly one token; A4: two to four tokens; A8: five to eight tokens
// (each: tiled codes, MB = 1).
template <int NB, int MB, bool I3, bool TL, int META = kMetaF32, int W = kWaves, bool A1 = false,
          bool A4 = false, bool A8 = false>
__global__ __launch_bounds__(64 * W) void decode_gemm_kernel(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr bool H16 = META == kMetaH16, MT = META == kMetaTiles;
  static_assert(META == kMetaF32 || TL, "the compact metadata goes with tiled codes");
  static_assert(!(A1 || A4 || A8) || (TL && MB == 1 && (int)A1 + (int)A4 + (int)A8 == 1),
                "the few-token forms take tiled codes and one token block");
  constexpr int kCols = 16 * NB;
  // (step, 128 + z) table, 8 to 64 KiB (none with metadata tiles).
  __shared__ float2 ssz[MT ? 1 : W][MT ? 1 : kCols][MT ? 1 : kWaveGroups];
  // Partial outputs of waves 1..W-1; with one token only lanes 0..15 hold
  // an output (row 0 of each 16-row fragment), so only their first element.
  __shared__ f32x4 red[A1 ? 1 : W - 1][MB][NB][A1 ? 1 : 64];
  __shared__ float red1[A1 ? W - 1 : 1][NB][16];

  const int lane = threadIdx.x & 63;
  // Wave index in an SGPR, so the buffer resources below are scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;        // MFMA row (A) and column (B, output)
  const int g4 = lane >> 4;         // quarter of the 128-channel group
  const int64_t M = p.M, N = p.N, K = p.K;
  // A rows past M repeat row M-1 (their outputs are never stored).
  int arow[MB];
  const int m0 = (int)blockIdx.z * 16 * MB;         // this workgroup's first token
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) arow[mb] = min(m0 + 16 * mb + c16, (int)M - 1);
  const int64_t G = K / kGroup;
  const int64_t n_blk = (int64_t)blockIdx.x * kCols;
  // This workgroup's groups [gb0, gb1); this wave's [g0, g0 + gn).
  const int64_t gb0 = (int64_t)blockIdx.y * p.groups_per_split;
  const int64_t gb1 = min(G, gb0 + p.groups_per_split);
  const int64_t per = (gb1 - gb0 + W - 1) / W;                      // <= kWaveGroups
  const int64_t g0 = gb0 + wave * per;
  const int gn = (int)max((int64_t)0, min(gb1, g0 + per) - g0);

  const rsrc_t ra = make_rsrc(p.a, M * K * 2);
  // Rows past N read as zero.  Words per row: K/8 (4-bit) or 3K/32 (INT3).
  const int64_t row_words = I3 ? 3 * K / 32 : K / 8;
  const int64_t row_blocks = (N + 15) / 16;
  const rsrc_t rq = TL ? make_rsrc(p.qweight, row_blocks * 16 * row_words * 4)
                       : make_rsrc(p.qweight + n_blk * row_words, (N - n_blk) * row_words * 4);
  const int64_t zrow = H16 ? (G + 1) / 2 : G;                // zero bytes per row
  const rsrc_t rs = H16 ? make_rsrc(p.steps16 + n_blk * G, (N - n_blk) * G * 2)
                        : make_rsrc(p.scales + n_blk * G, (N - n_blk) * G * 4);
  const rsrc_t rz = make_rsrc(p.zeros + n_blk * zrow, (N - n_blk) * zrow);
  const rsrc_t rm = make_rsrc(p.meta, MT ? row_blocks * G * 64 : 0);

  // (step, zero) of the workgroup's kCols rows x this wave's gn groups:
  // element e -> row e / gn, group e % gn (consecutive lanes read consecutive
  // groups of a row).  Past the rows, or for a wave without groups, the
  // offsets point outside the buffers and the loads return 0.
  constexpr int kSzIters = MT ? 1 : kCols * kWaveGroups / 64;
  uint32_t sz_step[kSzIters], sz_zero[kSzIters];
#pragma unroll
  for (int i = 0; i < kSzIters; ++i) {
    if constexpr (MT) break;
    const int e = i * 64 + lane;
    const int row = gn > 0 ? e / gn : kCols, gl = gn > 0 ? e - row * gn : 0;
    const bool ok = row < kCols;
    if constexpr (H16) {
      sz_step[i] = __builtin_amdgcn_raw_buffer_load_b16(
          rs, ok ? (uint32_t)((row * G + g0 + gl) * 2) : 0xFFFFFFF0u, 0, 0);
      sz_zero[i] = __builtin_amdgcn_raw_buffer_load_b8(
          rz, ok ? (uint32_t)(row * zrow + (g0 + gl) / 2) : 0xFFFFFFF0u, 0, 0);
    } else {
      sz_step[i] = __builtin_amdgcn_raw_buffer_load_b32(
          rs, ok ? (uint32_t)((row * G + g0 + gl) * 4) : 0xFFFFFFF0u, 0, 0);
      sz_zero[i] = __builtin_amdgcn_raw_buffer_load_b8(
          rz, ok ? (uint32_t)(row * G + g0 + gl) : 0xFFFFFFF0u, 0, 0);
    }
  }

  // A lane's codes of group g: bytes 64g + 16*g4 (4-bit) or 48g + 12*g4 (INT3)
  // of its row; tiled: the lane's piece of tile (row block, g).
  constexpr uint32_t kGroupBytes = I3 ? 48 : 64, kLaneBytes = I3 ? 12 : 16;
  constexpr uint32_t kStride = TL ? 16 * kGroupBytes : kGroupBytes;   // per group
  uint32_t q_off[NB];
#pragma unroll
  for (int b = 0; b < NB; ++b)
    q_off[b] = TL ? (uint32_t)(((n_blk / 16 + b) * G + g0) * kStride + kLaneBytes * lane)
                  : (uint32_t)((b * 16 + c16) * row_words * 4 + g0 * kGroupBytes + g4 * kLaneBytes);
  uint32_t a_off[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    a_off[mb] = (uint32_t)((arow[mb] * K + g0 * kGroup + 32 * g4) * 2);
  // One token (A1): every row of the activation fragments is the same, so
  // each 16-lane row loads its quarter of the group once, lane j of the row
  // channels 32*g4 + 8j .. +7 (lanes j + 4, j + 8, j + 12 the same), and the
  // four pieces are broadcast along the row: one load per group instead of
  // four (gate_up at M = 1: 16.35 -> 15.32 us; the others 1%).
  const uint32_t a1_off = (uint32_t)((g0 * kGroup + 32 * g4 + 8 * (lane & 3)) * 2);
  // Two to four tokens (A4): the 16 pieces a quarter-row of the fragments
  // holds (4 tokens x 4 pieces) are loaded once, lane r + 4q of the row
  // taking token r's piece q (tokens past M repeat token M - 1), and row
  // r < 4 takes piece j from lane r + 4j with a DPP row shift: one
  // activation load per group instead of four, and the ring of 4 then pays.
  // Five to eight tokens (A8): lane r < 8 loads pieces 0 and 1 of token r,
  // lane r + 8 pieces 2 and 3, and row r takes those two from lane r + 8:
  // two loads instead of four.  Llama-3-8B, us at 2 / 4 / 6 / 8 tokens:
  // qkv 6.48 / 6.45 / 7.22 / 7.35 -> 5.82 / 6.06 / 6.08 / 6.32, down 9.56 /
  // 10.62 / 10.68 / 13.04 -> 8.60 / 9.04 / 10.44 / 10.98 (the gather by
  // ds_bpermute it replaces was 0.3-0.6 us slower at 2 and 4 tokens).
  const uint32_t a4_off = (uint32_t)(((int64_t)min(c16 & 3, (int)M - 1) * K + g0 * kGroup +
                                      32 * g4 + 8 * (c16 >> 2)) * 2);
  const uint32_t a8_off = (uint32_t)(((int64_t)min(c16 & 7, (int)M - 1) * K + g0 * kGroup +
                                      32 * g4 + 16 * (c16 >> 3)) * 2);
  // Loads of local group gl.  Past the wave's last group the offset points
  // outside the buffer: the load returns zeros without a memory access.
  auto load = [&](GroupLoads<NB, MB>& L, int gl) {
    const bool in = gl < gn;
    if constexpr (MT) {
      // Word c16 of metadata tile (row block, group): this lane's row.
#pragma unroll
      for (int b = 0; b < NB; ++b)
        L.m[b] = __builtin_amdgcn_raw_buffer_load_b32(
            rm, in ? (uint32_t)((((n_blk / 16 + b) * G + g0 + gl) * 16 + c16) * 4) : 0xFFFFFFF0u,
            0, 0);
    }
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint32_t off = in ? q_off[b] + (uint32_t)gl * kStride : 0xFFFFFFF0u;
      L.q[b] = I3 ? ld_codes12(rq, off) : ld_codes16(rq, off);
    }
    if constexpr (A1) {
      L.a[0][0] = ld16(ra, in ? a1_off + (uint32_t)gl * (kGroup * 2) : 0xFFFFFFF0u);
    } else if constexpr (A4) {
      L.a[0][0] = ld16(ra, in ? a4_off + (uint32_t)gl * (kGroup * 2) : 0xFFFFFFF0u);
    } else if constexpr (A8) {
      L.a[0][0] = ld16(ra, in ? a8_off + (uint32_t)gl * (kGroup * 2) : 0xFFFFFFF0u);
      L.a[0][1] = ld16(ra, in ? a8_off + (uint32_t)gl * (kGroup * 2) + 16 : 0xFFFFFFF0u);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          L.a[mb][j] = ld16(ra, in ? a_off[mb] + (uint32_t)gl * (kGroup * 2) + 16 * j : 0xFFFFFFF0u);
    }
  };

  constexpr int kRing = (A1 || A4 || A8) ? kDepthOne : kDepth;
  GroupLoads<NB, MB> R[kRing];
#pragma unroll
  for (int d = 0; d < kRing; ++d) load(R[d], d);

  if constexpr (!MT) {
#pragma unroll
    for (int i = 0; i < kSzIters; ++i) {
      const int e = i * 64 + lane;
      const int row = gn > 0 ? e / gn : kCols, gl = gn > 0 ? e - row * gn : 0;
      if (row < kCols) {
        if constexpr (H16) {
          const uint32_t zq = (sz_zero[i] >> (4 * ((g0 + gl) & 1))) & 15u;
          ssz[wave][row][gl] = make_float2(
              (float)__builtin_bit_cast(_Float16, (uint16_t)sz_step[i]), 128.f + (float)zq);
        } else {
          ssz[wave][row][gl] = make_float2(__uint_as_float(sz_step[i]), 128.f + (float)sz_zero[i]);
        }
      }
    }
    // No barrier: each wave reads only its own table, and a wave's LDS
    // accesses complete in order.
  }

  uint32_t kc;   // see codes_b; an opaque VGPR value, so it is not folded back into a literal
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(kc));
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                       0x3F803F80u});
  f32x4 y[MB][NB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NB; ++b) y[mb][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const GroupLoads<NB, MB>& L, int gl) {
    // The codes as bf16 128 + q, once per group for every row block.
    bf16x8 bq[NB][4];
    float2 sz[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      if constexpr (I3 && TL) {
        lift_pairs3(L.q[b], bq[b], kc);
      } else {
        // Row-major words: codes k and k+4 of each word pair up (slot order
        // 0,4,1,5,2,6,3,7, matched by permute_a).  Tiles: the pairs are
        // channels 2p, 2p+1 (natural order).
        const uint4 qw = I3 ? nibbles_from_int3(L.q[b]) : L.q[b];
        const uint32_t words[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) bq[b][j] = codes_b(words[j], kc);
      }
      if constexpr (MT) {
        const uint32_t m = L.m[b];
        sz[b] = make_float2((float)__builtin_bit_cast(_Float16, (uint16_t)(m & 0xFFFFu)),
                            128.f + (float)((m >> 16) & 15u));
      } else {
        sz[b] = ssz[wave][b * 16 + c16][gl];
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      bf16x8 af[4];
      uint4 ad[4];
      if constexpr (A1) {
        const uint4 v = L.a[0][0];
        ad[0] = row_bcast<0>(v);
        ad[1] = row_bcast<1>(v);
        ad[2] = row_bcast<2>(v);
        ad[3] = row_bcast<3>(v);
      } else if constexpr (A4) {
        const uint4 v = L.a[0][0];
        ad[0] = v;
        ad[1] = row_shl<4>(v);
        ad[2] = row_shl<8>(v);
        ad[3] = row_shl<12>(v);
      } else if constexpr (A8) {
        ad[0] = L.a[0][0];
        ad[1] = L.a[0][1];
        ad[2] = row_shl<8>(L.a[0][0]);
        ad[3] = row_shl<8>(L.a[0][1]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) ad[j] = L.a[mb][j];
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (TL) {
          const uint4 d = ad[j];
          af[j] = __builtin_bit_cast(bf16x8, u32x4{d.x, d.y, d.z, d.w});
        } else {
          af[j] = permute_a(ad[j]);
        }
      }
      f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};             // sum A, rows 16mb + 4*g4 .. +3
#pragma unroll
      for (int j = 0; j < 4; ++j) sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], ones, sa, 0, 0, 0);
#pragma unroll
      for (int b = 0; b < NB; ++b) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], bq[b][j], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          y[mb][b][i] = fmaf(sz[b].x, fmaf(-sz[b].y, sa[i], acc[i]), y[mb][b][i]);
      }
    }
  };

  // Ring of kRing register sets, unrolled so every index is static.  Loads
  // are unconditional, so the compiler's wait counts stay exact.
  for (int gl = 0; gl < gn; gl += kRing) {
#pragma unroll
    for (int d = 0; d < kRing; ++d) {
      if (gl + d < gn) compute(R[d], gl + d);
      load(R[d], gl + d + kRing);
    }
  }

  // Sum the waves' partial outputs in wave order.
  if constexpr (A1) {
    if (wave > 0 && lane < 16) {
#pragma unroll
      for (int b = 0; b < NB; ++b) red1[wave - 1][b][lane] = y[0][b][0];
    }
    __syncthreads();
    if (wave != 0 || lane >= 16) return;
#pragma unroll
    for (int w = 0; w < W - 1; ++w)
#pragma unroll
      for (int b = 0; b < NB; ++b) y[0][b][0] += red1[w][b][lane];
  } else {
    if (wave > 0) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NB; ++b) red[wave - 1][mb][b][lane] = y[mb][b];
    }
    __syncthreads();
    if (wave != 0) return;
#pragma unroll
    for (int w = 0; w < W - 1; ++w)
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int b = 0; b < NB; ++b) y[mb][b] += red[w][mb][b][lane];
  }

  // Output: lane holds column c16 of each block and rows 16mb + 4*g4 + i.
  float* out = p.out + (int64_t)blockIdx.y * M * N;
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    const int64_t n = n_blk + b * 16 + c16;
    if (n < N) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = m0 + 16 * mb + 4 * g4 + i;
          if (m < M) out[m * N + n] = y[mb][b][i];
        }
    }
  }
#endif
}

// Large layers above 32 tokens: the waves of a workgroup split its columns
// instead of K.  Every wave walks the same groups, so each group's
// activations (MB token blocks x 128 channels, 4 KiB per block) are loaded
// once per workgroup, 16 bytes per lane, staged in LDS and read by all four
// waves as MFMA fragments.  A workgroup so covers 128 columns, twice what
// decode_gemm_kernel's waves hold in registers, which halves the activation
// traffic through L2, and with four token blocks it reads the codes once
// for up to 64 tokens.  Each wave owns NBW 16-column blocks and folds
// every group of the workgroup's range into its outputs in group order, so
// no cross-wave reduction is needed.  LDS ring of two stages: at step g the
// workgroup writes group g+1's activations (loaded two steps ahead into
// registers), computes group g, and ends with one barrier.  The codes stream
// through a per-wave register ring of CD groups as in decode_gemm_kernel.
// Row r's piece p (channels 8p .. 8p+7) of a token block sits at LDS slot
// 16r + (p ^ r): the 16 lanes of one fragment read (rows 0..15, one piece
// each) and of one write (one row, 16 pieces) then hit 64 distinct banks.
template <int NBW, int MB, int CD, bool I3, bool TL, int META>
__global__ __launch_bounds__(256) void decode_cols_kernel(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int W = 4;
  constexpr bool H16 = META == kMetaH16, MT = META == kMetaTiles;
  static_assert(META == kMetaF32 || TL, "the compact metadata goes with tiled codes");
  static_assert(CD % 2 == 0, "the activation stage follows the parity of the group");
  constexpr int kCols = 16 * NBW;                     // per wave
  __shared__ uint4 As[2][MB][256];
  // Steps (fp32) and zeros (u8) of each wave's rows and the workgroup's
  // groups: 40 KiB with two column blocks per wave, so that two workgroups
  // of four token blocks (32 KiB of activation stages each) share a CU.
  __shared__ float sst[MT ? 1 : W][MT ? 1 : kCols][MT ? 1 : kBlockGroups];
  __shared__ uint8_t szb[MT ? 1 : W][MT ? 1 : kCols][MT ? 1 : kBlockGroups];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int c16 = lane & 15, g4 = lane >> 4;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t G = K / kGroup;
  const int m0 = (int)blockIdx.z * 16 * MB;
  const int64_t n_wave = (int64_t)blockIdx.x * (W * kCols) + wave * kCols;
  const int64_t g0 = (int64_t)blockIdx.y * p.groups_per_split;
  const int gn = (int)max((int64_t)0, min(G, g0 + p.groups_per_split) - g0);   // <= 64

  const rsrc_t ra = make_rsrc(p.a, M * K * 2);
  const int64_t row_words = I3 ? 3 * K / 32 : K / 8;
  const int64_t row_blocks = (N + 15) / 16;
  const rsrc_t rq = TL ? make_rsrc(p.qweight, row_blocks * 16 * row_words * 4)
                       : make_rsrc(p.qweight + n_wave * row_words, (N - n_wave) * row_words * 4);
  const int64_t zrow = H16 ? (G + 1) / 2 : G;
  const rsrc_t rs = H16 ? make_rsrc(p.steps16 + n_wave * G, (N - n_wave) * G * 2)
                        : make_rsrc(p.scales + n_wave * G, (N - n_wave) * G * 4);
  const rsrc_t rz = make_rsrc(p.zeros + n_wave * zrow, (N - n_wave) * zrow);
  const rsrc_t rm = make_rsrc(p.meta, MT ? row_blocks * G * 64 : 0);

  // Steps and zeros of this wave's kCols rows x the gn groups, into the
  // wave's LDS table (rows past N read as zero).
  if constexpr (!MT) {
    constexpr int kSzIters = kCols * kBlockGroups / 64;
#pragma unroll 4
    for (int i = 0; i < kSzIters; ++i) {
      const int e = i * 64 + lane;
      const int row = gn > 0 ? e / gn : kCols, gl = gn > 0 ? e - row * gn : 0;
      if (row < kCols) {
        if constexpr (H16) {
          const uint32_t st = __builtin_amdgcn_raw_buffer_load_b16(
              rs, (uint32_t)((row * G + g0 + gl) * 2), 0, 0);
          const uint32_t zb = __builtin_amdgcn_raw_buffer_load_b8(
              rz, (uint32_t)(row * zrow + (g0 + gl) / 2), 0, 0);
          sst[wave][row][gl] = (float)__builtin_bit_cast(_Float16, (uint16_t)st);
          szb[wave][row][gl] = (uint8_t)((zb >> (4 * ((g0 + gl) & 1))) & 15u);
        } else {
          const uint32_t st = __builtin_amdgcn_raw_buffer_load_b32(
              rs, (uint32_t)((row * G + g0 + gl) * 4), 0, 0);
          const uint32_t zb = __builtin_amdgcn_raw_buffer_load_b8(
              rz, (uint32_t)(row * G + g0 + gl), 0, 0);
          sst[wave][row][gl] = __uint_as_float(st);
          szb[wave][row][gl] = (uint8_t)zb;
        }
      }
    }
  }

  // Codes of group gl for this wave's blocks (as decode_gemm_kernel).
  constexpr uint32_t kGroupBytes = I3 ? 48 : 64, kLaneBytes = I3 ? 12 : 16;
  constexpr uint32_t kStride = TL ? 16 * kGroupBytes : kGroupBytes;
  uint32_t q_off[NBW];
#pragma unroll
  for (int b = 0; b < NBW; ++b)
    q_off[b] = TL ? (uint32_t)(((n_wave / 16 + b) * G + g0) * kStride + kLaneBytes * lane)
                  : (uint32_t)((b * 16 + c16) * row_words * 4 + g0 * kGroupBytes + g4 * kLaneBytes);
  struct CodeLoads {
    uint32_t m[NBW];
    uint4 q[NBW];
  };
  auto load_codes = [&](CodeLoads& L, int gl) {
    const bool in = gl < gn;
    if constexpr (MT) {
#pragma unroll
      for (int b = 0; b < NBW; ++b)
        L.m[b] = __builtin_amdgcn_raw_buffer_load_b32(
            rm, in ? (uint32_t)((((n_wave / 16 + b) * G + g0 + gl) * 16 + c16) * 4) : 0xFFFFFFF0u,
            0, 0);
    }
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      const uint32_t off = in ? q_off[b] + (uint32_t)gl * kStride : 0xFFFFFFF0u;
      L.q[b] = I3 ? ld_codes12(rq, off) : ld_codes16(rq, off);
    }
  };

  // The workgroup's activations of group gl: thread t loads row t >> 4
  // (tokens past M repeat token M - 1, whose outputs are never stored),
  // piece t & 15, of each token block.
  const int ar = t >> 4, ap = t & 15;
  uint32_t a_off[MB];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
    a_off[mb] = (uint32_t)(((int64_t)min(m0 + 16 * mb + ar, (int)M - 1) * K + g0 * kGroup + 8 * ap) * 2);
  auto load_a = [&](uint4 (&P)[MB], int gl) {
    const bool in = gl < gn;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      P[mb] = ld16(ra, in ? a_off[mb] + (uint32_t)gl * (kGroup * 2) : 0xFFFFFFF0u);
  };
  auto write_a = [&](int stage, const uint4 (&P)[MB]) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) As[stage][mb][ar * 16 + (ap ^ ar)] = P[mb];
  };

  uint32_t kc;   // bf16 128 in both halves, in a VGPR (see codes_b)
  asm volatile("v_mov_b32 %0, 0x43004300" : "=v"(kc));
  const bf16x8 ones = __builtin_bit_cast(bf16x8, u32x4{0x3F803F80u, 0x3F803F80u, 0x3F803F80u,
                                                       0x3F803F80u});
  f32x4 y[MB][NBW];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int b = 0; b < NBW; ++b) y[mb][b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const CodeLoads& L, int stage, int gl) {
    bf16x8 bq[NBW][4];
    float2 sz[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
      if constexpr (I3 && TL) {
        lift_pairs3(L.q[b], bq[b], kc);
      } else {
        const uint4 qw = I3 ? nibbles_from_int3(L.q[b]) : L.q[b];
        const uint32_t words[4] = {qw.x, qw.y, qw.z, qw.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) bq[b][j] = codes_b(words[j], kc);
      }
      if constexpr (MT) {
        const uint32_t m = L.m[b];
        sz[b] = make_float2((float)__builtin_bit_cast(_Float16, (uint16_t)(m & 0xFFFFu)),
                            128.f + (float)((m >> 16) & 15u));
      } else {
        sz[b] = make_float2(sst[wave][b * 16 + c16][gl], 128.f + (float)szb[wave][b * 16 + c16][gl]);
      }
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      bf16x8 af[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint4 d = As[stage][mb][c16 * 16 + ((4 * g4 + j) ^ c16)];
        af[j] = TL ? __builtin_bit_cast(bf16x8, u32x4{d.x, d.y, d.z, d.w}) : permute_a(d);
      }
      f32x4 sa = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j) sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], ones, sa, 0, 0, 0);
#pragma unroll
      for (int b = 0; b < NBW; ++b) {
        f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], bq[b][j], acc, 0, 0, 0);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          y[mb][b][i] = fmaf(sz[b].x, fmaf(-sz[b].y, sa[i], acc[i]), y[mb][b][i]);
      }
    }
  };

  CodeLoads R[CD];
#pragma unroll
  for (int d = 0; d < CD; ++d) load_codes(R[d], d);
  uint4 P[2][MB];
  load_a(P[0], 0);
  load_a(P[1], 1);
  write_a(0, P[0]);
  load_a(P[0], 2);
  __syncthreads();
  // Step g: group g+1's activations into stage (g+1)&1 (read last at step
  // g-1, before that step's barrier), group g+3's into registers, group g
  // computed from stage g&1, then the barrier that publishes stage (g+1)&1.
  // gn is the same for every wave, so every wave passes every barrier.
  for (int gl = 0; gl < gn; gl += CD) {
#pragma unroll
    for (int d = 0; d < CD; ++d) {
      if (gl + d < gn) {
        write_a((d + 1) & 1, P[(d + 1) & 1]);
        load_a(P[(d + 1) & 1], gl + d + 3);
        compute(R[d], d & 1, gl + d);
        load_codes(R[d], gl + d + CD);
        __syncthreads();
      }
    }
  }

  float* out = p.out + (int64_t)blockIdx.y * M * N;
#pragma unroll
  for (int b = 0; b < NBW; ++b) {
    const int64_t n = n_wave + b * 16 + c16;
    if (n < N) {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int64_t m = m0 + 16 * mb + 4 * g4 + i;
          if (m < M) out[m * N + n] = y[mb][b][i];
        }
    }
  }
#endif
}

// Decode tiles from row-major packed words: one thread per W-word piece.
// 4-bit containers (W = 4): each word's nibbles 0..7 (channels 8j .. 8j+7)
// go to nibbles 0,4,1,5,2,6,3,7, so channels 2p, 2p+1 land in nibbles t,
// 4+t.  Dense INT3 (W = 3): the piece's 32 codes (code i at bit 3i of the
// 96-bit run) are re-placed by pair: pair p < 15 at bits 3(p%5) and
// 16 + 3(p%5) of word p/5, pair 15 bit by bit in bits 15 and 31.
template <int W>
__global__ __launch_bounds__(256) void decode_tiles_kernel(const uint32_t* __restrict__ qw,
                                                           int64_t N, int64_t G,
                                                           uint32_t* __restrict__ tiles) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (N + 15) / 16 * G * 64) return;
  const int64_t t = e / 64;
  const int l = (int)(e % 64), r = l & 15, q = l >> 4;
  const int64_t b = t / G, g = t - b * G, n = 16 * b + r;
  const int64_t row_words = G * 4 * W;
  uint32_t v[W];
#pragma unroll
  for (int i = 0; i < W; ++i) v[i] = n < N ? qw[n * row_words + (g * 4 + q) * W + i] : 0u;
  uint32_t o[W];
  if constexpr (W == 4) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint32_t x = 0u;
#pragma unroll
      for (int u = 0; u < 4; ++u)
        x |= ((v[j] >> (8 * u)) & 0xFu) << (4 * u) | ((v[j] >> (8 * u + 4)) & 0xFu) << (16 + 4 * u);
      o[j] = x;
    }
  } else {
    const uint64_t lo = (uint64_t)v[0] | ((uint64_t)v[1] << 32);
    const uint64_t hi = v[2];
    auto code = [&](int i) -> uint32_t {
      const int bit = 3 * i;
      if (bit + 3 <= 64) return (uint32_t)(lo >> bit) & 7u;
      if (bit >= 64) return (uint32_t)(hi >> (bit - 64)) & 7u;
      return (uint32_t)((lo >> bit) | (hi << (64 - bit))) & 7u;   // straddles bit 64
    };
    o[0] = o[1] = o[2] = 0u;
#pragma unroll
    for (int p = 0; p < 15; ++p)
      o[p / 5] |= code(2 * p) << (3 * (p % 5)) | code(2 * p + 1) << (16 + 3 * (p % 5));
    const uint32_t c30 = code(30), c31 = code(31);
#pragma unroll
    for (int i = 0; i < 3; ++i) o[i] |= ((c30 >> i) & 1u) << 15 | ((c31 >> i) & 1u) << 31;
  }
#pragma unroll
  for (int i = 0; i < W; ++i) tiles[e * W + i] = o[i];
}

// Metadata tiles from the compact metadata: word r of tile b*G + g holds the
// binary16 step of row 16b + r and group g in bits 0..15 and its zero in
// bits 16..19; rows past N give 0.  One thread per word.
__global__ __launch_bounds__(256) void meta_tiles_kernel(const uint16_t* __restrict__ steps16,
                                                         const uint8_t* __restrict__ zeros4,
                                                         int64_t N, int64_t G,
                                                         uint32_t* __restrict__ meta) {
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= (N + 15) / 16 * G * 16) return;
  const int64_t t = e / 16, b = t / G, g = t - b * G, n = 16 * b + e % 16;
  uint32_t word = 0u;
  if (n < N) {
    const uint32_t z = (zeros4[n * ((G + 1) / 2) + g / 2] >> (4 * (g & 1))) & 15u;
    word = (uint32_t)steps16[n * G + g] | (z << 16);
  }
  meta[e] = word;
}

// y[i] = sum over s of part[s][i], s ascending.
__global__ __launch_bounds__(256) void decode_reduce_kernel(const float* __restrict__ part,
                                                            int64_t count, int splits,
                                                            float* __restrict__ y) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= count) return;
  float acc = part[i];
  for (int s = 1; s < splits; ++s) acc += part[(int64_t)s * count + i];
  y[i] = acc;
}

// Up to 8 tokens: 16-column blocks per workgroup, from the number of
// workgroups one block each would give (b1, K splits included).  Measured
// (4 waves, ring of 2) on the Llama-3-8B layers: more columns let an
// activation fragment feed more codes, which pays once M > 4 if at least 384
// column blocks remain, and at any M on the widest layers.
int decode_blocks_per_group(int64_t M, int64_t N, int64_t splits) {
  const int64_t b1 = ceil_div(N, (int64_t)16) * splits;
  if ((M > 4 && b1 >= 384) || b1 >= 1024) return 2;
  return 1;
}

// Above 8 tokens every workgroup reads its token blocks' activations once per
// group for each 16-column block it does not share them with, so the
// activation traffic is (N / columns per workgroup) x M x K x 2 bytes, and at
// 64 tokens it outweighs the codes many times over (128 MiB against 8.9 MB on
// a 4096 x 4096 layer).  The plan therefore takes the fewest workgroups that
// still fill the chip: of the column blocks {1, 2, 4}, token blocks {1, 2}
// and K splits {s, 2s, 4s} (s the fewest with at most 64 groups per
// workgroup), the one with the fewest workgroups not below kMinWorkgroups
// (else the most workgroups); ties go to no K split (a second kernel and the
// partials cost more than a little parallelism), then more columns, then
// more tokens per workgroup.  Measured on the four Llama-3-8B layers at 16,
// 32 and 64 tokens against a sweep of all those combinations, the rule
// picks the fastest in 10 of 12 cases and is within 1% in the others; at
// 32 and 64 tokens it takes o_proj (4096 x 4096) from 10.3 and 20.0 us to
// 7.8 and 9.7, qkv (6144 x 4096) from 11.5 and 18.1 to 10.0 and 13.8, and
// down (4096 x 14336) at 64 tokens from 27.5 to 23.1 us.
constexpr int64_t kMinWorkgroups = 192;

// Above 32 tokens, layers of at least kColsMinWeights weights (48 MiB of
// 4-bit codes) take the column-split kernel (decode_cols_kernel).  Measured
// against the plan above (graph replays, weights from HBM, us): Llama-3-8B
// gate_up 28672 x 4096 at 33 / 48 / 64 tokens 37.3 / 39.3 / 44.0 -> 33.0 /
// 33.1 / 34.3; Llama-2-70B gate_up 57344 x 8192 at 48 / 64 tokens 125.6 /
// 139.1 -> 94.4 / 98.2 (four token blocks; 125.2 at 64 with two) and down
// 8192 x 28672 at 48 / 64 tokens 74.0 / 81.4 -> 63.7 / 64.4.  On smaller
// layers it was as fast or slower at every token count from 16 to 64
// (Llama-2-7B gate_up 22016 x 4096 at 48 tokens 31.7 -> 36.0; 4096 x 4096
// to 4096 x 14336 and 12288 x 4096 up to 1.6x slower): their workgroups wait
// at one barrier per group, and the plan above already keeps their
// activation traffic small.
constexpr int64_t kColsMinWeights = int64_t(96) << 20;
constexpr int64_t kColsOnePassBytes = int64_t(96) << 20;

struct Shape3 {
  int nb, mb;
  int64_t splits, groups_per_split, workgroups;
};

Shape3 many_token_shape(int64_t M, int64_t N, int64_t G) {
  const int64_t mb_all = ceil_div(M, (int64_t)16);
  const int64_t s_min = ceil_div(G, (int64_t)kBlockGroups);
  Shape3 best{0, 0, 0, 0, 0};
  auto key_better = [&](const Shape3& a, const Shape3& b) {
    // a before b among equal workgroup counts
    if ((a.splits > 1) != (b.splits > 1)) return a.splits == 1;
    if (a.nb != b.nb) return a.nb > b.nb;
    if (a.mb != b.mb) return a.mb > b.mb;
    return a.splits < b.splits;
  };
  for (int64_t f = 1; f <= 4; f *= 2) {
    int64_t s = std::min(G, s_min * f);
    const int64_t gps = ceil_div(G, s);
    s = ceil_div(G, gps);                     // no split without groups
    for (int nb = 1; nb <= 4; nb *= 2) {
      for (int mb = 1; mb <= kMaxTokenBlocks && mb <= mb_all; ++mb) {
        const Shape3 c{nb, mb, s, gps,
                       ceil_div(N, (int64_t)16 * nb) * s * ceil_div(mb_all, (int64_t)mb)};
        if (best.nb == 0) { best = c; continue; }
        const bool c_ok = c.workgroups >= kMinWorkgroups, b_ok = best.workgroups >= kMinWorkgroups;
        bool take;
        if (c_ok != b_ok) take = c_ok;
        else if (c.workgroups != best.workgroups)
          take = c_ok ? c.workgroups < best.workgroups : c.workgroups > best.workgroups;
        else take = key_better(c, best);
        if (take) best = c;
      }
    }
  }
  return best;
}

}  // namespace

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K) {
  DecodePlan d;
  const int64_t G = K / kGroup;
  if (M > 32 && N * K >= kColsMinWeights) {
    // Large layers at many tokens: the column-split kernel, 128 columns per
    // workgroup, two token blocks, or four (one pass over the codes) when
    // the 4-bit codes exceed kColsOnePassBytes (a second pass would no longer
    // come from the last-level cache), and the fewest K splits that keep
    // kMinWorkgroups workgroups.
    const int64_t mb_all = ceil_div(M, (int64_t)16);
    d.cols = true;
    d.col_blocks = 2;
    d.token_blocks = N * K / 2 > kColsOnePassBytes ? 4 : 2;
    const int64_t s_min = ceil_div(G, (int64_t)kBlockGroups);
    int64_t s = s_min;
    while (ceil_div(N, (int64_t)128) * s * ceil_div(mb_all, (int64_t)d.token_blocks) <
               kMinWorkgroups && s < 4 * s_min && s < G)
      s *= 2;
    d.groups_per_split = ceil_div(G, s);
    d.splits = ceil_div(G, d.groups_per_split);
  } else if (M > 8) {
    const Shape3 c = many_token_shape(M, N, G);
    d.splits = c.splits;
    d.groups_per_split = c.groups_per_split;
    d.col_blocks = c.nb;
    d.token_blocks = c.mb;
    d.cols = false;
  } else {
    // Up to 6 tokens, a K of more than 64 groups goes to workgroups of
    // kWavesWide waves and up to 128 groups, which halves the K splits (none
    // at all up to 128 groups, so no second kernel sums partials).  Measured
    // on the Llama-3-8B down layer (K = 14336) at M = 1 and 4: 14.5 -> 10.7
    // and 13.1 -> 11.3 us; on the Llama-2-70B down layer (K = 28672, dense
    // INT3) at M = 1, 2 and 4: 29.1 -> 26.6, 28.1 -> 26.8, 29.3 -> 27.4 us;
    // at M = 5 and 6 on 8B down 12.8 -> 11.6 and 13.3 -> 11.6 us.  At 8
    // tokens it was mixed (8B down 12.7 -> 13.1 us, 70B down 31.9 -> 30.6
    // us), and 8 waves over 64 groups or fewer were slower at every M.
    const int64_t max_groups = (M <= 6 && G > kBlockGroups) ? 2 * kBlockGroups : kBlockGroups;
    d.splits = ceil_div(G, max_groups);
    d.groups_per_split = ceil_div(G, d.splits);
    d.col_blocks = decode_blocks_per_group(M, N, d.splits);
    d.token_blocks = 1;
    d.cols = false;
  }
  d.ws_bytes = d.splits > 1 ? align_up((size_t)d.splits * M * N * sizeof(float)) : 0;
  return d;
}

size_t decode_meta_bytes(int64_t N, int64_t K) {
  return (size_t)((N + 15) / 16) * 16 * (size_t)(K / kGroup) * 4;
}

hipError_t launch_decode_meta(const uint16_t* steps16, const uint8_t* zeros4, int64_t N,
                              int64_t K, uint32_t* meta, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int64_t G = K / kGroup;
  const int64_t words = (N + 15) / 16 * G * 16;
  meta_tiles_kernel<<<(unsigned)ceil_div(words, (int64_t)256), 256, 0, stream>>>(steps16, zeros4,
                                                                                 N, G, meta);
  return hipGetLastError();
}

size_t decode_tiles_bytes(int64_t N, int64_t K, bool int3_dense) {
  return (size_t)((N + 15) / 16) * 16 * (size_t)(int3_dense ? 3 * K / 8 : K / 2);
}

hipError_t launch_decode_tiles(const uint32_t* qweight, int64_t N, int64_t K, bool int3_dense,
                               uint32_t* tiles, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const int64_t G = K / kGroup;
  const int64_t pieces = (N + 15) / 16 * G * 64;
  const unsigned blocks = (unsigned)ceil_div(pieces, (int64_t)256);
  if (int3_dense)
    decode_tiles_kernel<3><<<blocks, 256, 0, stream>>>(qweight, N, G, tiles);
  else
    decode_tiles_kernel<4><<<blocks, 256, 0, stream>>>(qweight, N, G, tiles);
  return hipGetLastError();
}

namespace {

// The column-split kernel: 2 16-column blocks per wave, 2 or 4 token blocks
// per workgroup, a code ring of kColsDepth groups.
template <int META>
hipError_t cols_dispatch(DecodeParams p, const DecodePlan& d, float* y, void* ws,
                         hipStream_t stream, bool int3_dense, bool tiled) {
  const int64_t M = p.M, N = p.N;
  const int mb_all = (int)ceil_div(M, (int64_t)16);
  const int mb = d.token_blocks, nbw = d.col_blocks;
  // The LDS table of steps and zeros holds at most kBlockGroups groups.
  if (d.groups_per_split > kBlockGroups || nbw != 2 || (mb != 2 && mb != 4))
    return hipErrorInvalidValue;
  dim3 grid((unsigned)ceil_div(N, (int64_t)64 * nbw), (unsigned)d.splits,
            (unsigned)ceil_div((int64_t)mb_all, (int64_t)mb));
  auto go = [&](auto NBc, auto MBc) {
    constexpr int nbv = decltype(NBc)::value, mbv = decltype(MBc)::value;
    constexpr int cd = kColsDepth;
    if constexpr (META != kMetaF32) {
      if (int3_dense)
        decode_cols_kernel<nbv, mbv, cd, true, true, META><<<grid, 256, 0, stream>>>(p);
      else
        decode_cols_kernel<nbv, mbv, cd, false, true, META><<<grid, 256, 0, stream>>>(p);
    } else {
      if (int3_dense && tiled)
        decode_cols_kernel<nbv, mbv, cd, true, true, kMetaF32><<<grid, 256, 0, stream>>>(p);
      else if (int3_dense)
        decode_cols_kernel<nbv, mbv, cd, true, false, kMetaF32><<<grid, 256, 0, stream>>>(p);
      else if (tiled)
        decode_cols_kernel<nbv, mbv, cd, false, true, kMetaF32><<<grid, 256, 0, stream>>>(p);
      else
        decode_cols_kernel<nbv, mbv, cd, false, false, kMetaF32><<<grid, 256, 0, stream>>>(p);
    }
  };
  using I2 = std::integral_constant<int, 2>;
  using I4 = std::integral_constant<int, 4>;
  if (mb == 4)
    go(I2{}, I4{});
  else
    go(I2{}, I2{});
  if (d.splits > 1) {
    const int64_t count = M * N;
    decode_reduce_kernel<<<(unsigned)ceil_div(count, (int64_t)256), 256, 0, stream>>>(
        (const float*)ws, count, (int)d.splits, y);
  }
  return hipGetLastError();
}

template <int META>
hipError_t decode_dispatch(DecodeParams p, const DecodePlan& d, float* y, void* ws,
                           hipStream_t stream, bool int3_dense, bool tiled) {
  if (d.cols) return cols_dispatch<META>(p, d, y, ws, stream, int3_dense, tiled);
  const int64_t M = p.M, N = p.N;
  const int mb_all = (int)ceil_div(M, (int64_t)16);
  const int64_t b1 = ceil_div(N, (int64_t)16) * d.splits;
  const int mb = d.token_blocks, nb = d.col_blocks;
  const int tz = (int)ceil_div((int64_t)mb_all, (int64_t)mb);   // token groups
  dim3 grid((unsigned)ceil_div(N, (int64_t)16 * nb), (unsigned)d.splits, (unsigned)tz);
  // More groups per workgroup than kWaves waves can take: the wide
  // workgroup (decode_plan gives it only to M <= 6, so one token block and
  // at most 2 column blocks).  Up to 8 tokens, layers with fewer than 320
  // column blocks (one workgroup per CU or less) take it too, with half the
  // groups per wave: more loads in flight per CU.  Measured on the
  // Llama-3-8B o_proj layer (4096 x 4096) at M = 1 and 4: 5.69 -> 5.35 and
  // 5.95 -> 5.72 us (LDS table), 5.67 -> 4.73 and 6.02 -> 5.06 us (metadata
  // tiles); at 16 tokens no faster.
  const bool wide = d.groups_per_split > kBlockGroups || (M <= 8 && b1 < 320 && mb == 1 && nb <= 2);
  if (wide && (mb != 1 || nb > 2 || d.groups_per_split > kWavesWide * kWaveGroups))
    return hipErrorInvalidValue;
  auto go = [&](auto NBc, auto MBc, auto Wc) {
    constexpr int nbv = decltype(NBc)::value, mbv = decltype(MBc)::value;
    constexpr int wv = decltype(Wc)::value;
    const unsigned threads = 64 * wv;
    if constexpr (mbv == 1) {
      if (M == 1 && tiled) {      // one token: the single-load activation form
        if (int3_dense)
          decode_gemm_kernel<nbv, 1, true, true, META, wv, true><<<grid, threads, 0, stream>>>(p);
        else
          decode_gemm_kernel<nbv, 1, false, true, META, wv, true><<<grid, threads, 0, stream>>>(p);
        return;
      }
      // Two to eight tokens: one or two loads and row shifts, with metadata
      // tiles only (with the LDS table, the few-token form, then a gather by
      // ds_bpermute, was slower on gate_up at 2 and 4 tokens: 16.4 -> 18.6
      // and 16.6 -> 19.0 us).
      if constexpr (META == kMetaTiles) {
        if (M <= 4) {
          if (int3_dense)
            decode_gemm_kernel<nbv, 1, true, true, META, wv, false, true>
                <<<grid, threads, 0, stream>>>(p);
          else
            decode_gemm_kernel<nbv, 1, false, true, META, wv, false, true>
                <<<grid, threads, 0, stream>>>(p);
          return;
        }
        if (M <= 8) {
          if (int3_dense)
            decode_gemm_kernel<nbv, 1, true, true, META, wv, false, false, true>
                <<<grid, threads, 0, stream>>>(p);
          else
            decode_gemm_kernel<nbv, 1, false, true, META, wv, false, false, true>
                <<<grid, threads, 0, stream>>>(p);
          return;
        }
      }
    }
    if constexpr (META != kMetaF32) {
      // The compact metadata and its tiles are read with tiled codes only.
      if (int3_dense)
        decode_gemm_kernel<nbv, mbv, true, true, META, wv><<<grid, threads, 0, stream>>>(p);
      else
        decode_gemm_kernel<nbv, mbv, false, true, META, wv><<<grid, threads, 0, stream>>>(p);
    } else {
      if (int3_dense && tiled)
        decode_gemm_kernel<nbv, mbv, true, true, kMetaF32, wv><<<grid, threads, 0, stream>>>(p);
      else if (int3_dense)
        decode_gemm_kernel<nbv, mbv, true, false, kMetaF32, wv><<<grid, threads, 0, stream>>>(p);
      else if (tiled)
        decode_gemm_kernel<nbv, mbv, false, true, kMetaF32, wv><<<grid, threads, 0, stream>>>(p);
      else
        decode_gemm_kernel<nbv, mbv, false, false, kMetaF32, wv><<<grid, threads, 0, stream>>>(p);
    }
  };
  auto go_mb = [&](auto NBc) {
    static_assert(kMaxTokenBlocks == 2, "instantiations below cover 1 or 2 token blocks");
    using One = std::integral_constant<int, 1>;
    if constexpr (decltype(NBc)::value <= 2) {
      if (wide) return go(NBc, One{}, std::integral_constant<int, kWavesWide>{});
    }
    if (mb == 1)
      go(NBc, One{}, std::integral_constant<int, kWaves>{});
    else
      go(NBc, std::integral_constant<int, 2>{}, std::integral_constant<int, kWaves>{});
  };
  if (nb == 4)
    go_mb(std::integral_constant<int, 4>{});
  else if (nb == 2)
    go_mb(std::integral_constant<int, 2>{});
  else
    go_mb(std::integral_constant<int, 1>{});
  if (d.splits > 1) {
    const int64_t count = M * N;
    decode_reduce_kernel<<<(unsigned)ceil_div(count, (int64_t)256), 256, 0, stream>>>(
        (const float*)ws, count, (int)d.splits, y);
  }
  return hipGetLastError();
}

DecodeParams decode_params(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                           const uint32_t* qweight, const DecodePlan& d, float* y, void* ws) {
  DecodeParams p;
  p.a = a;
  p.qweight = qweight;
  p.scales = nullptr;
  p.steps16 = nullptr;
  p.zeros = nullptr;
  p.meta = nullptr;
  p.out = d.splits > 1 ? (float*)ws : y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.groups_per_split = d.groups_per_split;
  return p;
}

}  // namespace

hipError_t launch_decode_gemm(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                              const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                              float* y, void* ws, hipStream_t stream, bool int3_dense,
                              bool tiled) {
  if (M == 0 || N == 0) return hipSuccess;
  const DecodePlan d = decode_plan(M, N, K);
  DecodeParams p = decode_params(a, M, N, K, qweight, d, y, ws);
  p.scales = scales;
  p.zeros = zeros;
  return decode_dispatch<kMetaF32>(p, d, y, ws, stream, int3_dense, tiled);
}

hipError_t launch_decode_gemm16(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                const uint32_t* tiles, const uint16_t* steps16,
                                const uint8_t* zeros4, float* y, void* ws, hipStream_t stream,
                                bool int3_dense) {
  if (M == 0 || N == 0) return hipSuccess;
  const DecodePlan d = decode_plan(M, N, K);
  DecodeParams p = decode_params(a, M, N, K, tiles, d, y, ws);
  p.steps16 = steps16;
  p.zeros = zeros4;
  return decode_dispatch<kMetaH16>(p, d, y, ws, stream, int3_dense, true);
}

hipError_t launch_decode_gemm_meta(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                                   const uint32_t* tiles, const uint32_t* meta, float* y, void* ws,
                                   hipStream_t stream, bool int3_dense) {
  if (M == 0 || N == 0) return hipSuccess;
  const DecodePlan d = decode_plan(M, N, K);
  DecodeParams p = decode_params(a, M, N, K, tiles, d, y, ws);
  p.meta = meta;
  return decode_dispatch<kMetaTiles>(p, d, y, ws, stream, int3_dense, true);
}

}  // namespace awq
