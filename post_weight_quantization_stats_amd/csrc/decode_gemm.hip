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
// or 64 output channels and a range of at most 64 groups along K (32 above 16
// tokens; 128 at up to 6 tokens when K exceeds 64 groups, with 8 waves
// instead of 4); its waves split that range, and each wave streams its columns'
// codes through a ring of two groups.  The waves' partial outputs are summed
// through LDS in wave order, so results do not depend on timing.  Only layers
// whose K exceeds that range also split K across workgroups; those write fp32
// partials that a second kernel sums in split order.  More columns per
// workgroup let one activation fragment feed more codes, which pays when M is
// large or the layer is wide enough to keep every CU busy anyway (the rule in
// decode_blocks_per_group was measured on the Llama-3-8B block's layers).
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
// The activations come from L2 (every workgroup reads the same few KiB).  The
// (step, 128 + zero) pairs of a wave's rows and groups are loaded into an LDS
// table up front, one distinct element per lane: loaded per group and per
// lane they would touch 16 cache lines for 64 useful bytes per instruction.
#include <algorithm>
#include <type_traits>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kWaves = 4;                     // waves per workgroup (kWavesWide: see decode_plan)
constexpr int kWavesWide = 8;
constexpr int kDepth = 2;                     // groups of codes in flight per wave
constexpr int kWaveGroups = 16;               // most groups per wave
constexpr int kBlockGroups = kWaves * kWaveGroups;   // 64 groups = 8192 channels
// Token blocks of 16 per workgroup: more tokens go to more workgroups along
// the grid's z (measured on the Llama-3-8B layers at 48 and 64 tokens: two
// blocks per workgroup beat four by up to 9%, and one block was slower on
// the wide layers).
constexpr int kMaxTokenBlocks = 2;

typedef __amdgpu_buffer_rsrc_t rsrc_t;

struct DecodeParams {
  const uint16_t* a;
  const uint32_t* qweight;
  const float* scales;        // fp32 steps [N][G] (unless H16)
  const uint16_t* steps16;    // H16: binary16 steps [N][G]
  const uint8_t* zeros;       // u8 [N][G], or H16: two per byte [N][ceil(G/2)]
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

// Dense INT3 (32 codes in three u32 words, code i at bit 3i): the lane's 32
// codes of a group come as 12 bytes; each 24-bit run of 8 codes is spread to
// 4-bit fields (code i at bit 4i) so the 4-bit path below applies unchanged.
__device__ __forceinline__ uint32_t spread3(uint32_t f) {
  const uint32_t y = (f & 0xFFFu) | ((f & 0xFFF000u) << 4);   // codes 0-3 | codes 4-7 << 16
  return (y & 0x00070007u) | ((y & 0x00380038u) << 1) | ((y & 0x01C001C0u) << 2) |
         ((y & 0x0E000E00u) << 3);
}
__device__ __forceinline__ uint4 nibbles_from_int3(uint4 v) {
  return make_uint4(spread3(v.x & 0xFFFFFFu), spread3((v.x >> 24) | ((v.y & 0xFFFFu) << 8)),
                    spread3((v.y >> 16) | ((v.z & 0xFFu) << 16)), spread3(v.z >> 8));
}

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

__device__ __forceinline__ uint4 ld12(rsrc_t r, uint32_t voff) {
  typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
  const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(r, voff, 0, 0);
  return make_uint4(v.x, v.y, v.z, 0u);
}

// One group's loads for one lane: its 16 bytes of codes per 16-column block
// and, per 16-row block of tokens, its 64 bytes of activations (channels
// 32*g4 .. 32*g4+31 of the group).
template <int NB, int MB>
struct GroupLoads {
  uint4 q[NB];
  uint4 a[MB][4];
};

// NB 16-column blocks per workgroup (all of its waves work on them) and MB
// 16-row blocks of tokens (M <= 16 * MB); I3: dense INT3 codes; TL: tiled;
// H16: the compact metadata (binary16 steps, 4-bit zeros).
// W waves per workgroup.
template <int NB, int MB, bool I3, bool TL, bool H16 = false, int W = kWaves>
__global__ __launch_bounds__(64 * W) void decode_gemm_kernel(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int kCols = 16 * NB;
  __shared__ float2 ssz[W][kCols][kWaveGroups];    // (step, 128 + z), 8 to 64 KiB
  __shared__ f32x4 red[W - 1][MB][NB][64];          // partial outputs of waves 1..W-1

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

  // (step, zero) of the workgroup's kCols rows x this wave's gn groups:
  // element e -> row e / gn, group e % gn (consecutive lanes read consecutive
  // groups of a row).  Past the rows, or for a wave without groups, the
  // offsets point outside the buffers and the loads return 0.
  constexpr int kSzIters = kCols * kWaveGroups / 64;
  uint32_t sz_step[kSzIters], sz_zero[kSzIters];
#pragma unroll
  for (int i = 0; i < kSzIters; ++i) {
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
  // Loads of local group gl.  Past the wave's last group the offset points
  // outside the buffer: the load returns zeros without a memory access.
  auto load = [&](GroupLoads<NB, MB>& L, int gl) {
    const bool in = gl < gn;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
      const uint32_t off = in ? q_off[b] + (uint32_t)gl * kStride : 0xFFFFFFF0u;
      L.q[b] = I3 ? ld12(rq, off) : ld16(rq, off);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        L.a[mb][j] = ld16(ra, in ? a_off[mb] + (uint32_t)gl * (kGroup * 2) + 16 * j : 0xFFFFFFF0u);
  };

  GroupLoads<NB, MB> R[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load(R[d], d);

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
  __syncthreads();

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
      sz[b] = ssz[wave][b * 16 + c16][gl];
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      bf16x8 af[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if constexpr (TL) {
          const uint4 d = L.a[mb][j];
          af[j] = __builtin_bit_cast(bf16x8, u32x4{d.x, d.y, d.z, d.w});
        } else {
          af[j] = permute_a(L.a[mb][j]);
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

  // Ring of kDepth register sets, unrolled so every index is static.  Loads
  // are unconditional, so the compiler's wait counts stay exact.
  for (int gl = 0; gl < gn; gl += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (gl + d < gn) compute(R[d], gl + d);
      load(R[d], gl + d + kDepth);
    }
  }

  // Sum the waves' partial outputs in wave order.
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

// 16-column blocks per workgroup, from the number of workgroups one block
// each would give (b1, K splits included).  Measured (4 waves, ring of 2) on
// the Llama-3-8B layers at M = 1, 16, 32 and 64: more columns let an
// activation fragment feed more codes, which pays once M > 4 if at least 192
// workgroups remain, and at any M on the widest layers.
int decode_blocks_per_group(int64_t M, int64_t N, int64_t splits) {
  const int64_t b1 = ceil_div(N, (int64_t)16) * splits;
  if (M > 8 && b1 >= 1024) return 4;
  if ((M > 4 && b1 >= 384) || b1 >= 1024) return 2;
  return 1;
}

}  // namespace

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K) {
  DecodePlan d;
  const int64_t G = K / kGroup;
  // Above 16 tokens each wave's groups cost more (more token blocks per
  // group), so workgroups take at most 32 groups and more of them share K:
  // measured on the Llama-3-8B down layer (K = 14336) at M = 32 and 64,
  // 22.3 -> 20.3 and 35.1 -> 29.0 us; 16 groups per workgroup was slower.
  int64_t max_groups = M > 16 ? kBlockGroups / 2 : kBlockGroups;
  // Up to 6 tokens, a K of more than 64 groups goes to workgroups of
  // kWavesWide waves and up to 128 groups, which halves the K splits (none
  // at all up to 128 groups, so no second kernel sums partials).  Measured
  // on the Llama-3-8B down layer (K = 14336) at M = 1 and 4: 14.5 -> 10.7
  // and 13.1 -> 11.3 us; on the Llama-2-70B down layer (K = 28672, dense
  // INT3) at M = 1, 2 and 4: 29.1 -> 26.6, 28.1 -> 26.8, 29.3 -> 27.4 us;
  // at M = 5 and 6 on 8B down 12.8 -> 11.6 and 13.3 -> 11.6 us.  At 8
  // tokens it was mixed (8B down 12.7 -> 13.1 us, 70B down 31.9 -> 30.6 us),
  // at 16 slower (8B down, 14.9 -> 18.8 us), and 8 waves over 64 groups or
  // fewer were slower at every M.
  if (M <= 6 && G > kBlockGroups) max_groups = 2 * kBlockGroups;
  d.splits = ceil_div(G, max_groups);
  d.groups_per_split = ceil_div(G, d.splits);
  d.ws_bytes = d.splits > 1 ? align_up((size_t)d.splits * M * N * sizeof(float)) : 0;
  return d;
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

template <bool H16>
hipError_t decode_dispatch(DecodeParams p, const DecodePlan& d, float* y, void* ws,
                           hipStream_t stream, bool int3_dense, bool tiled) {
  const int64_t M = p.M, N = p.N;
  const int mb_all = (int)ceil_div(M, (int64_t)16);
  // Narrow layers (fewer than 512 column blocks, K splits included) above 32
  // tokens take one token block per workgroup: more workgroups in flight
  // there beat sharing the converted codes (Llama-3-8B qkv at M = 48 and 64:
  // 17.2 -> 16.6 and 20.0 -> 16.8 us; the wide gate_up and down layers were
  // slower with one block).
  const int64_t b1 = ceil_div(N, (int64_t)16) * d.splits;
  const int mb = (M > 32 && b1 < 512) ? 1 : std::min(mb_all, kMaxTokenBlocks);
  const int tz = (int)ceil_div((int64_t)mb_all, (int64_t)mb);   // token groups
  const int nb = decode_blocks_per_group(std::min(M, (int64_t)16 * mb), N, d.splits);
  dim3 grid((unsigned)ceil_div(N, (int64_t)16 * nb), (unsigned)d.splits, (unsigned)tz);
  // More groups per workgroup than kWaves waves can take: the wide
  // workgroup (decode_plan gives it only to M <= 6, so one token block and
  // at most 2 column blocks).
  const bool wide = d.groups_per_split > kBlockGroups;
  if (wide && (mb != 1 || nb > 2 || d.groups_per_split > kWavesWide * kWaveGroups))
    return hipErrorInvalidValue;
  auto go = [&](auto NBc, auto MBc, auto Wc) {
    constexpr int nbv = decltype(NBc)::value, mbv = decltype(MBc)::value;
    constexpr int wv = decltype(Wc)::value;
    const unsigned threads = 64 * wv;
    if constexpr (H16) {
      // The compact metadata is read with tiled codes only.
      if (int3_dense)
        decode_gemm_kernel<nbv, mbv, true, true, true, wv><<<grid, threads, 0, stream>>>(p);
      else
        decode_gemm_kernel<nbv, mbv, false, true, true, wv><<<grid, threads, 0, stream>>>(p);
    } else {
      if (int3_dense && tiled)
        decode_gemm_kernel<nbv, mbv, true, true, false, wv><<<grid, threads, 0, stream>>>(p);
      else if (int3_dense)
        decode_gemm_kernel<nbv, mbv, true, false, false, wv><<<grid, threads, 0, stream>>>(p);
      else if (tiled)
        decode_gemm_kernel<nbv, mbv, false, true, false, wv><<<grid, threads, 0, stream>>>(p);
      else
        decode_gemm_kernel<nbv, mbv, false, false, false, wv><<<grid, threads, 0, stream>>>(p);
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
  return decode_dispatch<false>(p, d, y, ws, stream, int3_dense, tiled);
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
  return decode_dispatch<true>(p, d, y, ws, stream, int3_dense, true);
}

}  // namespace awq
