// Decode-shaped W4A16 contraction: Y[M][N] = A . Wd^T for M <= 16 tokens, with
// Wd[n][k] = (q[n][k] - z[n][g]) * step[n][g] taken from the packed weights
// (builderai AWQ page, "About": kernels for 4-bit weights and 16-bit
// activations; robotsatlas AWQ page, "Implementation pitfalls": without a
// matched INT4 kernel, dequantizing first throws the speedup away).
//
// At M <= 16 the contraction streams the packed weights once (0.54 bytes per
// weight) and does 2*M flops per weight, so it is bound by HBM, and the VALU
// work per weight has to stay near one instruction.  The kernel never forms
// (q - z) * step per weight:
//   * A code becomes the bf16 value 128 + q by OR-ing it into the mantissa of
//     bf16(128) (exact: 128..143).  One v_and_or_b32 builds two of them, which
//     takes codes k and k+4 of a packed word; the activation operand is
//     permuted the same way (slot order 0,4,1,5,2,6,3,7 within each 8 codes).
//   * v_mfma_f32_16x16x32_bf16 sums S = sum_k A[m][k] * (128 + q) over one
//     128-channel group (four MFMAs per 16 output channels).
//   * The group is then folded once per output: y += step * (S - (128 + z) *
//     sum A), with sum A per (token, group) computed once per workgroup.  The
//     products A * (128 + q) are exact in fp32, so the result is the
//     fp32-accumulated value of sum_k A * (q - z) * step.
// Memory: the workgroup's slice of A (at most 16 rows x 2048 channels) is
// copied into LDS once by the buffer unit (XOR-swizzled 16-byte chunks, so the
// 16 rows of a fragment read hit distinct banks).  Each wave also loads the
// (step, 128 + zero) pairs of its 32 rows for the whole slice into an LDS
// table up front, one distinct element per lane: loaded per group and per
// lane they would touch 16 cache lines for 64 useful bytes per instruction,
// which measured slower than the code stream itself.  The codes stream
// through a ring of kDepth groups of registers per wave (deeper rings
// measured no faster: the streams of the resident waves already cover the
// latency).
// Work split: a workgroup of 4 waves owns 128 output channels (two 16-column
// blocks per wave) and one range of at most 16 groups along K.  Each split
// of K writes an fp32 partial; a second kernel sums the partials in split
// order, so results do not depend on timing.
#include <algorithm>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kNB = 2;                        // 16-column blocks per wave
constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTileN = 16 * kNB * kWaves;     // output channels per workgroup
constexpr int kDepth = 2;                     // groups of codes in flight per wave
constexpr int kMaxSliceGroups = 16;           // A slice: 16 rows x 2048 channels
constexpr int kRowChunks = kMaxSliceGroups * kGroup / 8;   // 16-byte chunks per LDS row
constexpr int kTargetWaves = 1024;            // one wave per SIMD

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

struct DecodeParams {
  const uint16_t* a;
  const uint32_t* qweight;
  const float* scales;
  const uint8_t* zeros;
  float* out;                 // y, or partials [splits][M][N]
  int64_t M, N, K;
  int64_t groups_per_split;
};

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const uint32_t n = bytes <= 0 ? 0u : (bytes > 0xFFFFFFFFll ? 0xFFFFFFFFu : (uint32_t)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
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
__device__ __forceinline__ bf16x8 codes_b(uint32_t w) {
  u32x4 r;
  r.x = (w & 0x000F000Fu) | 0x43004300u;
  r.y = ((w >> 4) & 0x000F000Fu) | 0x43004300u;
  r.z = ((w >> 8) & 0x000F000Fu) | 0x43004300u;
  r.w = ((w >> 12) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(bf16x8, r);
}

// LDS chunk of A (row, logical 16-byte chunk c): the low three bits of the
// chunk index are XOR-ed with the row, so one chunk column of rows 0..7
// spreads over all banks.
__device__ __forceinline__ int a_slot(int row, int c) { return row * kRowChunks + (c ^ (row & 7)); }

struct GroupLoads {
  uint4 q[kNB];        // 4 code words of this lane's column per block
};

__global__ __launch_bounds__(kThreads) void decode_gemm_kernel(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  extern __shared__ uint4 sa[];                         // A slice: M rows x kRowChunks
  __shared__ float4 ssum[kMaxSliceGroups * 4];          // sum A [group][row], 1 KiB
  __shared__ float2 ssz[kWaves][16 * kNB][kMaxSliceGroups];   // (step, 128 + z), 16 KiB

  const int lane = threadIdx.x & 63;
  // Wave index in an SGPR, so the buffer resources below are scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;        // MFMA row (A) and column (B, output)
  const int g4 = lane >> 4;         // quarter of the 128-channel group
  const int64_t M = p.M, N = p.N, K = p.K;
  // A rows past M repeat row M-1 (their outputs are never stored), so every
  // LDS read stays inside the M rows allocated.
  const int arow = min(c16, (int)M - 1);
  const int64_t G = K / kGroup;
  const int64_t n_wave = (int64_t)blockIdx.x * kTileN + wave * (16 * kNB);
  const int64_t g_begin = (int64_t)blockIdx.y * p.groups_per_split;
  const int gs = (int)(min(G, g_begin + p.groups_per_split) - g_begin);   // groups here
  const int64_t k_begin = g_begin * kGroup;

  const rsrc_t ra = make_rsrc(p.a, M * K * 2);
  // Rows past N read as zero.
  const rsrc_t rq = make_rsrc(p.qweight + n_wave * (K / 8), (N - n_wave) * (K / 2));
  const rsrc_t rs = make_rsrc(p.scales + n_wave * G, (N - n_wave) * G * 4);
  const rsrc_t rz = make_rsrc(p.zeros + n_wave * G, (N - n_wave) * G);
  uint32_t q_off[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b)
    q_off[b] = (uint32_t)((b * 16 + c16) * (K / 2) + k_begin / 2 + g4 * 16);
  // Code loads of local group gl.  Past the last group the offset points
  // outside the buffer: the load returns zeros without a memory access.
  auto load = [&](GroupLoads& L, int gl) {
    const bool in = gl < gs;
#pragma unroll
    for (int b = 0; b < kNB; ++b)
      L.q[b] = ld16(rq, in ? q_off[b] + (uint32_t)gl * 64 : 0xFFFFFFF0u, 0);
  };

  // (step, zero) of the wave's 32 rows x gs groups: element e -> row e / gs,
  // group e % gs (consecutive lanes read consecutive groups of a row).
  constexpr int kSzIters = 16 * kNB * kMaxSliceGroups / 64;
  uint32_t sz_step[kSzIters], sz_zero[kSzIters];
#pragma unroll
  for (int i = 0; i < kSzIters; ++i) {
    const int e = i * 64 + lane;
    const int row = e / gs, gl = e - row * gs;
    const bool ok = row < 16 * kNB;   // past the wave's rows: offsets outside the buffers
    sz_step[i] = __builtin_amdgcn_raw_buffer_load_b32(
        rs, ok ? (uint32_t)((row * G + g_begin + gl) * 4) : 0xFFFFFFF0u, 0, 0);
    sz_zero[i] = __builtin_amdgcn_raw_buffer_load_b8(
        rz, ok ? (uint32_t)(row * G + g_begin + gl) : 0xFFFFFFF0u, 0, 0);
  }

  GroupLoads R[kDepth];
#pragma unroll
  for (int d = 0; d < kDepth; ++d) load(R[d], d);

  // A slice -> LDS: instruction `it` copies row it/4, chunks (it%4)*64 + lane.
  // Only the M rows in use are copied; chunks past the slice read as zero
  // (offset outside the buffer).
  {
    const int rc = gs * (kGroup / 8);                   // chunks in use per row
    for (int it = wave; it < (int)M * (kRowChunks / 64); it += kWaves) {
      const int row = it / (kRowChunks / 64);
      const int pc = (it % (kRowChunks / 64)) * 64 + lane;   // physical chunk
      const int c = pc ^ (row & 7);
      const uint32_t voff = pc < rc ? (uint32_t)(row * K * 2 + (k_begin + c * 8) * 2) : 0xFFFFFFF0u;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, (lds_void*)(sa + row * kRowChunks +
                                                               (it % (kRowChunks / 64)) * 64),
                                               16, voff, 0, 0, 0);
    }
  }
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < kSzIters; ++i) {
    const int e = i * 64 + lane;
    const int row = e / gs, gl = e - row * gs;
    if (row < 16 * kNB) ssz[wave][row][gl] = make_float2(__uint_as_float(sz_step[i]),
                                                          128.f + (float)sz_zero[i]);
  }
  __syncthreads();

  // sum A per (group, row) for this slice: thread t -> group t/16, row t%16.
  {
    const int gl = threadIdx.x >> 4, row = threadIdx.x & 15;
    if (gl < gs && row < M) {
      float sum = 0.f;
#pragma unroll 4
      for (int c = 0; c < kGroup / 8; ++c) {
        const uint4 v = sa[a_slot(row, gl * 16 + c)];
        sum += bf16_lo(v.x) + bf16_hi(v.x) + bf16_lo(v.y) + bf16_hi(v.y) +
               bf16_lo(v.z) + bf16_hi(v.z) + bf16_lo(v.w) + bf16_hi(v.w);
      }
      ((float*)ssum)[gl * 16 + row] = sum;
    }
  }
  __syncthreads();

  f32x4 y[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) y[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const GroupLoads& L, int gl) {
    bf16x8 af[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) af[j] = permute_a(sa[a_slot(arow, gl * 16 + 4 * g4 + j)]);
    const float4 sv = ssum[gl * 4 + g4];                // rows 4*g4 .. 4*g4+3
    const float sum_a[4] = {sv.x, sv.y, sv.z, sv.w};
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const uint32_t words[4] = {L.q[b].x, L.q[b].y, L.q[b].z, L.q[b].w};
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], codes_b(words[j]), acc, 0, 0, 0);
      const float2 sz = ssz[wave][b * 16 + c16][gl];
      const float step = sz.x, off = sz.y;
#pragma unroll
      for (int i = 0; i < 4; ++i) y[b][i] = fmaf(step, fmaf(-off, sum_a[i], acc[i]), y[b][i]);
    }
  };

  // Ring of kDepth register sets, unrolled so every index is static.  Loads
  // are unconditional, so the compiler's wait counts stay exact.
  for (int gl = 0; gl < gs; gl += kDepth) {
#pragma unroll
    for (int d = 0; d < kDepth; ++d) {
      if (gl + d < gs) compute(R[d], gl + d);
      load(R[d], gl + d + kDepth);
    }
  }

  // Output: lane holds column c16 of each block and rows 4*g4 + i.
  float* out = p.out + (int64_t)blockIdx.y * M * N;
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int64_t n = n_wave + b * 16 + c16;
    if (n < N) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int64_t m = 4 * g4 + i;
        if (m < M) out[m * N + n] = y[b][i];
      }
    }
  }
#endif
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

}  // namespace

DecodePlan decode_plan(int64_t M, int64_t N, int64_t K) {
  DecodePlan d;
  const int64_t G = K / kGroup;
  const int64_t waves = ceil_div(N, kTileN) * kWaves;
  int64_t splits = waves >= kTargetWaves ? 1 : ceil_div(kTargetWaves, waves);
  // At least two groups per split (each split also writes M*N partials), and
  // at most kMaxSliceGroups (the A slice in LDS).
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, G / 2));
  splits = std::max<int64_t>(splits, ceil_div(G, kMaxSliceGroups));
  d.groups_per_split = ceil_div(G, splits);
  d.splits = ceil_div(G, d.groups_per_split);
  d.ws_bytes = d.splits > 1 ? align_up((size_t)d.splits * M * N * sizeof(float)) : 0;
  return d;
}

hipError_t launch_decode_gemm(const uint16_t* a, int64_t M, int64_t N, int64_t K,
                              const uint32_t* qweight, const float* scales, const uint8_t* zeros,
                              float* y, void* ws, hipStream_t stream) {
  if (M == 0 || N == 0) return hipSuccess;
  const DecodePlan d = decode_plan(M, N, K);
  DecodeParams p;
  p.a = a;
  p.qweight = qweight;
  p.scales = scales;
  p.zeros = zeros;
  p.out = d.splits > 1 ? (float*)ws : y;
  p.M = M;
  p.N = N;
  p.K = K;
  p.groups_per_split = d.groups_per_split;
  dim3 grid((unsigned)ceil_div(N, kTileN), (unsigned)d.splits);
  const size_t lds = (size_t)M * kRowChunks * 16;
  static const hipError_t attr = hipFuncSetAttribute(
      (const void*)decode_gemm_kernel, hipFuncAttributeMaxDynamicSharedMemorySize,
      (int)(kDecodeMaxM * kRowChunks * 16));
  if (attr != hipSuccess) return attr;
  decode_gemm_kernel<<<grid, kThreads, lds, stream>>>(p);
  if (d.splits > 1) {
    const int64_t count = M * N;
    decode_reduce_kernel<<<(unsigned)ceil_div(count, 256), 256, 0, stream>>>(
        (const float*)ws, count, (int)d.splits, y);
  }
  return hipGetLastError();
}

}  // namespace awq
