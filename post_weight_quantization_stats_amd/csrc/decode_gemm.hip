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
//     128-channel group (four MFMAs), and one more set of four MFMAs with an
//     all-ones operand gives sum_k A[m][k] for the same group.
//   * The group is then folded once per output: y += step * (S - (128 + z) *
//     sum A).  The products A * (128 + q) are exact in fp32, so the result is
//     the fp32-accumulated value of sum_k A * (q - z) * step.
// Work split: a workgroup of 4 waves owns 128 output channels (two 16-column
// blocks per wave) and one range of groups along K.  When the output alone
// gives too few waves to keep enough loads in flight, K is split and each
// split writes an fp32 partial; a second kernel sums the partials in split
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
constexpr int kTargetWaves = 2048;            // two waves per SIMD

typedef __amdgpu_buffer_rsrc_t rsrc_t;

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

struct GroupLoads {
  uint4 a[4];          // 32 activations of this lane's row (k = 32*(lane/16) .. +32)
  uint4 q[kNB];        // 4 code words of this lane's column per block
  uint32_t step[kNB];  // raw fp32 bits
  uint32_t zero[kNB];
};

__global__ __launch_bounds__(kThreads) void decode_gemm_kernel(DecodeParams p) {
#if defined(__HIP_DEVICE_COMPILE__)
  const int lane = threadIdx.x & 63;
  // Wave index in an SGPR, so the buffer resources below are scalar.
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int c16 = lane & 15;        // MFMA row (A) and column (B, output)
  const int g4 = lane >> 4;         // quarter of the 128-channel group
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t G = K / kGroup;
  const int64_t n_wave = (int64_t)blockIdx.x * kTileN + wave * (16 * kNB);
  const int64_t g_begin = (int64_t)blockIdx.y * p.groups_per_split;
  const int64_t g_end = min(G, g_begin + p.groups_per_split);

  // Rows past M (activations) and N (weights) read as zero.
  const rsrc_t ra = make_rsrc(p.a, M * K * 2);
  const rsrc_t rq = make_rsrc(p.qweight + n_wave * (K / 8), (N - n_wave) * (K / 2));
  const rsrc_t rs = make_rsrc(p.scales + n_wave * G, (N - n_wave) * G * 4);
  const rsrc_t rz = make_rsrc(p.zeros + n_wave * G, (N - n_wave) * G);
  const uint32_t a_off = (uint32_t)(c16 * K * 2 + g4 * 64);
  uint32_t q_off[kNB], s_off[kNB], z_off[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) {
    const int row = b * 16 + c16;
    q_off[b] = (uint32_t)(row * (K / 2) + g4 * 16);
    s_off[b] = (uint32_t)(row * G * 4);
    z_off[b] = (uint32_t)(row * G);
  }

  // Loads of group g.  The prefetch of the group after the last is clamped to
  // the last group (data never used), so every address stays inside its
  // buffer and the loads need no branch.
  auto load = [&](GroupLoads& L, int64_t g) {
#pragma unroll
    for (int c = 0; c < 4; ++c) L.a[c] = ld16(ra, a_off + c * 16, (uint32_t)(g * 256));
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      L.q[b] = ld16(rq, q_off[b], (uint32_t)(g * 64));
      L.step[b] = __builtin_amdgcn_raw_buffer_load_b32(rs, s_off[b], (uint32_t)(g * 4), 0);
      L.zero[b] = __builtin_amdgcn_raw_buffer_load_b8(rz, z_off[b], (uint32_t)g, 0);
    }
  };

  const u32x4 ones_bits = {0x3F803F80u, 0x3F803F80u, 0x3F803F80u, 0x3F803F80u};
  const bf16x8 ones = __builtin_bit_cast(bf16x8, ones_bits);
  f32x4 y[kNB];
#pragma unroll
  for (int b = 0; b < kNB; ++b) y[b] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto compute = [&](const GroupLoads& L) {
    bf16x8 af[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) af[j] = permute_a(L.a[j]);
    f32x4 sum_a = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < 4; ++j) sum_a = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], ones, sum_a, 0, 0, 0);
#pragma unroll
    for (int b = 0; b < kNB; ++b) {
      const uint32_t words[4] = {L.q[b].x, L.q[b].y, L.q[b].z, L.q[b].w};
      f32x4 acc = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[j], codes_b(words[j]), acc, 0, 0, 0);
      const float step = __uint_as_float(L.step[b]);
      const float off = 128.f + (float)L.zero[b];
#pragma unroll
      for (int i = 0; i < 4; ++i) y[b][i] = fmaf(step, fmaf(-off, sum_a[i], acc[i]), y[b][i]);
    }
  };

  // Two register sets in turn (a copy between them would wait for the
  // prefetch to land).
  GroupLoads L0, L1;
  load(L0, g_begin);
  int64_t g = g_begin;
  for (; g + 1 < g_end; g += 2) {
    load(L1, g + 1);
    compute(L0);
    load(L0, min(g + 2, g_end - 1));
    compute(L1);
  }
  if (g < g_end) compute(L0);

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
  // At least two groups per split: each split also writes M*N partials.
  splits = std::max<int64_t>(1, std::min<int64_t>(splits, G / 2));
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
  decode_gemm_kernel<<<grid, kThreads, 0, stream>>>(p);
  if (d.splits > 1) {
    const int64_t count = M * N;
    decode_reduce_kernel<<<(unsigned)ceil_div(count, 256), 256, 0, stream>>>(
        (const float*)ws, count, (int)d.splits, y);
  }
  return hipGetLastError();
}

}  // namespace awq
