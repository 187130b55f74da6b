// Packed codes -> the bf16 weight operand of the many-token W4A16 product
// (builderai AWQ page, "About": kernels for 4-bit weights with 16-bit
// activations; sourcepulse AWQ project page, opening paragraph: 3- and 4-bit
// weights).  Writes
//   B[n][k] = bf16( f32( f32((q - z) * step) * inv_s[k] ) )
// (inv_s NULL: bf16(f32((q - z) * step))), the same operand the fused W4A16
// kernel dequantizes in LDS, once per call into a workspace, so the product
// runs on the bf16 matrix-core path.  With many tokens each weight is reused
// by every 256-row tile of activations; dequantizing it once instead of once
// per tile removes that VALU work from the contraction.
//
// HBM-bound: per weight 0.5 (4-bit containers) or 0.375 (dense INT3) bytes of
// codes plus 5/128 of step and zero are read and 2 bytes written.
//   * 4-bit containers: one lane per u32 word (8 codes): a 4-byte load and
//     one 16-byte store, both contiguous across the wave.
//   * Dense INT3: four lanes per 32-code run (three u32 words, 12 bytes),
//     each with 8 codes and one 16-byte store, contiguous across the wave
//     (one lane per run with four stores 64 bytes apart was 24% slower in the
//     staged product at 16 tokens on a 57344 x 8192 weight: 760 -> 580 us).
//   * One pass: as many blocks as lanes need (up to 2^22), no grid-stride
//     repetition (capping at 8192 blocks cost 6% there for 4-bit codes).
// Steps and zeros are read per lane (the 16 or 4 lanes of a group hit the
// same cache line).
#include <algorithm>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kThreads = 256;

template <bool kInvS>
__device__ __forceinline__ uint4 dequant8_codes(const float (&c)[8], float step, float zero,
                                                const float* inv) {
  float d[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    d[i] = (c[i] - zero) * step;           // exact difference, one fp32 rounding
    if constexpr (kInvS) d[i] = d[i] * inv[i];
  }
  uint4 r;
  r.x = pack_bf16x2(d[0], d[1]);
  r.y = pack_bf16x2(d[2], d[3]);
  r.z = pack_bf16x2(d[4], d[5]);
  r.w = pack_bf16x2(d[6], d[7]);
  return r;
}

template <bool kInvS>
__device__ __forceinline__ void load_inv8(const float* inv_s, int64_t k, float (&inv)[8]) {
  if constexpr (kInvS) {
    const float4 a = *(const float4*)(inv_s + k);
    const float4 b = *(const float4*)(inv_s + k + 4);
    inv[0] = a.x; inv[1] = a.y; inv[2] = a.z; inv[3] = a.w;
    inv[4] = b.x; inv[5] = b.y; inv[6] = b.z; inv[7] = b.w;
  }
}

// 4-bit containers: word t of row n holds codes k = 8t .. 8t+7 (code i at bits 4i).
template <bool kInvS>
__global__ __launch_bounds__(kThreads) void dequant_nibble_kernel(
    const uint32_t* __restrict__ qweight, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const float* __restrict__ inv_s, int64_t N, int64_t K,
    uint16_t* __restrict__ b) {
  const int64_t wpr = K / 8;                 // words per row
  const int64_t total = N * wpr;
  const int64_t G = K / kGroup;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * kThreads) {
    const int64_t n = u / wpr, t = u - n * wpr;
    const uint32_t qw = __builtin_nontemporal_load(qweight + u);
    const int64_t g = t / (kGroup / 8);
    const float step = scales[n * G + g];
    const float zero = (float)zeros[n * G + g];
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (float)((qw >> (4 * i)) & 0xFu);
    float inv[8];
    load_inv8<kInvS>(inv_s, 8 * t, inv);
    *(uint4*)(b + n * K + 8 * t) = dequant8_codes<kInvS>(c, step, zero, inv);
  }
}

// Dense INT3: run r of row n is the 96-bit little-endian value of words
// 3r .. 3r+2, code i of the run (channel 32r + i) at bits 3i .. 3i+2.  Four
// lanes share a run, lane p taking its codes 8p .. 8p+7 (bits 24p .. 24p+23)
// and writing their 16 bytes, so every store instruction of a wave is one
// contiguous span (the four lanes' loads of the run's 12 bytes coalesce).
template <bool kInvS>
__global__ __launch_bounds__(kThreads) void dequant_int3_kernel(
    const uint32_t* __restrict__ qweight3, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const float* __restrict__ inv_s, int64_t N, int64_t K,
    uint16_t* __restrict__ b) {
  const int64_t rpr = K / 32;                // runs per row
  const int64_t total = N * rpr * 4;         // lanes: 4 per run
  const int64_t G = K / kGroup;
  for (int64_t u4 = (int64_t)blockIdx.x * kThreads + threadIdx.x; u4 < total;
       u4 += (int64_t)gridDim.x * kThreads) {
    const int64_t u = u4 >> 2;
    const int part = (int)(u4 & 3);
    const int64_t n = u / rpr, r = u - n * rpr;
    const uint32_t* src = qweight3 + 3 * u;
    const uint32_t w0 = src[0], w1 = src[1], w2 = src[2];
    uint32_t v24;                             // bits 24*part .. 24*part + 23 of the run
    switch (part) {
      case 0: v24 = w0 & 0xFFFFFFu; break;
      case 1: v24 = (w0 >> 24) | ((w1 & 0xFFFFu) << 8); break;
      case 2: v24 = (w1 >> 16) | ((w2 & 0xFFu) << 16); break;
      default: v24 = w2 >> 8; break;
    }
    const int64_t g = r / (kGroup / 32);
    const float step = scales[n * G + g];
    const float zero = (float)zeros[n * G + g];
    float c[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) c[i] = (float)((v24 >> (3 * i)) & 7u);
    float inv[8];
    load_inv8<kInvS>(inv_s, 32 * r + 8 * part, inv);
    *(uint4*)(b + n * K + 32 * r + 8 * part) = dequant8_codes<kInvS>(c, step, zero, inv);
  }
}

unsigned grid_for(int64_t units) {
  const int64_t blocks = ceil_div(units, kThreads);
  return (unsigned)std::min<int64_t>(blocks, (int64_t)1 << 22);
}

}  // namespace

hipError_t launch_dequant_packed(const uint32_t* qweight, const float* scales,
                                 const uint8_t* zeros, const float* inv_s, int64_t N, int64_t K,
                                 bool int3_dense, uint16_t* b, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (int3_dense) {
    const unsigned grid = grid_for(N * (K / 32) * 4);
    if (inv_s)
      dequant_int3_kernel<true><<<grid, kThreads, 0, stream>>>(qweight, scales, zeros, inv_s, N, K, b);
    else
      dequant_int3_kernel<false><<<grid, kThreads, 0, stream>>>(qweight, scales, zeros, inv_s, N, K, b);
  } else {
    const unsigned grid = grid_for(N * (K / 8));
    if (inv_s)
      dequant_nibble_kernel<true><<<grid, kThreads, 0, stream>>>(qweight, scales, zeros, inv_s, N, K, b);
    else
      dequant_nibble_kernel<false><<<grid, kThreads, 0, stream>>>(qweight, scales, zeros, inv_s, N, K, b);
  }
  return hipGetLastError();
}

}  // namespace awq
