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
//   * Dense INT3: one lane per 32-code run (three u32 words, 12 bytes): four
//     16-byte stores.
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
// 3r .. 3r+2, code i of the run (channel 32r + i) at bits 3i .. 3i+2.
template <bool kInvS>
__global__ __launch_bounds__(kThreads) void dequant_int3_kernel(
    const uint32_t* __restrict__ qweight3, const float* __restrict__ scales,
    const uint8_t* __restrict__ zeros, const float* __restrict__ inv_s, int64_t N, int64_t K,
    uint16_t* __restrict__ b) {
  const int64_t rpr = K / 32;                // runs per row
  const int64_t total = N * rpr;
  const int64_t G = K / kGroup;
  for (int64_t u = (int64_t)blockIdx.x * kThreads + threadIdx.x; u < total;
       u += (int64_t)gridDim.x * kThreads) {
    const int64_t n = u / rpr, r = u - n * rpr;
    const uint32_t* src = qweight3 + 3 * u;
    const uint64_t lo = (uint64_t)src[0] | ((uint64_t)src[1] << 32);
    const uint32_t hi = src[2];
    const int64_t g = r / (kGroup / 32);
    const float step = scales[n * G + g];
    const float zero = (float)zeros[n * G + g];
    uint16_t* dst = b + n * K + 32 * r;
#pragma unroll
    for (int part = 0; part < 4; ++part) {
      float c[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int bit = 3 * (8 * part + i);  // compile-time
        uint32_t v;
        if (bit + 3 <= 64)
          v = (uint32_t)(lo >> bit) & 7u;
        else if (bit >= 64)
          v = (hi >> (bit - 64)) & 7u;
        else                                  // straddles bits 63 | 64
          v = ((uint32_t)(lo >> bit) | (hi << (64 - bit))) & 7u;
        c[i] = (float)v;
      }
      float inv[8];
      load_inv8<kInvS>(inv_s, 32 * r + 8 * part, inv);
      *(uint4*)(dst + 8 * part) = dequant8_codes<kInvS>(c, step, zero, inv);
    }
  }
}

unsigned grid_for(int64_t units) {
  const int64_t blocks = ceil_div(units, kThreads);
  return (unsigned)std::min<int64_t>(blocks, 8192);
}

}  // namespace

hipError_t launch_dequant_packed(const uint32_t* qweight, const float* scales,
                                 const uint8_t* zeros, const float* inv_s, int64_t N, int64_t K,
                                 bool int3_dense, uint16_t* b, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  if (int3_dense) {
    const unsigned grid = grid_for(N * (K / 32));
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
