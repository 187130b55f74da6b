// Group-wise asymmetric quantization and packing of W . diag(s)
// (robotsatlas AWQ page, "How it works": group-wise quantization once the
// scales are set; "Components": groups of 128 with a per-group scale;
// "Hyperparameters": 4 or 3 bits; builderai AWQ page, "About": the real
// integer weights are written).
//
// Layout: 16 lanes own one (row, 128-channel group); each lane loads 8 bf16
// (16 B, so a wave reads 1 KiB contiguous), reduces min/max with xor
// shuffles inside its 16-lane segment, and writes one u32 of 8 packed
// nibbles.  Every arithmetic step is one IEEE fp32 operation, in the order of
// the contract: ws = w*s; step = (max(mx,0) - min(mn,0)) / qmax (1 if 0);
// z = clamp(rint(-mn/step)); q = clamp(rint(ws/step) + z).  Divisions are the
// correctly rounded fp32 divide (no reciprocal approximation).
#include <math.h>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kThreads = 256;
constexpr int kGroupsPerBlock = kThreads / 16;

template <int BITS>
__global__ __launch_bounds__(kThreads) void quantize_pack_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, const float* __restrict__ s,
    const int32_t* __restrict__ s_sel, uint32_t* __restrict__ qweight,
    float* __restrict__ scales, uint8_t* __restrict__ zeros) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  const int64_t G = K / kGroup;
  const int64_t grp = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x >> 4);
  const int t16 = threadIdx.x & 15;
  const bool valid = grp < N * G;
  const int64_t n = valid ? grp / G : 0;
  const int64_t g = valid ? grp % G : 0;
  const int64_t k0 = g * kGroup + t16 * 8;

  const float* srow = s;
  if (s != nullptr && s_sel != nullptr) srow = s + (int64_t)max(*s_sel, 0) * K;

  float ws[8];
  if (valid) {
    const uint4 v = *(const uint4*)(w + n * K + k0);
    ws[0] = bf16_lo(v.x); ws[1] = bf16_hi(v.x);
    ws[2] = bf16_lo(v.y); ws[3] = bf16_hi(v.y);
    ws[4] = bf16_lo(v.z); ws[5] = bf16_hi(v.z);
    ws[6] = bf16_lo(v.w); ws[7] = bf16_hi(v.w);
    if (srow != nullptr) {
      const float4 s0 = *(const float4*)(srow + k0);
      const float4 s1 = *(const float4*)(srow + k0 + 4);
      ws[0] *= s0.x; ws[1] *= s0.y; ws[2] *= s0.z; ws[3] *= s0.w;
      ws[4] *= s1.x; ws[5] *= s1.y; ws[6] *= s1.z; ws[7] *= s1.w;
    }
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) ws[j] = 0.f;
  }
  float mx = ws[0], mn = ws[0];
#pragma unroll
  for (int j = 1; j < 8; ++j) {
    mx = fmaxf(mx, ws[j]);
    mn = fminf(mn, ws[j]);
  }
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) {
    mx = fmaxf(mx, __shfl_xor(mx, o, 16));
    mn = fminf(mn, __shfl_xor(mn, o, 16));
  }
  mx = fmaxf(mx, 0.f);
  mn = fminf(mn, 0.f);
  const float range = mx - mn;
  float step = range / qmax;
  if (!(step > 0.f)) step = 1.f;
  const float z = fminf(fmaxf(rintf(-mn / step), 0.f), qmax);
  uint32_t word = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const float q = fminf(fmaxf(rintf(ws[j] / step) + z, 0.f), qmax);
    word |= (uint32_t)q << (4 * j);
  }
  if (valid) {
    qweight[n * (K / 8) + k0 / 8] = word;
    if (t16 == 0) {
      scales[grp] = step;
      zeros[grp] = (uint8_t)z;
    }
  }
}

}  // namespace

hipError_t launch_quantize_pack(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                const int32_t* s_sel, int bits, uint32_t* qweight,
                                float* scales, uint8_t* zeros, hipStream_t stream) {
  const int64_t groups = N * (K / kGroup);
  if (groups == 0) return hipSuccess;
  const unsigned blocks = (unsigned)ceil_div(groups, kGroupsPerBlock);
  if (bits == 4)
    quantize_pack_kernel<4><<<blocks, kThreads, 0, stream>>>(w, N, K, s, s_sel, qweight, scales, zeros);
  else
    quantize_pack_kernel<3><<<blocks, kThreads, 0, stream>>>(w, N, K, s, s_sel, qweight, scales, zeros);
  return hipGetLastError();
}

}  // namespace awq
