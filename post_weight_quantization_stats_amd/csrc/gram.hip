// Gram-form loss helpers.  Under the fold of 1/s into the weight operand the
// candidate's output error is X (B - W)^T, so its squared sum is
//   sum_n D_n G D_n^T  with  D = B - W  and  G = X^T X
// (robotsatlas AWQ page, "How it works": the scale is chosen by minimising the
// layer's output error; "Computational complexity": one pass over all
// calibration tokens per grid point -- here once per layer, for G).
//
//   * transpose_pad_kernel writes X^T (bf16 [K][Mp], Mp = M rounded up to the
//     contraction's k-step granularity, zero columns past M) so that G is the
//     same K-contiguous bf16 contraction as every other product here.
//   * gram_split_kernel turns fp32 G into the operand [hi(G) | lo(G)] (bf16
//     [K][2K]; hi = RNE to bf16, lo = RNE of the exact remainder).  D = B - W
//     is a bf16 value (the quantizer's grid keeps B within a factor of two of
//     W), so with the candidate's [D | D] one contraction of length 2K gives
//     D hi(G) + D lo(G), i.e. D G to about 2^-16 relative, on bf16 matrix
//     cores.
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kT = 64;   // transpose tile

// Block (bx, by) moves the 64 x 64 tile X[bx*64 .. +64][by*64 .. +64] (tokens
// on x: Mp / 64 can exceed the 65535 limit of the y dimension).
__global__ __launch_bounds__(256) void transpose_pad_kernel(const uint16_t* __restrict__ x,
                                                            int64_t M, int64_t K, int64_t Mp,
                                                            uint16_t* __restrict__ xt) {
  __shared__ uint16_t tile[kT][kT + 2];
  const int t = threadIdx.x;
  const int64_t m0 = (int64_t)blockIdx.x * kT, k0 = (int64_t)blockIdx.y * kT;
  {
    const int r = t >> 2, c = (t & 3) * 16;          // row r of the tile, 16 columns
    const int64_t m = m0 + r;
    uint4 v0 = make_uint4(0, 0, 0, 0), v1 = v0;
    if (m < M) {
      const uint4* src = (const uint4*)(x + m * K + k0 + c);
      v0 = src[0];
      v1 = src[1];
    }
    const uint32_t w[8] = {v0.x, v0.y, v0.z, v0.w, v1.x, v1.y, v1.z, v1.w};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      tile[r][c + 2 * j] = (uint16_t)(w[j] & 0xFFFFu);
      tile[r][c + 2 * j + 1] = (uint16_t)(w[j] >> 16);
    }
  }
  __syncthreads();
  {
    const int r = t >> 2, c = (t & 3) * 16;          // output row k0 + r, columns m0 + c ..
    uint32_t w[8];
#pragma unroll
    for (int j = 0; j < 8; ++j)
      w[j] = (uint32_t)tile[c + 2 * j][r] | ((uint32_t)tile[c + 2 * j + 1][r] << 16);
    uint4* dst = (uint4*)(xt + (k0 + r) * Mp + m0 + c);
    dst[0] = make_uint4(w[0], w[1], w[2], w[3]);
    dst[1] = make_uint4(w[4], w[5], w[6], w[7]);
  }
}

// Eight fp32 values of G per thread -> two 16-byte pieces of the split operand.
__global__ __launch_bounds__(256) void gram_split_kernel(const float* __restrict__ g, int64_t K,
                                                         uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;   // element index in G
  if (i >= K * K) return;
  const int64_t row = i / K, col = i - row * K;
  const float4 a = *(const float4*)(g + i);
  const float4 b = *(const float4*)(g + i + 4);
  const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  uint32_t hi[4], lo[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    hi[j] = pack_bf16x2(v[2 * j], v[2 * j + 1]);
    lo[j] = pack_bf16x2(v[2 * j] - bf16_lo(hi[j]), v[2 * j + 1] - bf16_hi(hi[j]));
  }
  uint16_t* r = out + row * 2 * K + col;
  *(uint4*)r = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  *(uint4*)(r + K) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
}

}  // namespace

int64_t gram_padded_m(int64_t M) { return ceil_div(M, kGroup) * kGroup; }

hipError_t launch_transpose_pad(const uint16_t* x, int64_t M, int64_t K, uint16_t* xt,
                                hipStream_t stream) {
  const int64_t Mp = gram_padded_m(M);
  dim3 grid((unsigned)(Mp / kT), (unsigned)(K / kT));
  transpose_pad_kernel<<<grid, 256, 0, stream>>>(x, M, K, Mp, xt);
  return hipGetLastError();
}

hipError_t launch_gram_split(const float* g, int64_t K, uint16_t* out, hipStream_t stream) {
  const int64_t n8 = K * K / 8;
  gram_split_kernel<<<(unsigned)ceil_div(n8, 256), 256, 0, stream>>>(g, K, out);
  return hipGetLastError();
}

}  // namespace awq
