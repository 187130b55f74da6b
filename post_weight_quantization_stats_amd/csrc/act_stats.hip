// Activation statistics: mean |x| per input channel over the calibration
// tokens (robotsatlas AWQ page, "How it works" and "Components" / activation
// saliency analysis).
//
// HBM-bound column reduction of X bf16 [M][K].  Each wave streams 1 KiB
// contiguous row segments (64 lanes x 16 B); lanes accumulate |x| of their 8
// columns in fp64 (the partial sums of bf16 magnitudes stay exact in
// practice), the four waves of a block are combined in a fixed order, and a
// second kernel adds the per-block partials in a fixed order.
#include <algorithm>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kThreads = 256;
constexpr int kColsPerBlock = 512;  // 64 lanes x 8 bf16

__device__ __forceinline__ void acc_abs8(double (&acc)[8], uint4 v) {
  acc[0] += (double)fabsf(bf16_lo(v.x));
  acc[1] += (double)fabsf(bf16_hi(v.x));
  acc[2] += (double)fabsf(bf16_lo(v.y));
  acc[3] += (double)fabsf(bf16_hi(v.y));
  acc[4] += (double)fabsf(bf16_lo(v.z));
  acc[5] += (double)fabsf(bf16_hi(v.z));
  acc[6] += (double)fabsf(bf16_lo(v.w));
  acc[7] += (double)fabsf(bf16_hi(v.w));
}

__global__ __launch_bounds__(kThreads) void act_stats_partial_kernel(
    const uint16_t* __restrict__ x, int64_t M, int64_t K, int64_t rows_per_block,
    double* __restrict__ partial) {
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int64_t col0 = (int64_t)blockIdx.x * kColsPerBlock + lane * 8;
  const int64_t r_begin = (int64_t)blockIdx.y * rows_per_block;
  const int64_t r_end = min(M, r_begin + rows_per_block);
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (col0 < K) {
    const uint16_t* p = x + col0;
    int64_t r = r_begin + wave;
    // eight rows in flight per lane
    for (; r + 28 < r_end; r += 32) {
      uint4 v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = load_stream16(p + (r + 4 * u) * K);
#pragma unroll
      for (int u = 0; u < 8; ++u) acc_abs8(acc, v[u]);
    }
    for (; r < r_end; r += 4) acc_abs8(acc, *(const uint4*)(p + r * K));
  }
  __shared__ double red[4][kColsPerBlock];
#pragma unroll
  for (int j = 0; j < 8; ++j) red[wave][lane * 8 + j] = acc[j];
  __syncthreads();
  for (int c = threadIdx.x; c < kColsPerBlock; c += kThreads) {
    const int64_t col = (int64_t)blockIdx.x * kColsPerBlock + c;
    if (col < K)
      partial[(int64_t)blockIdx.y * K + col] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
  }
}

// Column k's partials are split over 4 row-block strides (one wave each,
// 64 columns per block) and combined in a fixed order.
__global__ __launch_bounds__(kThreads) void act_stats_finalize_kernel(
    const double* __restrict__ partial, int64_t R, int64_t K, int64_t M, float* __restrict__ out) {
  const int c = threadIdx.x & 63;
  const int g = threadIdx.x >> 6;
  const int64_t k = (int64_t)blockIdx.x * 64 + c;
  double s = 0.0;
  if (k < K) {
#pragma unroll 8
    for (int64_t r = g; r < R; r += 4) s += partial[r * K + k];
  }
  __shared__ double red[4][64];
  red[g][c] = s;
  __syncthreads();
  if (g == 0 && k < K)
    out[k] = (float)((((red[0][c] + red[1][c]) + red[2][c]) + red[3][c]) / (double)M);
}

}  // namespace

StatsPlan stats_plan(int64_t M, int64_t K) {
  // At most one block per CU (256 in all, rounded down so that no second
  // round of blocks trails), each wave with eight rows in flight and a long
  // run of rows.  Measured against two blocks per CU with four rows in
  // flight: X 16384 x 8192 49.4 -> 45.1 us (5.96 TB/s), 65536 x 4096 85.7
  // -> 83.4, 32768 x 14336 163.3 -> 142.2, 65536 x 11008 253.2 -> 217.1;
  // rounding the count up instead (280 blocks for K = 14336) cost 24% there,
  // and two blocks per CU with eight rows in flight 3-14%.  At least 64 rows
  // per block, at most 1024 row blocks.
  const int64_t col_blocks = ceil_div(K, (int64_t)kColsPerBlock);
  int64_t R = std::max((int64_t)1, (int64_t)256 / col_blocks);
  if (R > ceil_div(M, (int64_t)64)) R = ceil_div(M, (int64_t)64);
  if (R > 1024) R = 1024;
  if (R < 1) R = 1;
  int64_t rpb = ceil_div(M, R);
  rpb = ceil_div(rpb, 4) * 4;
  R = ceil_div(M, rpb);
  if (R < 1) R = 1;
  return StatsPlan{rpb, R};
}

hipError_t launch_act_stats(const uint16_t* x, int64_t M, int64_t K, float* mean_abs,
                            double* partial, hipStream_t stream) {
  const StatsPlan plan = stats_plan(M, K);
  dim3 grid((unsigned)ceil_div(K, kColsPerBlock), (unsigned)plan.row_blocks);
  act_stats_partial_kernel<<<grid, kThreads, 0, stream>>>(x, M, K, plan.rows_per_block, partial);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  act_stats_finalize_kernel<<<(unsigned)ceil_div(K, 64), kThreads, 0, stream>>>(
      partial, plan.row_blocks, K, M, mean_abs);
  return hipGetLastError();
}

}  // namespace awq
