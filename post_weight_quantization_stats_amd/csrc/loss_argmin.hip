// Per-candidate loss and selection (robotsatlas AWQ page, "How it works" and
// "Key mechanisms": the scale with the smallest layer output error wins).
//
// losses[i] = (sum over workgroup partials of candidate i) / (M N), summed in
// fp64 in a fixed order (strided per-thread sums, then a fixed tree), so the
// result is bit-reproducible.  The argmin takes the first smallest loss and
// skips NaN; it writes -1 when every loss is NaN.
#include <math.h>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void loss_reduce_kernel(
    const double* __restrict__ partials, int64_t T, double divisor, double* __restrict__ losses) {
  const int i = blockIdx.x;
  const double* p = partials + (int64_t)i * T;
  double s = 0.0;
  for (int64_t t = threadIdx.x; t < T; t += kThreads) s += p[t];
  __shared__ double red[kThreads];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = kThreads / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) losses[i] = red[0] / divisor;
}

__global__ void argmin_kernel(const double* __restrict__ losses, int n, int32_t* __restrict__ best) {
  if (threadIdx.x != 0 || blockIdx.x != 0) return;
  int b = -1;
  double bv = 0.0;
  for (int i = 0; i < n; ++i) {
    const double v = losses[i];
    if (isnan(v)) continue;
    if (b < 0 || v < bv) {
      b = i;
      bv = v;
    }
  }
  *best = b;
}

__global__ __launch_bounds__(kThreads) void select_row_kernel(
    const float* __restrict__ s, const int32_t* __restrict__ sel, int64_t K, float* __restrict__ out) {
  const int64_t k = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (k < K) out[k] = s[(int64_t)max(*sel, 0) * K + k];
}

__global__ void fill_f64_kernel(double* p, int64_t n, double v) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = v;
}

}  // namespace

hipError_t launch_loss_reduce(const double* partials, int64_t T, int n_grid, double divisor,
                              double* losses, hipStream_t stream) {
  loss_reduce_kernel<<<n_grid, kThreads, 0, stream>>>(partials, T, divisor, losses);
  return hipGetLastError();
}

hipError_t launch_argmin(const double* losses, int n_grid, int32_t* best, hipStream_t stream) {
  argmin_kernel<<<1, 64, 0, stream>>>(losses, n_grid, best);
  return hipGetLastError();
}

hipError_t launch_select_row(const float* s, const int32_t* sel, int64_t K, float* out,
                             hipStream_t stream) {
  select_row_kernel<<<(unsigned)ceil_div(K, kThreads), kThreads, 0, stream>>>(s, sel, K, out);
  return hipGetLastError();
}

hipError_t launch_fill_f64(double* p, int64_t n, double v, hipStream_t stream) {
  if (n <= 0) return hipSuccess;
  fill_f64_kernel<<<(unsigned)ceil_div(n, 256), 256, 0, stream>>>(p, n, v);
  return hipGetLastError();
}

}  // namespace awq
