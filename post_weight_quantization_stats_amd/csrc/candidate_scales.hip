// Candidate per-channel scales of the grid search (robotsatlas AWQ page,
// "How it works": a factor per input channel derived from the activation
// statistic; "Key mechanisms": grid search over the scales).
//
// For alpha_i = i / n_grid:  r = max(a^alpha, 1e-4) in fp64,
// s = fp32(r / sqrt(max_k r * min_k r)),  inv_s = fp32(1 / s).
// Tiny work (n_grid * K elements); two launches, min/max combined in a fixed
// order (min and max are exact, so the result does not depend on it).
#include <math.h>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr double kFloor = 1e-4;

__global__ __launch_bounds__(kScaleThreads) void scales_r_kernel(
    const float* __restrict__ a, int64_t K, int n_grid, double* __restrict__ r,
    double* __restrict__ mm) {
  const int i = blockIdx.y;
  const int64_t k = (int64_t)blockIdx.x * kScaleThreads + threadIdx.x;
  const double alpha = (double)i / (double)n_grid;
  double lo = INFINITY, hi = -INFINITY;
  if (k < K) {
    const double v = fmax(pow((double)a[k], alpha), kFloor);
    r[(int64_t)i * K + k] = v;
    lo = hi = v;
  }
  __shared__ double slo[kScaleThreads], shi[kScaleThreads];
  slo[threadIdx.x] = lo;
  shi[threadIdx.x] = hi;
  __syncthreads();
  for (int o = kScaleThreads / 2; o > 0; o >>= 1) {
    if ((int)threadIdx.x < o) {
      slo[threadIdx.x] = fmin(slo[threadIdx.x], slo[threadIdx.x + o]);
      shi[threadIdx.x] = fmax(shi[threadIdx.x], shi[threadIdx.x + o]);
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    const int64_t nb = gridDim.x;
    mm[((int64_t)i * nb + blockIdx.x) * 2 + 0] = slo[0];
    mm[((int64_t)i * nb + blockIdx.x) * 2 + 1] = shi[0];
  }
}

__global__ __launch_bounds__(kScaleThreads) void scales_norm_kernel(
    const double* __restrict__ r, const double* __restrict__ mm, int64_t K, int64_t nb,
    float* __restrict__ s, float* __restrict__ inv_s) {
  const int i = blockIdx.y;
  __shared__ double c;
  if (threadIdx.x == 0) {
    double lo = INFINITY, hi = -INFINITY;
    for (int64_t b = 0; b < nb; ++b) {
      lo = fmin(lo, mm[((int64_t)i * nb + b) * 2 + 0]);
      hi = fmax(hi, mm[((int64_t)i * nb + b) * 2 + 1]);
    }
    c = sqrt(hi * lo);
  }
  __syncthreads();
  const int64_t k = (int64_t)blockIdx.x * kScaleThreads + threadIdx.x;
  if (k < K) {
    const float sv = (float)(r[(int64_t)i * K + k] / c);
    s[(int64_t)i * K + k] = sv;
    inv_s[(int64_t)i * K + k] = (float)(1.0 / (double)sv);
  }
}

}  // namespace

hipError_t launch_candidate_scales(const float* mean_abs, int64_t K, int n_grid, float* s,
                                   float* inv_s, void* ws, hipStream_t stream) {
  const int64_t nb = ceil_div(K, kScaleThreads);
  double* r = (double*)ws;
  double* mm = (double*)((char*)ws + align_up((size_t)n_grid * K * sizeof(double)));
  dim3 grid((unsigned)nb, (unsigned)n_grid);
  scales_r_kernel<<<grid, kScaleThreads, 0, stream>>>(mean_abs, K, n_grid, r, mm);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  scales_norm_kernel<<<grid, kScaleThreads, 0, stream>>>(r, mm, K, nb, s, inv_s);
  return hipGetLastError();
}

}  // namespace awq
