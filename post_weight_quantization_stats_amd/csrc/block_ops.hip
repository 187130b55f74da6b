// The ops either side of the search in a Llama-shaped feed-forward sublayer,
// for running the search layer after layer (robotsatlas AWQ page, "How it
// works": the activation is divided by the same per-channel factor that
// multiplies the weight, which a deployment folds into the preceding
// operation; "Computational complexity": one search per layer, in order).
//
//   rmsnorm      u = bf16(f32(f32(x * r) * gamma)), r = f32(1/sqrt(mean x^2 + eps))
//   silu_mul     H = bf16(f32(silu(g) * v)) for y = [g | v], in fp64
//   divide_rows  out[r][c] = f32(v[r][c] / s[r])  (the folds of 1/s)
//   residual     x_next = bf16(f32(x + y))
//
// All are HBM-bound streams; each rounding point is the contract's, so the
// results match the CPU reference bit for bit up to the last-ulp accuracy of
// fp64 exp and the order of an fp64 sum.
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

// A 16-byte non-temporal load of four floats.
__device__ __forceinline__ float4 load_nt4(const float* p) {
  const f32x4 v = __builtin_nontemporal_load((const f32x4*)p);
  return make_float4(v.x, v.y, v.z, v.w);
}

// Round-to-nearest-even of an fp32 value to bf16 (bit pattern).
__device__ __forceinline__ uint16_t bf16_rne(float v) {
  return (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFFu);
}

// One workgroup per token row: fixed-order fp64 sum of squares, then the
// normalised row.  K is a multiple of 8.
__global__ __launch_bounds__(256) void rmsnorm_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                      const float* __restrict__ gamma, double eps,
                                                      uint16_t* __restrict__ u,
                                                      float* __restrict__ r_out) {
  const int64_t m = blockIdx.x;
  const uint16_t* row = x + m * K;
  double ss = 0.0;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < K; c += 256 * 8) {
    const uint4 v = *(const uint4*)(row + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = bf16_lo(w[j]), b = bf16_hi(w[j]);
      ss += a * a;          // exact square; the sum rounds in fp64
      ss += b * b;
    }
  }
  ss = wave_sum_f64(ss);
  __shared__ double part[4];
  __shared__ float r_sh;
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = ((part[0] + part[1]) + part[2]) + part[3];
    r_sh = (float)(1.0 / sqrt(tot / (double)K + eps));
    if (r_out != nullptr) r_out[m] = r_sh;
  }
  __syncthreads();
  const float r = r_sh;
  uint16_t* out = u + m * K;
  for (int64_t c = (int64_t)threadIdx.x * 8; c < K; c += 256 * 8) {
    const uint4 v = *(const uint4*)(row + c);
    const float4 g0 = *(const float4*)(gamma + c);
    const float4 g1 = *(const float4*)(gamma + c + 4);
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(w[j]) * r, b = bf16_hi(w[j]) * r;
      o[j] = pack_bf16x2(a * gv[2 * j], b * gv[2 * j + 1]);
    }
    *(uint4*)(out + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// The same for rows of at most 2048 P channels (P <= 8), each thread's P pieces of 8
// kept in registers between the sum of squares and the normalised row (one
// read of the row instead of two; the same sums in the same order).
template <int P>
__global__ __launch_bounds__(256) void rmsnorm_regs_kernel(const uint16_t* __restrict__ x, int64_t K,
                                                           const float* __restrict__ gamma,
                                                           double eps, uint16_t* __restrict__ u,
                                                           float* __restrict__ r_out) {
  const int64_t m = blockIdx.x;
  const uint16_t* row = x + m * K;
  uint4 v[P];
  double ss = 0.0;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int64_t c = (int64_t)threadIdx.x * 8 + 2048 * p;
    v[p] = c < K ? *(const uint4*)(row + c) : make_uint4(0u, 0u, 0u, 0u);
  }
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const double a = bf16_lo(w[j]), b = bf16_hi(w[j]);
      ss += a * a;          // exact square; the sum rounds in fp64 (zeros past K add nothing)
      ss += b * b;
    }
  }
  ss = wave_sum_f64(ss);
  __shared__ double part[4];
  __shared__ float r_sh;
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  if (threadIdx.x == 0) {
    const double tot = ((part[0] + part[1]) + part[2]) + part[3];
    r_sh = (float)(1.0 / sqrt(tot / (double)K + eps));
    if (r_out != nullptr) r_out[m] = r_sh;
  }
  __syncthreads();
  const float r = r_sh;
  uint16_t* out = u + m * K;
#pragma unroll
  for (int p = 0; p < P; ++p) {
    const int64_t c = (int64_t)threadIdx.x * 8 + 2048 * p;
    if (c >= K) break;
    const float4 g0 = *(const float4*)(gamma + c);
    const float4 g1 = *(const float4*)(gamma + c + 4);
    const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
    const uint32_t w[4] = {v[p].x, v[p].y, v[p].z, v[p].w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_lo(w[j]) * r, b = bf16_hi(w[j]) * r;
      o[j] = pack_bf16x2(a * gv[2 * j], b * gv[2 * j + 1]);
    }
    *(uint4*)(out + c) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// Four outputs of H from one quad of g and the matching quad of v.
__device__ __forceinline__ uint2 silu_mul_quad(float4 g, float4 v) {
  const float gs[4] = {g.x, g.y, g.z, g.w}, vs[4] = {v.x, v.y, v.z, v.w};
  uint16_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const double gd = gs[j];
    const double hv = gd / (1.0 + exp(-gd)) * (double)vs[j];
    o[j] = bf16_rne((float)hv);
  }
  return make_uint2((uint32_t)o[0] | ((uint32_t)o[1] << 16), (uint32_t)o[2] | ((uint32_t)o[3] << 16));
}

// Two quads of outputs per thread, 256 quads apart (each with its own row),
// their four 16-byte loads issued together and marked non-temporal (y is read
// once); F is a multiple of 4.  Against one quad per thread with plain loads
// this is 2-3% faster; the fp64 exp and division keep it near the ALU's rate.
__global__ __launch_bounds__(256) void silu_mul_kernel(const float* __restrict__ y, int64_t M,
                                                       int64_t F, uint16_t* __restrict__ h) {
  const int64_t nq = M * F / 4;
  const int64_t q0 = (int64_t)blockIdx.x * 512 + threadIdx.x, q1 = q0 + 256;
  if (q0 >= nq) return;
  const bool two = q1 < nq;
  const int64_t i0 = q0 * 4, i1 = (two ? q1 : q0) * 4;   // elements of H
  const int64_t m0 = i0 / F, f0 = i0 - m0 * F, m1 = i1 / F, f1 = i1 - m1 * F;
  const float4 g0 = load_nt4(y + m0 * 2 * F + f0), v0 = load_nt4(y + m0 * 2 * F + F + f0);
  const float4 g1 = load_nt4(y + m1 * 2 * F + f1), v1 = load_nt4(y + m1 * 2 * F + F + f1);
  *(uint2*)(h + i0) = silu_mul_quad(g0, v0);
  if (two) *(uint2*)(h + i1) = silu_mul_quad(g1, v1);
}

__global__ __launch_bounds__(256) void divide_rows_kernel(const float* __restrict__ v, int64_t R,
                                                          int64_t C, const float* __restrict__ s,
                                                          float* __restrict__ out) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= R * C) return;
  out[i] = v[i] / s[i / C];          // IEEE division, one rounding
}

// Eight elements per thread; K is a multiple of 8.
__global__ __launch_bounds__(256) void residual_kernel(const uint16_t* __restrict__ x,
                                                       const float* __restrict__ y, int64_t n,
                                                       uint16_t* __restrict__ out) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 8;
  if (i >= n) return;
  const uint4 xv = *(const uint4*)(x + i);
  const float4 y0 = *(const float4*)(y + i);
  const float4 y1 = *(const float4*)(y + i + 4);
  const float yv[8] = {y0.x, y0.y, y0.z, y0.w, y1.x, y1.y, y1.z, y1.w};
  const uint32_t w[4] = {xv.x, xv.y, xv.z, xv.w};
  uint32_t o[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) o[j] = pack_bf16x2(bf16_lo(w[j]) + yv[2 * j], bf16_hi(w[j]) + yv[2 * j + 1]);
  *(uint4*)(out + i) = make_uint4(o[0], o[1], o[2], o[3]);
}

}  // namespace

hipError_t launch_rmsnorm(const uint16_t* x, int64_t M, int64_t K, const float* gamma,
                          double eps, uint16_t* u, float* r, hipStream_t stream) {
  if (M == 0) return hipSuccess;
  const int64_t pieces = ceil_div(K, (int64_t)2048);
  switch (pieces) {
    case 1: rmsnorm_regs_kernel<1><<<(unsigned)M, 256, 0, stream>>>(x, K, gamma, eps, u, r); break;
    case 2: rmsnorm_regs_kernel<2><<<(unsigned)M, 256, 0, stream>>>(x, K, gamma, eps, u, r); break;
    case 3: rmsnorm_regs_kernel<3><<<(unsigned)M, 256, 0, stream>>>(x, K, gamma, eps, u, r); break;
    case 4: rmsnorm_regs_kernel<4><<<(unsigned)M, 256, 0, stream>>>(x, K, gamma, eps, u, r); break;
    case 5: rmsnorm_regs_kernel<5><<<(unsigned)M, 256, 0, stream>>>(x, K, gamma, eps, u, r); break;
    case 6: rmsnorm_regs_kernel<6><<<(unsigned)M, 256, 0, stream>>>(x, K, gamma, eps, u, r); break;
    case 7: rmsnorm_regs_kernel<7><<<(unsigned)M, 256, 0, stream>>>(x, K, gamma, eps, u, r); break;
    case 8: rmsnorm_regs_kernel<8><<<(unsigned)M, 256, 0, stream>>>(x, K, gamma, eps, u, r); break;
    default: rmsnorm_kernel<<<(unsigned)M, 256, 0, stream>>>(x, K, gamma, eps, u, r); break;
  }
  return hipGetLastError();
}

hipError_t launch_silu_mul(const float* y, int64_t M, int64_t F, uint16_t* h, hipStream_t stream) {
  if (M == 0 || F == 0) return hipSuccess;
  silu_mul_kernel<<<(unsigned)ceil_div(M * F / 4, (int64_t)512), 256, 0, stream>>>(y, M, F, h);
  return hipGetLastError();
}

hipError_t launch_divide_rows(const float* v, int64_t R, int64_t C, const float* s, float* out,
                              hipStream_t stream) {
  if (R == 0 || C == 0) return hipSuccess;
  divide_rows_kernel<<<(unsigned)ceil_div(R * C, (int64_t)256), 256, 0, stream>>>(v, R, C, s, out);
  return hipGetLastError();
}

hipError_t launch_residual_add(const uint16_t* x, const float* y, int64_t n, uint16_t* out,
                               hipStream_t stream) {
  if (n == 0) return hipSuccess;
  residual_kernel<<<(unsigned)ceil_div(n / 8, (int64_t)256), 256, 0, stream>>>(x, y, n, out);
  return hipGetLastError();
}

}  // namespace awq
