// W4A16 contraction Y = X . B^T with the weight operand dequantized on chip
// (builderai AWQ page, "About": kernels for 4-bit weights and 16-bit
// activations; robotsatlas AWQ page, "Implementation pitfalls": a separate
// dequantize-then-GEMM pass loses the benefit), with the squared error
// against the unquantized output fused into the epilogue (robotsatlas "How it
// works": the scale minimises the layer's output error).  The same template
// with a bf16 weight operand computes that unquantized output Y = X . W^T.
//
// gfx950 design:
//   * 256x256 output tile per workgroup, BK = 64, 4 waves in a 2x2 grid; each
//     wave owns 128x128 = 4x4 v_mfma_f32_32x32x16_bf16 blocks (256 fp32
//     accumulators per lane).
//   * Operands staged in LDS as [row][8 x 16 B chunks] with an XOR swizzle of
//     the chunk index, double buffered (2 x 64 KiB); one barrier per k-step.
//   * INT4 path: packed codes, group step/zero and 1/s are loaded to
//     registers one k-step ahead and dequantized to bf16 straight into LDS:
//     B = bf16(f32(f32((q - z) * step) * inv_s)); never written to HBM.
//   * Epilogue: optional fp32 store of Y; optional fp64 sum of
//     (Y - Y_ref)^2 per workgroup, written to a partial slot (the partials
//     are reduced later in a fixed order, so results are bit-reproducible).
#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int BM = kGemmBM;
constexpr int BN = kGemmBN;
constexpr int BK = 64;
constexpr int NT = 256;
constexpr int kChunks = BK / 8;                 // 16-byte chunks per tile row
constexpr int kRowsPerPass = NT / kChunks;      // 32 rows per load pass
constexpr int kPasses = BM / kRowsPerPass;      // 8 loads per thread per operand
static_assert(BM == BN, "load mapping assumes square tiles");

struct Params {
  const uint16_t* x;
  const uint16_t* w;
  const uint32_t* qweight;
  const float* scales;
  const uint8_t* zeros;
  const float* inv_s;
  const float* y_ref;
  float* y;
  double* partials;
  int64_t M, N, K;
  int64_t tiles_n;
};

// 16-byte slot of (row, chunk) inside one operand tile; conflict-free for
// ds_read_b128 both in 8-lane and 16-lane phases (rows r and r+8 differ).
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ ((row ^ (row >> 3)) & 7));
}

struct Int4Regs {
  uint32_t q[kPasses];
  float step[kPasses];
  float zero[kPasses];
  float inv[8];
};

__device__ __forceinline__ uint4 dequant8(uint32_t qw, float step, float zero, const float (&inv)[8]) {
  float d[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    float v = (float)((qw >> (4 * e)) & 15u) - zero;  // exact small integer
    v = v * step;                                      // fp32 round
    d[e] = v * inv[e];                                 // fp32 round
  }
  uint4 r;
  r.x = pack_bf16x2(d[0], d[1]);
  r.y = pack_bf16x2(d[2], d[3]);
  r.z = pack_bf16x2(d[4], d[5]);
  r.w = pack_bf16x2(d[6], d[7]);
  return r;
}

template <bool kInt4>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(Params p) {
  __shared__ uint4 lds[2][(BM + BN) * kChunks];

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;

  const int64_t bid = blockIdx.x;
  const int64_t tm = bid / p.tiles_n;
  const int64_t tn = bid % p.tiles_n;
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t G = K / kGroup;

  // global -> register mapping: chunk c of rows r0 + 32 j
  const int c = t & (kChunks - 1);
  const int r0 = t / kChunks;

  uint4 areg[kPasses];
  uint4 breg[kPasses];
  Int4Regs qreg;

  auto load_tile = [&](int64_t k0) {
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      const int64_t m = m0 + r0 + kRowsPerPass * j;
      areg[j] = (m < M) ? *(const uint4*)(p.x + m * K + k0 + c * 8) : make_uint4(0, 0, 0, 0);
    }
    if constexpr (kInt4) {
      const int64_t g = k0 / kGroup;
#pragma unroll
      for (int j = 0; j < kPasses; ++j) {
        const int64_t n = n0 + r0 + kRowsPerPass * j;
        if (n < N) {
          qreg.q[j] = p.qweight[n * (K / 8) + k0 / 8 + c];
          qreg.step[j] = p.scales[n * G + g];
          qreg.zero[j] = (float)p.zeros[n * G + g];
        } else {
          qreg.q[j] = 0u;
          qreg.step[j] = 0.f;
          qreg.zero[j] = 0.f;
        }
      }
      if (p.inv_s != nullptr) {
        const float4 i0 = *(const float4*)(p.inv_s + k0 + c * 8);
        const float4 i1 = *(const float4*)(p.inv_s + k0 + c * 8 + 4);
        qreg.inv[0] = i0.x; qreg.inv[1] = i0.y; qreg.inv[2] = i0.z; qreg.inv[3] = i0.w;
        qreg.inv[4] = i1.x; qreg.inv[5] = i1.y; qreg.inv[6] = i1.z; qreg.inv[7] = i1.w;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) qreg.inv[e] = 1.f;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kPasses; ++j) {
        const int64_t n = n0 + r0 + kRowsPerPass * j;
        breg[j] = (n < N) ? *(const uint4*)(p.w + n * K + k0 + c * 8) : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_tile = [&](int stage) {
    uint4* la = lds[stage];
    uint4* lb = lds[stage] + BM * kChunks;
#pragma unroll
    for (int j = 0; j < kPasses; ++j) la[swz(r0 + kRowsPerPass * j, c)] = areg[j];
#pragma unroll
    for (int j = 0; j < kPasses; ++j) {
      uint4 v;
      if constexpr (kInt4) {
        v = dequant8(qreg.q[j], qreg.step[j], qreg.zero[j], qreg.inv);
      } else {
        v = breg[j];
      }
      lb[swz(r0 + kRowsPerPass * j, c)] = v;
    }
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  const int64_t KT = K / BK;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int64_t kt = 0; kt < KT; ++kt) {
    const int cur = (int)(kt & 1);
    if (kt + 1 < KT) load_tile((kt + 1) * BK);
    const uint4* la = lds[cur];
    const uint4* lb = lds[cur] + BM * kChunks;
#pragma unroll
    for (int s = 0; s < BK / 16; ++s) {
      bf16x8 af[4], bf[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        af[i] = __builtin_bit_cast(bf16x8, la[swz(wm * 128 + i * 32 + lr, 2 * s + lk)]);
#pragma unroll
      for (int j = 0; j < 4; ++j)
        bf[j] = __builtin_bit_cast(bf16x8, lb[swz(wn * 128 + j * 32 + lr, 2 * s + lk)]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < KT) store_tile(cur ^ 1);
    __syncthreads();
  }

  // Epilogue.  32x32 block layout: lane holds column (lane & 31) and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for accumulator register r.
  double sse = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t gn = n0 + wn * 128 + j * 32 + lr;
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t gm = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);
        if (gm < M && gn < N) {
          const float v = acc[i][j][r];
          if (p.y != nullptr) p.y[gm * N + gn] = v;
          if (p.partials != nullptr) {
            const float d = v - p.y_ref[gm * N + gn];
            sse += (double)d * (double)d;
          }
        }
      }
    }
  }
  if (p.partials != nullptr) {
    sse = wave_sum_f64(sse);
    __shared__ double wsum[NT / 64];
    if (lane == 0) wsum[wave] = sse;
    __syncthreads();
    if (t == 0) p.partials[bid] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
  }
}

}  // namespace

hipError_t launch_gemm(const GemmOperands& op, hipStream_t stream) {
  if (op.M == 0 || op.N == 0) return hipSuccess;
  Params p;
  p.x = op.x;
  p.w = op.w;
  p.qweight = op.qweight;
  p.scales = op.scales;
  p.zeros = op.zeros;
  p.inv_s = op.inv_s;
  p.y_ref = op.y_ref;
  p.y = op.y;
  p.partials = op.partials;
  p.M = op.M;
  p.N = op.N;
  p.K = op.K;
  p.tiles_n = ceil_div(op.N, BN);
  const unsigned blocks = (unsigned)(ceil_div(op.M, BM) * p.tiles_n);
  if (op.qweight != nullptr)
    gemm_kernel<true><<<blocks, NT, 0, stream>>>(p);
  else
    gemm_kernel<false><<<blocks, NT, 0, stream>>>(p);
  return hipGetLastError();
}

}  // namespace awq
