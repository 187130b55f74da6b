// Group-wise asymmetric quantization and packing of W . diag(s)
// (robotsatlas AWQ page, "How it works": group-wise quantization once the
// scales are set; "Components": groups of 128 with a per-group scale;
// "Hyperparameters": 4 or 3 bits; builderai AWQ page, "About": the real
// integer weights are written).
//
// Layout: 8 lanes own one 128-channel group, 16 channels (32 B of bf16) per
// lane, so a wave covers 8 groups = 2 KiB of one row.  A block of 256 lanes
// spans 32 groups and walks rows kRows at a time in a grid-stride loop; each
// lane loads its 16 scale factors once.  Group min/max is reduced with three DPP steps inside each 8-lane
// segment (quad swaps, then the half-row mirror); each lane writes two u32 of
// packed nibbles.  Every arithmetic step is one IEEE fp32 operation, in the
// order of the contract: ws = w*s; step = (max(mx,0) - min(mn,0)) / qmax
// (1 if 0); z = clamp(rint(-mn/step)); q = clamp(rint(ws/step) + z).
//
// The quotients must be the correctly rounded ones (the codes are their rint).
// With y = RN(1/b), q0 = RN(a*y) and the exact residual r = a - b*q0 (one
// fma), RN(q0 + r*y) is the correctly rounded a/b (P. Markstein, "Computation
// of elementary functions on the IBM RISC System/6000 processor", IBM J. Res.
// Dev. 34(1), 1990; Muller et al., Handbook of Floating-Point Arithmetic,
// 2018, the division theorem for fused multiply-add).  The theorem needs the
// residual not to underflow.  A group takes this path when its range lies in
// [2^-90, 2^100]: then step >= 2^-94, every |a| >= step/2 has a residual far
// above the subnormal range, and for |a| < step/2 both quotients round to a
// code of 0 (checked exhaustively for the constant divisors 15 and 7 and on
// 2e8 random (a, step) pairs).  Other groups (zero, tiny, huge or non-finite
// ranges) take plain IEEE divisions.
#include <math.h>

#include <algorithm>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerGroup = 8;
constexpr int kGroupsPerBlock = kThreads / kLanesPerGroup;
constexpr int kRows = 4;

template <int CTRL>
__device__ __forceinline__ float dpp(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}

__device__ __forceinline__ float markstein_div(float a, float b, float y) {
  const float q0 = a * y;
  const float r = fmaf(-q0, b, a);              // exact residual
  return fmaf(r, y, q0);                        // RN(a / b)
}

// One lane's 16 channels of a group: their codes (as floats) and the group's
// step and zero (identical in all 8 lanes of the group).  kCentred: q[j] holds
// the centred code q - z instead, formed as clamp(rint(ws/step), -z, qmax - z)
// (equal to clamp(rint(ws/step) + z, 0, qmax) - z: every value is a small
// integer), one median instead of an add, a clamp and a subtract.
template <int BITS, bool kHalf = false, bool kCentred = false>
__device__ __forceinline__ void quantize16(const float (&ws)[16], float (&q)[16],
                                           float& step_out, float& z_out) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  constexpr float inv_qmax = 1.0f / qmax;       // RN(1/qmax), folded by the compiler
  float mx = fmaxf(ws[0], ws[1]), mn = fminf(ws[0], ws[1]);
#pragma unroll
  for (int j = 2; j < 16; ++j) {
    mx = fmaxf(mx, ws[j]);
    mn = fminf(mn, ws[j]);
  }
  mx = fmaxf(mx, dpp<0xB1>(mx));                // lanes ^1
  mn = fminf(mn, dpp<0xB1>(mn));
  mx = fmaxf(mx, dpp<0x4E>(mx));                // lanes ^2
  mn = fminf(mn, dpp<0x4E>(mn));
  mx = fmaxf(mx, dpp<0x141>(mx));               // lane i <-> 7-i of each half row
  mn = fminf(mn, dpp<0x141>(mn));
  mx = fmaxf(mx, 0.f);
  mn = fminf(mn, 0.f);
  const float range = mx - mn;
  const bool fast = range >= 0x1p-90f && range <= 0x1p100f;

  if constexpr (kHalf) {
    // Compact format: the fp32 step limited to [2^-24, 65504] and rounded to
    // binary16 (v_cvt_f16_f32, nearest even); zero and codes use that step.
    // It is >= 2^-24 (far above the bound above) and, below the upper limit,
    // within a binary16 rounding of range / qmax, so the quotients keep the
    // same correctly rounded fast path.
    float step = fast ? markstein_div(range, qmax, inv_qmax) : range / qmax;
    if (!(step > 0.f)) step = 1.f;
    step = (float)(_Float16)fminf(fmaxf(step, 0x1p-24f), 65504.f);
    const float y = 1.0f / step;
    float zq = markstein_div(-mn, step, y);
    float qt[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) qt[j] = markstein_div(ws[j], step, y);
    if (__builtin_expect(!fast, 0)) {
      asm volatile("" ::: "memory");
      zq = -mn / step;
#pragma unroll
      for (int j = 0; j < 16; ++j) qt[j] = ws[j] / step;
    }
    static_assert(!kCentred, "the compact format writes codes");
    const float z = fminf(fmaxf(rintf(zq), 0.f), qmax);
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = fminf(fmaxf(rintf(qt[j]) + z, 0.f), qmax);
    step_out = step;
    z_out = z;
    return;
  }

  float step = markstein_div(range, qmax, inv_qmax);
  float y = 1.0f / step;
  float zq = markstein_div(-mn, step, y);
  float qt[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) qt[j] = markstein_div(ws[j], step, y);
  if (__builtin_expect(!fast, 0)) {
    // Outside the proven range: plain correctly rounded divides.  The empty
    // asm keeps this a real branch (no speculated divides on the fast path).
    asm volatile("" ::: "memory");
    step = range / qmax;
    if (!(step > 0.f)) step = 1.f;
    zq = -mn / step;
#pragma unroll
    for (int j = 0; j < 16; ++j) qt[j] = ws[j] / step;
  }
  const float z = fminf(fmaxf(rintf(zq), 0.f), qmax);
  if constexpr (kCentred) {
    const float lo = -z, hi = qmax - z;
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = __builtin_amdgcn_fmed3f(rintf(qt[j]), lo, hi);
  } else {
#pragma unroll
    for (int j = 0; j < 16; ++j) q[j] = fminf(fmaxf(rintf(qt[j]) + z, 0.f), qmax);
  }
  step_out = step;
  z_out = z;
}

// Eight codes -> one u32 (code j at bits 4j).  Codes are small integers, so
// a pair packs exactly as lo + 16*hi into one byte with v_cvt_pk_u8_f32.
__device__ __forceinline__ uint32_t pack8(const float* q) {
  uint32_t w = 0u;
#pragma unroll
  for (int b = 0; b < 4; ++b) w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[2 * b + 1], 16.f, q[2 * b]), b, w);
  return w;
}

// Output modes.  kPack: packed codes, steps and zeros.  kOperand: the
// search's weight operand B = bf16(f32(f32((q - z) * step) * inv_s[k])) as a
// bf16 [N][K] matrix, written once per candidate so that the contraction
// reads a plain bf16 operand instead of dequantizing it again for every tile
// of calibration tokens.  kDiffOp: D = B - W as bf16 [N][K], the operand whose
// product with X is the output error X B^T - X W^T itself.  That rounding is
// exact: B is nonzero only where |W s| >= step / 2, so B and W share a sign
// and B / W lies in [1/2, 2] (up to the roundings of s and 1/s), and by
// Sterbenz's lemma the difference of two such bf16 values is a bf16 value.
// kDiff: for the Gram-form loss D G D^T, D as fp32 [N][K] and the operand
// [D | D] as bf16 [N][2K] (against [hi(G) | lo(G)]).  kPack3: INT3 codes in
// the dense layout (each run of 32 codes along K is one 96-bit little-endian
// value, code i at bits 3i, in three u32 words), steps and zeros.
enum QuantMode { kPack = 0, kOperand = 1, kDiff = 2, kDiffOp = 3, kPack3 = 4 };
// Modes that write codes (the rest write a dequantized operand).
constexpr bool writes_codes(int mode) { return mode == kPack || mode == kPack3; }

// Sixteen 3-bit codes (as floats) -> the 48-bit value sum q_i << 3i, split
// into bits 0..31 and 32..47.
__device__ __forceinline__ void pack48(const float (&q)[16], uint32_t& lo, uint32_t& hi) {
  lo = 0;
  hi = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const uint32_t c = (uint32_t)q[i];
    const int b = 3 * i;
    if (b + 3 <= 32) {
      lo |= c << b;
    } else if (b >= 32) {
      hi |= c << (b - 32);
    } else {
      lo |= c << b;
      hi |= c >> (32 - b);
    }
  }
}

// kHalf (code modes only): the compact format, binary16 steps in steps16
// [N][G] and zeros two per byte in zeros [N][ceil(G/2)] (even group in the
// low nibble; the high nibble past the last group is 0).
template <int BITS, int kMode, bool kHalf = false>
__global__ __launch_bounds__(kThreads) void quantize_kernel(
    const uint16_t* __restrict__ w, int64_t N, int64_t K, const float* __restrict__ s,
    const int32_t* __restrict__ s_sel, const float* __restrict__ inv_s,
    uint32_t* __restrict__ qweight, float* __restrict__ scales, uint8_t* __restrict__ zeros,
    uint16_t* __restrict__ bout, float* __restrict__ dout, uint16_t* __restrict__ steps16) {
  static_assert(!kHalf || writes_codes(kMode), "the compact format is a code mode");
  const int64_t G = K / kGroup;
  const int64_t g = (int64_t)blockIdx.x * kGroupsPerBlock + (threadIdx.x / kLanesPerGroup);
  const int t8 = threadIdx.x % kLanesPerGroup;
  const bool gvalid = g < G;
  const int64_t k0 = (gvalid ? g : 0) * kGroup + t8 * 16;

  auto load16 = [&](const float* row, float (&v)[16]) {
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const float4 t = *(const float4*)(row + k0 + 4 * c);
      v[4 * c] = t.x; v[4 * c + 1] = t.y; v[4 * c + 2] = t.z; v[4 * c + 3] = t.w;
    }
  };
  float sv[16], iv[16];
  const float* srow = s;
  if (s != nullptr && s_sel != nullptr) srow = s + (int64_t)max(*s_sel, 0) * K;
  if (srow != nullptr) load16(srow, sv);
  if constexpr (!writes_codes(kMode)) {
    // No inverse scale: a factor of 1, which every multiply keeps exactly,
    // so the loop below multiplies unconditionally (no per-element select).
    if (inv_s != nullptr) {
      load16(inv_s, iv);
    } else {
#pragma unroll
      for (int j = 0; j < 16; ++j) iv[j] = 1.0f;
    }
  }

  // Rows in a grid-stride loop: each block takes kRows rows at a time and
  // issues the loads of its next kRows before quantizing the current ones,
  // so the memory pipe stays busy through the arithmetic (a block that loads,
  // then computes, then stores leaves it idle for much of its life).
  auto load_rows = [&](uint4 (&v)[kRows][2], int64_t nb) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t n = nb + r;
      const bool ok = gvalid && n < N;
      const uint16_t* src = w + (ok ? n : 0) * K + k0;
      v[r][0] = ok ? load_stream16(src) : make_uint4(0, 0, 0, 0);
      v[r][1] = ok ? load_stream16(src + 8) : make_uint4(0, 0, 0, 0);
    }
  };
  auto process_rows = [&](const uint4 (&v)[kRows][2], int64_t n_begin) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t n = n_begin + r;
      float ws[16];
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        ws[8 * c + 0] = bf16_lo(v[r][c].x); ws[8 * c + 1] = bf16_hi(v[r][c].x);
        ws[8 * c + 2] = bf16_lo(v[r][c].y); ws[8 * c + 3] = bf16_hi(v[r][c].y);
        ws[8 * c + 4] = bf16_lo(v[r][c].z); ws[8 * c + 5] = bf16_hi(v[r][c].z);
        ws[8 * c + 6] = bf16_lo(v[r][c].w); ws[8 * c + 7] = bf16_hi(v[r][c].w);
      }
      float wv[16];
#pragma unroll
      for (int j = 0; j < 16; ++j) wv[j] = ws[j];
      if (srow != nullptr) {
#pragma unroll
        for (int j = 0; j < 16; ++j) ws[j] *= sv[j];
      }
      float q[16], step, z;
      quantize16<BITS, kHalf, !writes_codes(kMode)>(ws, q, step, z);
      // The zero of the neighbouring group (lanes ^ 8: same row, group g ^ 1).
      uint32_t z_next = 0u;
      if constexpr (kHalf) z_next = (uint32_t)__shfl_xor((int)z, kLanesPerGroup);
      uint32_t p_lo = 0, p_hi = 0, o_lo = 0, o_hi = 0;
      if constexpr (kMode == kPack3) {
        // Lanes 2m and 2m+1 hold the two halves of one 32-code run; the even
        // lane takes its neighbour's 48 bits (quad_perm [1,0,3,2]) and writes
        // the run's three words.  Both lanes of a pair are active or inactive
        // together (same group and row).
        pack48(q, p_lo, p_hi);
        o_lo = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p_lo, 0xB1, 0xF, 0xF, false);
        o_hi = (uint32_t)__builtin_amdgcn_update_dpp(0, (int)p_hi, 0xB1, 0xF, 0xF, false);
      }
      if (!(gvalid && n < N)) continue;
      if constexpr (!writes_codes(kMode)) {
        float bv[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) {
          bv[j] = q[j] * step * iv[j];                // q holds q - z: two roundings
        }
        uint32_t d[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) d[j] = pack_bf16x2(bv[2 * j], bv[2 * j + 1]);
        if constexpr (kMode == kOperand) {
          uint4* dst = (uint4*)(bout + n * K + k0);
          dst[0] = make_uint4(d[0], d[1], d[2], d[3]);
          dst[1] = make_uint4(d[4], d[5], d[6], d[7]);
        } else if constexpr (kMode == kDiffOp) {
          uint32_t e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j)
            e[j] = pack_bf16x2(bf16_lo(d[j]) - wv[2 * j], bf16_hi(d[j]) - wv[2 * j + 1]);
          uint4* dst = (uint4*)(bout + n * K + k0);
          dst[0] = make_uint4(e[0], e[1], e[2], e[3]);
          dst[1] = make_uint4(e[4], e[5], e[6], e[7]);
        } else {
          static_assert(kMode == kDiff, "unhandled operand mode");
          float dd[16];
          uint32_t e[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            dd[2 * j] = bf16_lo(d[j]) - wv[2 * j];
            dd[2 * j + 1] = bf16_hi(d[j]) - wv[2 * j + 1];
            e[j] = pack_bf16x2(dd[2 * j], dd[2 * j + 1]);
          }
          float4* df = (float4*)(dout + n * K + k0);
#pragma unroll
          for (int c = 0; c < 4; ++c)
            df[c] = make_float4(dd[4 * c], dd[4 * c + 1], dd[4 * c + 2], dd[4 * c + 3]);
          uint16_t* arow = bout + n * 2 * K;
          const uint4 e0 = make_uint4(e[0], e[1], e[2], e[3]);
          const uint4 e1 = make_uint4(e[4], e[5], e[6], e[7]);
          ((uint4*)(arow + k0))[0] = e0;
          ((uint4*)(arow + k0))[1] = e1;
          ((uint4*)(arow + K + k0))[0] = e0;
          ((uint4*)(arow + K + k0))[1] = e1;
        }
      } else {
        static_assert(writes_codes(kMode), "unhandled code mode");
        if constexpr (kMode == kPack3) {
          if ((t8 & 1) == 0) {
            uint32_t* dst = qweight + n * (3 * K / 32) + (k0 / 32) * 3;
            dst[0] = p_lo;
            dst[1] = p_hi | (o_lo << 16);
            dst[2] = (o_lo >> 16) | (o_hi << 16);
          }
        } else {
          *(uint2*)(qweight + n * (K / 8) + k0 / 8) = make_uint2(pack8(q), pack8(q + 8));
        }
        if (t8 == 0) {
          if constexpr (kHalf) {
            steps16[n * G + g] = __builtin_bit_cast(uint16_t, (_Float16)step);   // exact
            if ((g & 1) == 0)
              zeros[n * ((G + 1) / 2) + g / 2] = (uint8_t)((uint32_t)z | (g + 1 < G ? z_next << 4 : 0u));
          } else {
            scales[n * G + g] = step;
            zeros[n * G + g] = (uint8_t)z;
          }
        }
      }
    }
  };
  const int64_t stride = (int64_t)gridDim.y * kRows;
  int64_t nb = (int64_t)blockIdx.y * kRows;
  uint4 va[kRows][2], vb[kRows][2];
  load_rows(va, nb);
  while (nb < N) {                       // uniform across the block
    load_rows(vb, nb + stride);
    process_rows(va, nb);
    nb += stride;
    if (nb >= N) break;
    load_rows(va, nb + stride);
    process_rows(vb, nb);
    nb += stride;
  }
}

// Compact metadata -> fp32 steps and u8 zeros, one thread per (row, group).
__global__ __launch_bounds__(256) void expand_meta16_kernel(const uint16_t* __restrict__ steps16,
                                                            const uint8_t* __restrict__ zeros4,
                                                            int64_t N, int64_t G,
                                                            float* __restrict__ scales,
                                                            uint8_t* __restrict__ zeros) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= N * G) return;
  const int64_t n = i / G, g = i - n * G;
  scales[i] = (float)__builtin_bit_cast(_Float16, steps16[i]);
  zeros[i] = (uint8_t)((zeros4[n * ((G + 1) / 2) + g / 2] >> (4 * (g & 1))) & 15);
}

// Blocks along K cover kGroupsPerBlock groups each; along N, enough row
// slots for about eight blocks per CU (the rest is the grid-stride loop).
dim3 quant_grid(int64_t N, int64_t K) {
  const int64_t gx = ceil_div(K / kGroup, (int64_t)kGroupsPerBlock);
  const int64_t gy = std::min(ceil_div(N, (int64_t)kRows), std::max((int64_t)1, (int64_t)2048 / gx));
  return dim3((unsigned)gx, (unsigned)gy);
}

}  // namespace

hipError_t launch_quantize_pack16(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                  int bits, bool int3_dense, uint32_t* qweight, uint16_t* steps16,
                                  uint8_t* zeros4, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const dim3 grid = quant_grid(N, K);
  if (int3_dense)
    quantize_kernel<3, kPack3, true><<<grid, kThreads, 0, stream>>>(
        w, N, K, s, nullptr, nullptr, qweight, nullptr, zeros4, nullptr, nullptr, steps16);
  else if (bits == 4)
    quantize_kernel<4, kPack, true><<<grid, kThreads, 0, stream>>>(
        w, N, K, s, nullptr, nullptr, qweight, nullptr, zeros4, nullptr, nullptr, steps16);
  else
    quantize_kernel<3, kPack, true><<<grid, kThreads, 0, stream>>>(
        w, N, K, s, nullptr, nullptr, qweight, nullptr, zeros4, nullptr, nullptr, steps16);
  return hipGetLastError();
}

hipError_t launch_expand_meta16(const uint16_t* steps16, const uint8_t* zeros4, int64_t N,
                                int64_t G, float* scales, uint8_t* zeros, hipStream_t stream) {
  if (N == 0 || G == 0) return hipSuccess;
  expand_meta16_kernel<<<(unsigned)ceil_div(N * G, (int64_t)256), 256, 0, stream>>>(
      steps16, zeros4, N, G, scales, zeros);
  return hipGetLastError();
}

hipError_t launch_quantize_pack(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                const int32_t* s_sel, int bits, uint32_t* qweight,
                                float* scales, uint8_t* zeros, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const dim3 grid = quant_grid(N, K);
  if (bits == 4)
    quantize_kernel<4, kPack><<<grid, kThreads, 0, stream>>>(w, N, K, s, s_sel, nullptr, qweight,
                                                             scales, zeros, nullptr, nullptr, nullptr);
  else
    quantize_kernel<3, kPack><<<grid, kThreads, 0, stream>>>(w, N, K, s, s_sel, nullptr, qweight,
                                                             scales, zeros, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_pack3(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                 uint32_t* qweight3, float* scales, uint8_t* zeros,
                                 hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const dim3 grid = quant_grid(N, K);
  quantize_kernel<3, kPack3><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, nullptr, qweight3,
                                                            scales, zeros, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_dequant(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                   const float* inv_s, int bits, uint16_t* b_out,
                                   hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const dim3 grid = quant_grid(N, K);
  if (bits == 4)
    quantize_kernel<4, kOperand><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, inv_s, nullptr,
                                                                nullptr, nullptr, b_out, nullptr, nullptr);
  else
    quantize_kernel<3, kOperand><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, inv_s, nullptr,
                                                                nullptr, nullptr, b_out, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_diff_operand(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                        const float* inv_s, int bits, uint16_t* d_out,
                                        hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const dim3 grid = quant_grid(N, K);
  if (bits == 4)
    quantize_kernel<4, kDiffOp><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, inv_s, nullptr,
                                                               nullptr, nullptr, d_out, nullptr, nullptr);
  else
    quantize_kernel<3, kDiffOp><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, inv_s, nullptr,
                                                               nullptr, nullptr, d_out, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_diff(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                const float* inv_s, int bits, uint16_t* a_split, float* d32,
                                hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const dim3 grid = quant_grid(N, K);
  if (bits == 4)
    quantize_kernel<4, kDiff><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, inv_s, nullptr,
                                                             nullptr, nullptr, a_split, d32, nullptr);
  else
    quantize_kernel<3, kDiff><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, inv_s, nullptr,
                                                             nullptr, nullptr, a_split, d32, nullptr);
  return hipGetLastError();
}

}  // namespace awq
