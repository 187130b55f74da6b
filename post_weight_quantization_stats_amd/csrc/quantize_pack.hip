// Group-wise asymmetric quantization and packing of W . diag(s)
// (robotsatlas AWQ page, "How it works": group-wise quantization once the
// scales are set; "Components": groups of 128 with a per-group scale;
// "Hyperparameters": 4 or 3 bits; builderai AWQ page, "About": the real
// integer weights are written).
//
// Layout: a block of 256 lanes owns 32 groups (4096 channels) of a row, in
// two halves of 2048 channels; lane l holds channels 8l .. 8l+7 of each
// half, so every load and store instruction of a wave covers one contiguous
// span (two 16-byte pieces 16 bytes apart per lane, the previous layout, ran
// about 10% slower in a plain copy of the same bytes).  The 16 lanes of a
// DPP row hold one group per half; its min/max is reduced in four DPP steps
// (quad swaps, half-row mirror, row mirror) on the values' bit patterns.
// Each block takes 4 rows per step.  The operand modes launch one block per
// step (every row read once, no loop); the code modes run a grid-stride loop
// over about 32 blocks per CU, the next rows' loads issued before the
// current ones are quantized.  Every arithmetic step is one
// IEEE fp32 operation, in the order of the contract: ws = w*s;
// step = (max(mx,0) - min(mn,0)) / qmax (1 if 0); z = clamp(rint(-mn/step));
// q = clamp(rint(ws/step) + z).
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
// ranges) take plain IEEE divisions.  y = RN(1/step) is the hardware
// reciprocal refined by one Newton step with a fused residual; that equals
// the IEEE quotient 1/b for every binary32 b with exponent -100 .. 100
// (checked exhaustively on the device, 1.69e9 values), which holds every
// step of the fast path.
#include <math.h>

#include <algorithm>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int kThreads = 256;
constexpr int kLanesPerGroup = 16;
constexpr int kGroupsPerBlock = 32;
constexpr int kHalfGroups = kGroupsPerBlock / 2;
constexpr int kRowsCodes = 4;         // rows per step: the code modes
constexpr int kRowsOperand = 4;       // the operand modes

typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t row_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           0x00020000);
}

// 16 bytes at voff; kAux 2: non-temporal.
template <int kAux>
__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t voff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, 0, kAux);
  return make_uint4(v.x, v.y, v.z, v.w);
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}

// RN(1 / b) for b with exponent -100 .. 100: the hardware reciprocal and one
// Newton step with a fused residual (equal to the IEEE quotient there).
__device__ __forceinline__ float rcp_rn(float b) {
  const float y0 = __builtin_amdgcn_rcpf(b);
  return fmaf(fmaf(-b, y0, 1.0f), y0, y0);
}

__device__ __forceinline__ float markstein_div(float a, float b, float y) {
  const float q0 = a * y;
  const float r = fmaf(-q0, b, a);              // exact residual
  return fmaf(r, y, q0);                        // RN(a / b)
}

// One lane's 8 channels of a group: their codes (as floats) and the group's
// step and zero (identical in all 16 lanes of the group).  kCentred: q[j]
// holds the centred code q - z instead, formed as clamp(rint(ws/step), -z,
// qmax - z) (equal to clamp(rint(ws/step) + z, 0, qmax) - z: every value is a
// small integer), one median instead of an add, a clamp and a subtract.
template <int BITS, bool kHalf = false, bool kCentred = false>
__device__ __forceinline__ void quantize8(const float (&ws)[8], float (&q)[8],
                                          float& step_out, float& z_out) {
  constexpr float qmax = (float)((1 << BITS) - 1);
  constexpr float inv_qmax = 1.0f / qmax;       // RN(1/qmax), folded by the compiler
  // max(0, max ws) and min(0, min ws) on the bit patterns (finite inputs):
  // as signed integers, non-negative floats order like their values and
  // every negative float is below 0; as unsigned integers, negative floats
  // order by magnitude above every non-negative one.  So the signed max
  // with 0 is max(0, max ws), and the unsigned max is the most negative
  // member (or a non-negative value, which the signed min with 0 turns into
  // +0).  Integer max needs no canonicalisation and folds into the DPP moves.
  int32_t mxi = 0;
  uint32_t mnu = 0u;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    mxi = max(mxi, (int32_t)__float_as_uint(ws[j]));
    mnu = max(mnu, __float_as_uint(ws[j]));
  }
  mxi = max(mxi, (int32_t)dpp<0xB1>((uint32_t)mxi));    // lanes ^1
  mnu = max(mnu, dpp<0xB1>(mnu));
  mxi = max(mxi, (int32_t)dpp<0x4E>((uint32_t)mxi));    // lanes ^2
  mnu = max(mnu, dpp<0x4E>(mnu));
  mxi = max(mxi, (int32_t)dpp<0x141>((uint32_t)mxi));   // lane i <-> 7-i of each half row
  mnu = max(mnu, dpp<0x141>(mnu));
  mxi = max(mxi, (int32_t)dpp<0x140>((uint32_t)mxi));   // lane i <-> 15-i of the row
  mnu = max(mnu, dpp<0x140>(mnu));
  const float mx = __int_as_float(mxi);
  const float mn = __int_as_float(min((int32_t)mnu, 0));
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
    const float y = rcp_rn(step);
    float zq = markstein_div(-mn, step, y);
    float qt[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) qt[j] = markstein_div(ws[j], step, y);
    if (__builtin_expect(!fast, 0)) {
      asm volatile("" ::: "memory");
      zq = -mn / step;
#pragma unroll
      for (int j = 0; j < 8; ++j) qt[j] = ws[j] / step;
    }
    static_assert(!kCentred, "the compact format writes codes");
    const float z = fminf(fmaxf(rintf(zq), 0.f), qmax);
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = fminf(fmaxf(rintf(qt[j]) + z, 0.f), qmax);
    step_out = step;
    z_out = z;
    return;
  }

  float step = markstein_div(range, qmax, inv_qmax);
  float y = rcp_rn(step);
  float zq = markstein_div(-mn, step, y);
  float qt[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) qt[j] = markstein_div(ws[j], step, y);
  if (__builtin_expect(!fast, 0)) {
    // Outside the proven range: plain correctly rounded divides.  The empty
    // asm keeps this a real branch (no speculated divides on the fast path).
    asm volatile("" ::: "memory");
    step = range / qmax;
    if (!(step > 0.f)) step = 1.f;
    zq = -mn / step;
#pragma unroll
    for (int j = 0; j < 8; ++j) qt[j] = ws[j] / step;
  }
  const float z = fminf(fmaxf(rintf(zq), 0.f), qmax);
  if constexpr (kCentred) {
    const float lo = -z, hi = qmax - z;
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = __builtin_amdgcn_fmed3f(rintf(qt[j]), lo, hi);
  } else {
#pragma unroll
    for (int j = 0; j < 8; ++j) q[j] = fminf(fmaxf(rintf(qt[j]) + z, 0.f), qmax);
  }
  step_out = step;
  z_out = z;
}

// Eight codes -> one u32 (code j at bits 4j).  Codes are small integers, so
// a pair packs exactly as lo + 16*hi into one byte with v_cvt_pk_u8_f32.
__device__ __forceinline__ uint32_t pack8(const float (&q)[8]) {
  uint32_t w = 0u;
#pragma unroll
  for (int b = 0; b < 4; ++b) w = __builtin_amdgcn_cvt_pk_u8_f32(fmaf(q[2 * b + 1], 16.f, q[2 * b]), b, w);
  return w;
}

// Eight 3-bit codes (as floats) -> the 24-bit value sum q_i << 3i.
__device__ __forceinline__ uint32_t pack24(const float (&q)[8]) {
  uint32_t c = 0u;
#pragma unroll
  for (int i = 0; i < 8; ++i) c |= (uint32_t)q[i] << (3 * i);
  return c;
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
constexpr int rows_per_step(int mode) { return writes_codes(mode) ? kRowsCodes : kRowsOperand; }

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
  const int lane = threadIdx.x;
  const int j16 = lane % kLanesPerGroup;        // position inside the group
  // Half h: group g[h], the lane's channels k[h] .. k[h] + 7 (an invalid
  // group past G reads the last group's channels and stores nothing).
  int64_t g[2], k[2];
  bool gvalid[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    g[h] = (int64_t)blockIdx.x * kGroupsPerBlock + h * kHalfGroups + lane / kLanesPerGroup;
    gvalid[h] = g[h] < G;
    k[h] = (gvalid[h] ? g[h] : G - 1) * kGroup + 8 * j16;
  }

  auto load8 = [&](const float* row, float (&v)[2][8]) {
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const float4 t = *(const float4*)(row + k[h] + 4 * c);
        v[h][4 * c] = t.x; v[h][4 * c + 1] = t.y; v[h][4 * c + 2] = t.z; v[h][4 * c + 3] = t.w;
      }
  };
  float sv[2][8], iv[2][8];
  const float* srow = s;
  if (s != nullptr && s_sel != nullptr) srow = s + (int64_t)max(*s_sel, 0) * K;
  if (srow != nullptr) load8(srow, sv);
  if constexpr (!writes_codes(kMode)) {
    // No inverse scale: a factor of 1, which every multiply keeps exactly,
    // so the loop below multiplies unconditionally (no per-element select).
    if (inv_s != nullptr) {
      load8(inv_s, iv);
    } else {
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int j = 0; j < 8; ++j) iv[h][j] = 1.0f;
    }
  }

  // Row indices are 32-bit (N < 2^31) and uniform, so each row's base lives
  // in scalar registers (one buffer resource per row) and the lane's offsets
  // in the row are fixed: no per-row vector address arithmetic, whose
  // temporaries would otherwise share registers with loads in flight and
  // make the wave wait for its own prefetch.  Rows past N re-read row N - 1
  // (never stored).
  // Non-temporal loads where the weight is only read (the code modes: pack
  // 230 -> 208 us on the 57344 x 8192 weight); the operand modes, which
  // write as much as they read, were 1-2% slower with them.
  constexpr int kLoadAux = writes_codes(kMode) ? 2 : 0;
  const uint32_t n_last = (uint32_t)N - 1u;
  const uint32_t off0 = (uint32_t)(k[0] * 2), off1 = (uint32_t)(k[1] * 2);
  constexpr int kRows = rows_per_step(kMode);
  auto load_rows = [&](uint4 (&v)[kRows][2], uint32_t nb) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const uint32_t n = min(nb + (uint32_t)r, n_last);
      const rsrc_t rw = row_rsrc(w + (int64_t)n * K, K * 2);
      v[r][0] = ld16<kLoadAux>(rw, off0);
      v[r][1] = ld16<kLoadAux>(rw, off1);
    }
  };
  auto process_rows = [&](const uint4 (&v)[kRows][2], uint32_t n_begin) {
#pragma unroll
    for (int r = 0; r < kRows; ++r) {
      const int64_t n = (int64_t)n_begin + r;
      const bool row_ok = n_begin + (uint32_t)r < (uint32_t)N;   // scalar compare
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        float ws[8];
        ws[0] = bf16_lo(v[r][h].x); ws[1] = bf16_hi(v[r][h].x);
        ws[2] = bf16_lo(v[r][h].y); ws[3] = bf16_hi(v[r][h].y);
        ws[4] = bf16_lo(v[r][h].z); ws[5] = bf16_hi(v[r][h].z);
        ws[6] = bf16_lo(v[r][h].w); ws[7] = bf16_hi(v[r][h].w);
        float wv[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) wv[j] = ws[j];
        if (srow != nullptr) {
#pragma unroll
          for (int j = 0; j < 8; ++j) ws[j] *= sv[h][j];
        }
        float q[8], step, z;
        quantize8<BITS, kHalf, !writes_codes(kMode)>(ws, q, step, z);
        // The zero of the neighbouring group (lanes ^ 16: same row and half,
        // group g ^ 1).
        uint32_t z_next = 0u;
        if constexpr (kHalf) z_next = (uint32_t)__shfl_xor((int)z, kLanesPerGroup);
        // Dense INT3: lanes 4m .. 4m+3 of a row hold one run of 32 codes,
        // 24 bits each; lane 4m+i (i < 3) writes the run's word i from its
        // own bits and its right neighbour's (quad_perm [1,2,3,3]).
        uint32_t c24 = 0u, c24_next = 0u;
        if constexpr (kMode == kPack3) {
          c24 = pack24(q);
          c24_next = dpp<0xF9>(c24);
        }
        if (!(gvalid[h] && row_ok)) continue;
        if constexpr (!writes_codes(kMode)) {
          float bv[8];
#pragma unroll
          for (int j = 0; j < 8; ++j) {
            bv[j] = q[j] * step * iv[h][j];           // q holds q - z: two roundings
          }
          uint32_t d[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) d[j] = pack_bf16x2(bv[2 * j], bv[2 * j + 1]);
          if constexpr (kMode == kOperand) {
            *(uint4*)(bout + n * K + k[h]) = make_uint4(d[0], d[1], d[2], d[3]);
          } else if constexpr (kMode == kDiffOp) {
            uint32_t e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j)
              e[j] = pack_bf16x2(bf16_lo(d[j]) - wv[2 * j], bf16_hi(d[j]) - wv[2 * j + 1]);
            *(uint4*)(bout + n * K + k[h]) = make_uint4(e[0], e[1], e[2], e[3]);
          } else {
            static_assert(kMode == kDiff, "unhandled operand mode");
            float dd[8];
            uint32_t e[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              dd[2 * j] = bf16_lo(d[j]) - wv[2 * j];
              dd[2 * j + 1] = bf16_hi(d[j]) - wv[2 * j + 1];
              e[j] = pack_bf16x2(dd[2 * j], dd[2 * j + 1]);
            }
            float4* df = (float4*)(dout + n * K + k[h]);
            df[0] = make_float4(dd[0], dd[1], dd[2], dd[3]);
            df[1] = make_float4(dd[4], dd[5], dd[6], dd[7]);
            uint16_t* arow = bout + n * 2 * K;
            const uint4 ev = make_uint4(e[0], e[1], e[2], e[3]);
            *(uint4*)(arow + k[h]) = ev;
            *(uint4*)(arow + K + k[h]) = ev;
          }
        } else {
          static_assert(writes_codes(kMode), "unhandled code mode");
          if constexpr (kMode == kPack3) {
            const int i = j16 & 3;
            if (i < 3)
              qweight[n * (3 * K / 32) + (k[h] / 32) * 3 + i] =
                  (c24 >> (8 * i)) | (c24_next << (24 - 8 * i));
          } else {
            // Non-temporal: the codes are not read back here (pack 206 -> 203 us).
            __builtin_nontemporal_store(pack8(q), qweight + n * (K / 8) + k[h] / 8);
          }
          if (j16 == 0) {
            const int64_t gh = g[h];
            if constexpr (kHalf) {
              steps16[n * G + gh] = __builtin_bit_cast(uint16_t, (_Float16)step);   // exact
              if ((gh & 1) == 0)
                zeros[n * ((G + 1) / 2) + gh / 2] =
                    (uint8_t)((uint32_t)z | (gh + 1 < G ? z_next << 4 : 0u));
            } else {
              scales[n * G + gh] = step;
              zeros[n * G + gh] = (uint8_t)z;
            }
          }
        }
      }
    }
  };
  const uint32_t stride = gridDim.y * kRows, n_rows = (uint32_t)N;
  uint32_t nb = blockIdx.y * kRows;
  uint4 va[kRows][2], vb[kRows][2];
  load_rows(va, nb);
  if (stride >= n_rows) {                // one step per block: nothing to prefetch
    // (skipping the loads of the row past the end: dequant operand 329 -> 321 us)
    process_rows(va, nb);
    return;
  }
  while (nb < n_rows) {                  // uniform across the block
    load_rows(vb, nb + stride);
    process_rows(va, nb);
    nb += stride;
    if (nb >= n_rows) break;
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

// Blocks along K cover kGroupsPerBlock groups each.  Along N: the operand
// modes, which write as much as they read, one block per 4-row step (up to
// 65535 row slots, then the grid-stride loop); the code modes enough row
// slots for about 32 blocks per CU.  Measured on the 57344 x 8192 weight
// (us, difference operand / pack): 8 blocks per CU 355 / 230, 16: 350 / 208,
// 32: 341 / 206, 64: 329 / 207, one pass: 315 / 218; one pass with 1, 2 or 8
// rows per step: 426, 347, 341 for the difference operand.
dim3 quant_grid(int64_t N, int64_t K, int mode) {
  const int64_t gx = ceil_div(K / kGroup, (int64_t)kGroupsPerBlock);
  const int64_t rows = ceil_div(N, (int64_t)rows_per_step(mode));
  const int64_t gy = writes_codes(mode) ? std::min(rows, std::max((int64_t)1, (int64_t)8192 / gx))
                                        : std::min(rows, (int64_t)65535);
  return dim3((unsigned)gx, (unsigned)gy);
}

}  // namespace

hipError_t launch_quantize_pack16(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                  int bits, bool int3_dense, uint32_t* qweight, uint16_t* steps16,
                                  uint8_t* zeros4, hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const dim3 grid = quant_grid(N, K, kPack);
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
  const dim3 grid = quant_grid(N, K, kPack);
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
  const dim3 grid = quant_grid(N, K, kPack);
  quantize_kernel<3, kPack3><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, nullptr, qweight3,
                                                            scales, zeros, nullptr, nullptr, nullptr);
  return hipGetLastError();
}

hipError_t launch_quantize_dequant(const uint16_t* w, int64_t N, int64_t K, const float* s,
                                   const float* inv_s, int bits, uint16_t* b_out,
                                   hipStream_t stream) {
  if (N == 0) return hipSuccess;
  const dim3 grid = quant_grid(N, K, kOperand);
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
  const dim3 grid = quant_grid(N, K, kDiffOp);
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
  const dim3 grid = quant_grid(N, K, kDiff);
  if (bits == 4)
    quantize_kernel<4, kDiff><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, inv_s, nullptr,
                                                             nullptr, nullptr, a_split, d32, nullptr);
  else
    quantize_kernel<3, kDiff><<<grid, kThreads, 0, stream>>>(w, N, K, s, nullptr, inv_s, nullptr,
                                                             nullptr, nullptr, a_split, d32, nullptr);
  return hipGetLastError();
}

}  // namespace awq
