// Device helpers for the gfx950 kernels of libawq_mi355x.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace awq {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// 16-byte streaming load (data read once: bypass cache retention).
__device__ __forceinline__ uint4 load_stream16(const void* p) {
  const u32x4 v = __builtin_nontemporal_load((const u32x4*)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// bf16 is the top half of a binary32: widening is a shift.
__device__ __forceinline__ float bf16_lo(uint32_t pair) { return __uint_as_float(pair << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t pair) { return __uint_as_float(pair & 0xFFFF0000u); }

// Two binary32 values -> packed bf16 pair, round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950 (converting the halves separately costs two
// converts and an or).  `lo` lands in bits 0..15.
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
}

// Dense INT3 (each run of 32 codes along K one 96-bit little-endian value in
// three u32 words, code i at bit 3i) widened to 4-bit fields: each 24-bit
// run of 8 codes is spread so that code i lands at bit 4i of one u32.
__device__ __forceinline__ uint32_t spread3(uint32_t f) {
  const uint32_t y = (f & 0xFFFu) | ((f & 0xFFF000u) << 4);   // codes 0-3 | codes 4-7 << 16
  return (y & 0x00070007u) | ((y & 0x00380038u) << 1) | ((y & 0x01C001C0u) << 2) |
         ((y & 0x0E000E00u) << 3);
}
// The three words of one 32-code run (v.w unused) -> four words of nibbles.
__device__ __forceinline__ uint4 nibbles_from_int3(uint4 v) {
  return make_uint4(spread3(v.x & 0xFFFFFFu), spread3((v.x >> 24) | ((v.y & 0xFFFFu) << 8)),
                    spread3((v.y >> 16) | ((v.z & 0xFFu) << 16)), spread3(v.z >> 8));
}

__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

}  // namespace awq
