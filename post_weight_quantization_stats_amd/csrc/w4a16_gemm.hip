// W4A16 contraction Y = X . B^T with the weight operand dequantized on chip
// (builderai AWQ page, "About": kernels for 4-bit weights and 16-bit
// activations; robotsatlas AWQ page, "Implementation pitfalls": a separate
// dequantize-then-GEMM pass loses the benefit), with the squared error
// against the unquantized output fused into the epilogue (robotsatlas "How it
// works": the scale minimises the layer's output error).  The same template
// with a bf16 weight operand computes that unquantized output Y = X . W^T.
//
// gfx950 design
//   * 256x256 output tile per workgroup, BK = 32, 4 waves in a 2x2 grid; each
//     wave owns 128x128 = 4x4 v_mfma_f32_32x32x16_bf16 blocks (256 fp32
//     accumulators per lane, held in AGPRs).
//   * LDS tiles are [row][4 x 16 B chunks] with an XOR swizzle of the chunk
//     index that keeps ds_read_b128 of the MFMA fragment pattern free of bank
//     conflicts (8- and 16-lane phases alike).
//   * The activation tile (and the bf16 weight tile of the reference product)
//     is copied global -> LDS by the buffer unit (buffer_load_dwordx4 ... lds)
//     into a ring of 4 stages, three k-steps ahead; no VGPRs are involved.
//     Each stage is its own __shared__ array and the k-loop is unrolled by 4,
//     so the compiler sees which stage every DMA and every read touches and
//     waits (vmcnt) only for the copy a read depends on.
//   * Stages are published two k-steps ahead: before the barrier that ends
//     step k each wave waits for its own copy into stage k+2 (other waves
//     read it after the barrier).  So the fragments of step k+1's first k16
//     substep are read before that barrier, and those of the second substep
//     during the first substep's MFMAs; LDS latency never sits between a
//     barrier and the next MFMA.
//   * INT4 path: thread t owns weight row t of the tile.  Its 16 bytes of codes
//     for a k-step (plus the group's step and zero) are loaded three k-steps
//     ahead into one of two register sets; the dequantized bf16 values
//     B = bf16(f32(f32((q - z) * step) * inv_s[k])) are written into a
//     4-stage B ring two k-steps ahead, interleaved with the current step's
//     MFMAs.  inv_s[k] is uniform and comes from SGPRs.  The dequantized
//     operand is never written to HBM.
//   * Buffer resources: 32-bit per-lane offsets, the k offset in an SGPR,
//     and rows past M / N read as zero, so the loads need no branches.
//   * Workgroup ids are remapped so each XCD (ids are dealt round-robin over
//     the 8 XCDs) works on a compact group of tiles sharing A and B panels in
//     its L2.
//   * Epilogue: optional fp32 store of Y; optional fp64 sum of (Y - Y_ref)^2
//     per tile written to a partial slot (partials are reduced later in a
//     fixed order, so results are bit-reproducible).
#include <type_traits>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace {

constexpr int BM = kGemmBM;
constexpr int BN = kGemmBN;
constexpr int BK = 32;
constexpr int NT = 256;
constexpr int kChunks = BK / 8;             // 16-byte chunks per tile row
constexpr int kSlots = 256 * kChunks;       // 16-byte slots per operand tile (16 KiB)
constexpr int kDmaPerWave = 4;              // 1 KiB per DMA instruction, 4 KiB per wave
static_assert(BM == 256 && BN == 256 && NT == 256, "mapping assumes 256x256 tiles, 256 threads");
static_assert(kGroup % BK == 0, "a k-step must not straddle a quantization group");

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;

struct Params {
  const uint16_t* x;
  const uint16_t* w;
  const uint32_t* qweight;
  const float* scales;
  const uint8_t* zeros;
  const float* y_ref;
  float* y;
  double* partials;
  int64_t M, N, K;
  int64_t tiles_m, tiles_n;
};

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint64_t bytes) {
  const uint32_t n = bytes > 0xFFFFFFFFull ? 0xFFFFFFFFu : (uint32_t)bytes;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)n, 0x00020000);
}

__device__ __forceinline__ uint4 ld16(rsrc_t r, uint32_t voff, uint32_t soff) {
  const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// Swizzle of a row's chunk index: rows r, r+2, r+4, r+6 and rows r, r+4, r+8,
// r+12 all get different values, so 8-lane and 16-lane phases of a
// ds_read_b128 that walk consecutive rows at one chunk hit distinct banks.
__device__ __forceinline__ int chunk_swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ chunk_swz(row));
}

__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Tile of workgroup `bid`: ids are dealt round-robin over the 8 XCDs, so give
// each XCD a contiguous range, and walk it in column-major groups of 4
// M-tiles so concurrently resident tiles share A and B panels.
__device__ __forceinline__ void tile_coords(int64_t bid, int64_t tiles_m, int64_t tiles_n,
                                            int64_t& tm, int64_t& tn) {
  const int64_t T = tiles_m * tiles_n;
  int64_t id = bid;
  if ((T & 7) == 0) id = (bid & 7) * (T >> 3) + (bid >> 3);
  constexpr int64_t GM = 4;
  const int64_t group = id / (GM * tiles_n);
  const int64_t first_m = group * GM;
  const int64_t gm = min(GM, tiles_m - first_m);
  const int64_t in = id - group * GM * tiles_n;
  tm = first_m + in % gm;
  tn = in / gm;
}

// Eight codes (one u32, code i at bits 4i) -> eight bf16 weights.
template <bool kInvS>
__device__ __forceinline__ uint4 dequant8(uint32_t qw, float step, float zero, const float* inv) {
  const uint32_t e = qw & 0x0F0F0F0Fu;          // codes 0,2,4,6 in bytes 0..3
  const uint32_t o = (qw >> 4) & 0x0F0F0F0Fu;   // codes 1,3,5,7
  float d[8];
  d[0] = (float)(e & 0xFFu);
  d[1] = (float)(o & 0xFFu);
  d[2] = (float)((e >> 8) & 0xFFu);
  d[3] = (float)((o >> 8) & 0xFFu);
  d[4] = (float)((e >> 16) & 0xFFu);
  d[5] = (float)((o >> 16) & 0xFFu);
  d[6] = (float)(e >> 24);
  d[7] = (float)(o >> 24);
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    d[i] = (d[i] - zero) * step;          // exact difference, one fp32 rounding
    if constexpr (kInvS) d[i] = d[i] * inv[i];
  }
  uint4 r;
  r.x = pack_bf16x2(d[0], d[1]);
  r.y = pack_bf16x2(d[2], d[3]);
  r.z = pack_bf16x2(d[4], d[5]);
  r.w = pack_bf16x2(d[6], d[7]);
  return r;
}

struct CodeRegs {
  uint4 q;            // 32 codes of this thread's row for one k-step
  uint32_t step_bits; // raw; converted when used so the load stays in flight
  uint32_t zero;
};

template <bool kInt4, bool kInvS>
__global__ __launch_bounds__(NT, 1) void gemm_kernel(Params p, const float* __restrict__ inv_s) {
  // Separate objects per stage: the compiler tracks LDS-DMA writes per object.
  __shared__ uint4 sa0[kSlots], sa1[kSlots], sa2[kSlots], sa3[kSlots];
  __shared__ uint4 sb0[kSlots], sb1[kSlots], sb2[kSlots], sb3[kSlots];
  uint4* const SA[4] = {sa0, sa1, sa2, sa3};
  uint4* const SB[4] = {sb0, sb1, sb2, sb3};

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int lr = lane & 31, lk = lane >> 5;

  int64_t tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t G = K / kGroup;

  // DMA mapping: instruction i of wave w fills slots [(4w+i)*64, +64): lane L
  // -> row 64w + 16i + L/4, physical chunk L%4 = logical chunk ^ swizzle.
  uint32_t dma_off[kDmaPerWave];
#pragma unroll
  for (int i = 0; i < kDmaPerWave; ++i) {
    const int row = 64 * wave + 16 * i + (lane >> 2);
    const int chunk = (lane & 3) ^ chunk_swz(row);
    dma_off[i] = (uint32_t)(row * K * 2 + chunk * 16);
  }
  const int dma_slot = wave * (kDmaPerWave * 64);

  const rsrc_t ra = make_rsrc(p.x + m0 * K, (uint64_t)(M - m0) * K * 2);
  rsrc_t rb, rq, rsc, rz;
  if constexpr (kInt4) {
    rq = make_rsrc(p.qweight + n0 * (K / 8), (uint64_t)(N - n0) * (K / 2));
    rsc = make_rsrc(p.scales + n0 * G, (uint64_t)(N - n0) * G * 4);
    rz = make_rsrc(p.zeros + n0 * G, (uint64_t)(N - n0) * G);
  } else {
    rb = make_rsrc(p.w + n0 * K, (uint64_t)(N - n0) * K * 2);
  }
  const uint32_t q_off = (uint32_t)(t * (K / 2));
  const uint32_t sc_off = (uint32_t)(t * G * 4);
  const uint32_t z_off = (uint32_t)(t * G);

  auto dma_tile = [&](rsrc_t r, uint4* stage, int64_t k0) {
#pragma unroll
    for (int i = 0; i < kDmaPerWave; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(stage + dma_slot + 64 * i), 16,
                                               dma_off[i], (uint32_t)(k0 * 2), 0, 0);
  };
  auto load_codes = [&](CodeRegs& C, int64_t k0) {
    C.q = ld16(rq, q_off, (uint32_t)(k0 / 2));
    const uint32_t g = (uint32_t)(k0 / kGroup);
    C.step_bits = __builtin_amdgcn_raw_buffer_load_b32(rsc, sc_off, g * 4, 0);
    C.zero = __builtin_amdgcn_raw_buffer_load_b8(rz, z_off, g, 0);
  };
  // Dequantize the codes into row t of a B stage.  The empty asm statements
  // pin the first use of each loaded register to this point (after the
  // previous barrier); otherwise the scheduler hoists the conversion up to the
  // load and the wait for it drains every later prefetch.
  auto dequant_half = [&](const CodeRegs& C, uint4* stage, int64_t k0, int w0) {
    uint32_t sbits = C.step_bits, zraw = C.zero;
    uint32_t words[2] = {w0 == 0 ? C.q.x : C.q.z, w0 == 0 ? C.q.y : C.q.w};
    asm volatile("" : "+v"(sbits), "+v"(zraw), "+v"(words[0]), "+v"(words[1]));
    const float step = __uint_as_float(sbits);
    const float zero = (float)zraw;
#pragma unroll
    for (int w = 0; w < 2; ++w)
      stage[swz(t, w0 + w)] = dequant8<kInvS>(words[w], step, zero,
                                              kInvS ? inv_s + k0 + 8 * (w0 + w) : nullptr);
  };
  // Wait until this wave's DMA into `stage` has landed (the compiler inserts
  // the exact vmcnt for a read of an object with a pending DMA write).
  auto own_dma_done = [&](const uint4* stage) {
    const uint32_t v = *(const uint32_t*)(stage + dma_slot);
    asm volatile("" ::"v"(v));
  };

  f32x16 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  struct Frags {
    bf16x8 a[4], b[4];
  };
  auto read_frags = [&](Frags& F, const uint4* la, const uint4* lb, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      F.a[i] = __builtin_bit_cast(bf16x8, la[swz(wm * 128 + i * 32 + lr, 2 * s + lk)]);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      F.b[j] = __builtin_bit_cast(bf16x8, lb[swz(wn * 128 + j * 32 + lr, 2 * s + lk)]);
  };
  auto mfma16 = [&](const Frags& F) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[i], F.b[j], acc[i][j], 0, 0, 0);
  };

  const int64_t KT = K / BK;   // multiple of 4 (K is a multiple of 128)
  CodeRegs C[2];
  Frags F0, F1;

  // Prologue: A(0..2) [and bf16 B(0..2)] in flight; INT4 B(0), B(1)
  // dequantized; stages 0 and 1 published; step 0's first fragments read.
  dma_tile(ra, SA[0], 0);
  dma_tile(ra, SA[1], BK);
  dma_tile(ra, SA[2], 2 * BK);
  if constexpr (kInt4) {
    load_codes(C[0], 0);
    load_codes(C[1], BK);
    dequant_half(C[0], SB[0], 0, 0);
    dequant_half(C[0], SB[0], 0, 2);
    dequant_half(C[1], SB[1], BK, 0);
    dequant_half(C[1], SB[1], BK, 2);
    load_codes(C[0], 2 * BK);
  } else {
    dma_tile(rb, SB[0], 0);
    dma_tile(rb, SB[1], BK);
    dma_tile(rb, SB[2], 2 * BK);
    own_dma_done(SB[0]);
    own_dma_done(SB[1]);
  }
  own_dma_done(SA[0]);
  own_dma_done(SA[1]);
  barrier_lds();
  read_frags(F0, SA[0], SB[0], 0);

  // One k-step; every stage index is a compile-time constant.  The loads are
  // issued unconditionally (also past the end of K, where they read other
  // rows' data or zeros into stages that are never read), so the compiler's
  // wait counts are exact on every path.
  auto step = [&](int64_t k, auto I) {
    constexpr int i = decltype(I)::value;      // k % 4
    dma_tile(ra, SA[(i + 3) & 3], (k + 3) * BK);
    if constexpr (kInt4) {
      load_codes(C[(i + 1) & 1], (k + 3) * BK);
    } else {
      dma_tile(rb, SB[(i + 3) & 3], (k + 3) * BK);
    }
    read_frags(F1, SA[i], SB[i], 1);
    mfma16(F0);
    if constexpr (kInt4) dequant_half(C[i & 1], SB[(i + 2) & 3], (k + 2) * BK, 0);
    __builtin_amdgcn_sched_barrier(0);
    mfma16(F1);
    if constexpr (kInt4) dequant_half(C[i & 1], SB[(i + 2) & 3], (k + 2) * BK, 2);
    read_frags(F0, SA[(i + 1) & 3], SB[(i + 1) & 3], 0);
    __builtin_amdgcn_sched_barrier(0);
    own_dma_done(SA[(i + 2) & 3]);
    if constexpr (!kInt4) own_dma_done(SB[(i + 2) & 3]);
    barrier_lds();
  };

  for (int64_t k = 0; k < KT; k += 4) {
    step(k, std::integral_constant<int, 0>{});
    step(k + 1, std::integral_constant<int, 1>{});
    step(k + 2, std::integral_constant<int, 2>{});
    step(k + 3, std::integral_constant<int, 3>{});
  }

  // Epilogue.  32x32 block layout: lane holds column (lane & 31) and rows
  // 8*(r/4) + 4*(lane/32) + r%4 for accumulator register r.
  const int64_t row0 = wm * 128 + 4 * lk;        // within the tile
  const int64_t col0 = n0 + wn * 128 + lr;
  if (p.y != nullptr) {
    // Rows past M fall outside the buffer resource and are dropped.
    const rsrc_t ro = make_rsrc(p.y + m0 * N + n0, ((uint64_t)(M - m0) * N - n0) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if (n0 + wn * 128 + j * 32 + lr < N) {
        const uint32_t cbase = (uint32_t)((row0 * N + wn * 128 + j * 32 + lr) * 4);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const uint32_t roff = (uint32_t)((i * 32 + 8 * (r >> 2) + (r & 3)) * N * 4);
            __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[i][j][r]), ro, cbase + roff, 0, 0);
          }
        }
      }
    }
  }
  if (p.partials != nullptr) {
    // Sum of (acc - y_ref)^2.  The wave's 128 x 128 block of y_ref is staged
    // through LDS (the k-loop's stage buffers are free now) by the buffer
    // unit, 64 rows at a time, so the whole block is in flight at once; each
    // wave copies and reads only its own rows, so no barrier is needed
    // between the copy and the reads.  Rows past M read 0 through the buffer
    // resource (their accumulators are 0 too); columns past N are masked.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // stray prefetches into LDS
    barrier_lds();                                      // every wave is done with the stages
    float* const reg_w[8] = {(float*)sa0, (float*)sa1, (float*)sa2, (float*)sa3,
                             (float*)sb0, (float*)sb1, (float*)sb2, (float*)sb3};
    float* const mine0 = wave == 0 ? reg_w[0] : wave == 1 ? reg_w[2] : wave == 2 ? reg_w[4] : reg_w[6];
    float* const mine1 = wave == 0 ? reg_w[1] : wave == 1 ? reg_w[3] : wave == 2 ? reg_w[5] : reg_w[7];
    const rsrc_t ry = make_rsrc(p.y_ref + m0 * N + n0, ((uint64_t)(M - m0) * N - n0) * 4);
    // DMA q of a phase: rows 2q, 2q+1 of the phase's 64 rows; lane L -> row
    // 2q + L/32, columns 4*(L%32) .. +3 of the wave's 128 columns.
    const uint32_t ybase = (uint32_t)((((int64_t)wm * 128 + (lane >> 5)) * N + wn * 128 + 4 * (lane & 31)) * 4);
    bool col_ok[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) col_ok[j] = n0 + wn * 128 + j * 32 + lr < N;
    double sse = 0.0;
#pragma unroll
    for (int phase = 0; phase < 2; ++phase) {
      if (phase == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads of phase 0 done
#pragma unroll
      for (int q = 0; q < 32; ++q) {
        float* dst = (q < 16 ? mine0 : mine1) + (q & 15) * 256;
        const uint32_t roff = (uint32_t)(((int64_t)phase * 64 + 2 * q) * N * 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ry, (lds_void*)dst, 16, ybase + roff, 0, 0, 0);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * phase + ii;
        double dpart = 0.0;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rho = ii * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);   // row within the phase
            const float yv = (rho < 32 ? mine0 : mine1)[(rho & 31) * 128 + j * 32 + lr];
            float d = acc[i][j][r] - yv;
            d = col_ok[j] ? d : 0.f;
            dpart += (double)d * (double)d;
          }
        }
        sse += dpart;
      }
    }
    sse = wave_sum_f64(sse);
    __shared__ double wsum[NT / 64];
    if (lane == 0) wsum[wave] = sse;
    __syncthreads();
    if (t == 0) p.partials[tm * p.tiles_n + tn] = ((wsum[0] + wsum[1]) + wsum[2]) + wsum[3];
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
  p.y_ref = op.y_ref;
  p.y = op.y;
  p.partials = op.partials;
  p.M = op.M;
  p.N = op.N;
  p.K = op.K;
  p.tiles_m = ceil_div(op.M, BM);
  p.tiles_n = ceil_div(op.N, BN);
  const unsigned blocks = (unsigned)(p.tiles_m * p.tiles_n);
  if (op.qweight == nullptr)
    gemm_kernel<false, false><<<blocks, NT, 0, stream>>>(p, nullptr);
  else if (op.inv_s != nullptr)
    gemm_kernel<true, true><<<blocks, NT, 0, stream>>>(p, op.inv_s);
  else
    gemm_kernel<true, false><<<blocks, NT, 0, stream>>>(p, nullptr);
  return hipGetLastError();
}

}  // namespace awq
