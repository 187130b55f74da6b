// W4A16 contraction Y = X . B^T with the weight operand dequantized on chip
// (builderai AWQ page, "About": kernels for 4-bit weights and 16-bit
// activations; robotsatlas AWQ page, "Implementation pitfalls": a separate
// dequantize-then-GEMM pass loses the benefit), with the squared error
// against the unquantized output fused into the epilogue (robotsatlas "How it
// works": the scale minimises the layer's output error).  The same template
// with a bf16 weight operand computes that unquantized output Y = X . W^T.
//
// gfx950 design
//   * 256x256 output tile per workgroup, BK = 32.  INT4 path: 4 waves in a
//     2x2 grid, each owning 128x128 = 4x4 v_mfma_f32_32x32x16_bf16 blocks
//     (256 fp32 accumulators per lane, held in AGPRs).  bf16 path: 8 waves in
//     a 2x4 grid of 128x64 (two waves per SIMD).
//   * LDS tiles are [row][4 x 16 B chunks] with an XOR swizzle of the chunk
//     index by the row's quad, which keeps ds_read_b128 of the MFMA fragment
//     pattern free of bank conflicts (measured: see chunk_swz).
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
//   * Every product with a bf16 weight operand (the search's sum of squares
//     of X . D^T for a difference operand D, the reference product, the
//     staged W4A16 product, the Gram form's contractions, the candidate SSE
//     against Y_ref) runs mfma16_kernel below: the same tiles, ring and
//     publication, with v_mfma_f32_16x16x32_bf16 instead of 32x32x16.
#include <type_traits>

#include "awq_internal.h"
#include "device_common.h"

namespace awq {

namespace gemm_detail {

constexpr int BM = kGemmBM;
constexpr int BN = kGemmBN;
constexpr int BK = 32;
constexpr int kChunks = BK / 8;             // 16-byte chunks per tile row
constexpr int kSlots = 256 * kChunks;       // 16-byte slots per operand tile (16 KiB)
static_assert(BM == 256 && BN == 256, "mapping assumes 256x256 tiles");

// Wave grid: 2 waves along M (128 rows each) by WN waves along N.  WN = 2:
// 4 waves of 128x128 (one per SIMD); WN = 4: 8 waves of 128x64 (two per
// SIMD, so one wave's waits are covered by the other's MFMAs).
template <int WN>
struct Cfg {
  static constexpr int kWaves = 2 * WN;
  static constexpr int kThreads = 64 * kWaves;
  static constexpr int kTN = 256 / WN;              // wave tile columns
  static constexpr int kBJ = kTN / 32;              // 32x32 blocks along N per wave
  static constexpr int kDma = kSlots / 64 / kWaves; // 1 KiB DMA instructions per wave per tile
  static constexpr int kTPR = kThreads / 256;       // threads per weight row (INT4 dequant)
  static constexpr int kWPT = 4 / kTPR;             // code words per thread per k-step
  static constexpr int kFragReads = 4 + kBJ;        // ds_read_b128 per k16 substep
};
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

// One wave's share of an operand tile: DPW buffer->LDS copies of 1 KiB.
template <int DPW>
__device__ __forceinline__ void dma_tile_wave(rsrc_t r, uint4* dst, const uint32_t (&off)[DPW],
                                              uint32_t soff) {
#pragma unroll
  for (int i = 0; i < DPW; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(dst + 64 * i), 16, off[i], soff, 0, 0);
}

// Copy of 16 bytes per lane from a buffer into LDS at dst + 16 * lane.
__device__ __forceinline__ void dma16(rsrc_t r, float* dst, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)dst, 16, voff, 0, 0, 0);
}

__device__ __forceinline__ uint2 ld8(rsrc_t r, uint32_t voff, uint32_t soff) {
  typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
  const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return make_uint2(v.x, v.y);
}

// Swizzle of a row's chunk index by the row's quad: rows 4j .. 4j+3 share
// one value and quads j, j+1, j+2, j+3 get all four, so the 16 consecutive
// rows that a ds_read_b128 of the MFMA fragment pattern (or a ds_write of
// the dequantized rows) touches at one logical chunk cover all 64 banks once.
// Measured with rocprofv3 (SQ_LDS_BANK_CONFLICT) on the search contraction:
// zero conflict cycles, against 0.6e9 for a swizzle by (row>>1 ^ row>>3) and
// 1.8e9 unswizzled; LDS active cycles halve.
__device__ __forceinline__ int chunk_swz(int row) { return (row >> 2) & 3; }
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * kChunks + (chunk ^ chunk_swz(row));
}

__device__ __forceinline__ void barrier_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// Barrier that waits only for this wave's LDS operations older than its last
// N (LDS operations of a wave complete in order): the last N are fragment
// reads for the next step, which need not land before the barrier.
template <int N>
__device__ __forceinline__ void barrier_lds_keep() {
  if constexpr (N == 8)
    asm volatile("s_waitcnt lgkmcnt(8)\n\ts_barrier" ::: "memory");
  else if constexpr (N == 6)
    asm volatile("s_waitcnt lgkmcnt(6)\n\ts_barrier" ::: "memory");
  else
    asm volatile("s_barrier" ::: "memory");
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

template <int WPT>
struct CodeRegs {
  uint32_t q[WPT];    // this thread's code words of its row for one k-step
  uint32_t step_bits; // raw; converted when used so the load stays in flight
  uint32_t zero;
};

// kStoreY: write the fp32 product; kSse: fp64 sum of (Y - Y_ref)^2 per tile,
// or with kDot the fp64 sum of Y * Y_ref (a quadratic form's last factor).
// kI3: the packed codes in the dense INT3 layout (32 codes of a row in three
// u32 words per k-step), widened to the 4-bit fields the dequantization reads;
// for the same codes Y is the same bit for bit.
template <bool kInt4, bool kInvS, int WN, bool kStoreY, bool kSse, bool kDot = false,
          bool kI3 = false>
__global__ __launch_bounds__(Cfg<WN>::kThreads, 1) void gemm_kernel(Params p,
                                                                    const float* __restrict__ inv_s) {
  // The body exists only in the device pass; the host pass needs just the
  // signature to emit the launch stub.
#if defined(__HIP_DEVICE_COMPILE__)
  using C_ = Cfg<WN>;
  constexpr int NW = C_::kWaves, BJ = C_::kBJ, TN = C_::kTN, DPW = C_::kDma;
  constexpr int TPR = C_::kTPR, WPT = C_::kWPT;
  static_assert(!kI3 || (kInt4 && WPT == 4), "dense INT3: one thread per row, a whole run per k-step");
  // Separate objects per stage: the compiler tracks LDS-DMA writes per object.
  __shared__ uint4 sa0[kSlots], sa1[kSlots], sa2[kSlots], sa3[kSlots];
  __shared__ uint4 sb0[kSlots], sb1[kSlots], sb2[kSlots], sb3[kSlots];
  uint4* const SA[4] = {sa0, sa1, sa2, sa3};
  uint4* const SB[4] = {sb0, sb1, sb2, sb3};

  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / WN, wn = wave % WN;
  const int lr = lane & 31, lk = lane >> 5;

  int64_t tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t M = p.M, N = p.N, K = p.K;
  const int64_t G = K / kGroup;

  // DMA mapping: instruction i of wave w fills slots [(DPW*w+i)*64, +64):
  // lane L -> row 16*(DPW*w+i) + L/4, physical chunk L%4 = logical ^ swizzle.
  uint32_t dma_off[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int row = 16 * (DPW * wave + i) + (lane >> 2);
    const int chunk = (lane & 3) ^ chunk_swz(row);
    dma_off[i] = (uint32_t)(row * K * 2 + chunk * 16);
  }
  const int dma_slot = wave * (DPW * 64);

  const rsrc_t ra = make_rsrc(p.x + m0 * K, (uint64_t)(M - m0) * K * 2);
  rsrc_t rb, rq, rsc, rz;
  if constexpr (kInt4) {
    rq = kI3 ? make_rsrc(p.qweight + n0 * (3 * K / 32), (uint64_t)(N - n0) * (3 * K / 8))
             : make_rsrc(p.qweight + n0 * (K / 8), (uint64_t)(N - n0) * (K / 2));
    rsc = make_rsrc(p.scales + n0 * G, (uint64_t)(N - n0) * G * 4);
    rz = make_rsrc(p.zeros + n0 * G, (uint64_t)(N - n0) * G);
  } else {
    rb = make_rsrc(p.w + n0 * K, (uint64_t)(N - n0) * K * 2);
  }
  // INT4 dequant mapping: thread t owns words [wq0, wq0 + WPT) of row brow.
  const int brow = t / TPR;
  const int wq0 = (t % TPR) * WPT;
  const uint32_t q_off = kI3 ? (uint32_t)(brow * (3 * K / 8))
                             : (uint32_t)(brow * (K / 2) + wq0 * 4);
  const uint32_t sc_off = (uint32_t)(brow * G * 4);
  const uint32_t z_off = (uint32_t)(brow * G);

  auto dma_tile = [&](rsrc_t r, uint4* stage, int64_t k0) {
    dma_tile_wave<DPW>(r, stage + dma_slot, dma_off, (uint32_t)(k0 * 2));
  };
  auto load_codes = [&](CodeRegs<WPT>& C, int64_t k0) {
    if constexpr (kI3) {
      // The k-step's 32 codes of the row: one 12-byte run.
      typedef uint32_t u32x3 __attribute__((ext_vector_type(3)));
      const u32x3 v = __builtin_amdgcn_raw_buffer_load_b96(rq, q_off, (uint32_t)(k0 / 32 * 12), 0);
      C.q[0] = v.x; C.q[1] = v.y; C.q[2] = v.z; C.q[3] = 0u;
    } else if constexpr (WPT == 4) {
      const uint4 v = ld16(rq, q_off, (uint32_t)(k0 / 2));
      C.q[0] = v.x; C.q[1] = v.y; C.q[2] = v.z; C.q[3] = v.w;
    } else {
      const uint2 v = ld8(rq, q_off, (uint32_t)(k0 / 2));
      C.q[0] = v.x; C.q[1] = v.y;
    }
    const uint32_t g = (uint32_t)(k0 / kGroup);
    C.step_bits = __builtin_amdgcn_raw_buffer_load_b32(rsc, sc_off, g * 4, 0);
    C.zero = __builtin_amdgcn_raw_buffer_load_b8(rz, z_off, g, 0);
  };
  // Dequantization of one k-step's codes, one word (8 codes, one 16-byte LDS
  // write) at a time.  pin() is an empty asm that fixes the first use of the
  // loaded registers at the start of the step that dequantizes them;
  // otherwise the scheduler hoists the conversion up to the load and the
  // wait for it drains every later prefetch.
  struct Unpacked {
    uint32_t words[WPT];
    float step, zero;
  };
  auto pin = [&](const CodeRegs<WPT>& C) {
    Unpacked U;
    uint32_t sbits = C.step_bits, zraw = C.zero;
#pragma unroll
    for (int w = 0; w < WPT; ++w) U.words[w] = C.q[w];
    asm volatile("" : "+v"(sbits), "+v"(zraw));
#pragma unroll
    for (int w = 0; w < (kI3 ? 3 : WPT); ++w) asm volatile("" : "+v"(U.words[w]));
    if constexpr (kI3) {
      const uint4 n = nibbles_from_int3(make_uint4(U.words[0], U.words[1], U.words[2], 0u));
      U.words[0] = n.x; U.words[1] = n.y; U.words[2] = n.z; U.words[3] = n.w;
    }
    U.step = __uint_as_float(sbits);
    U.zero = (float)zraw;
    return U;
  };
  auto dequant_word = [&](const Unpacked& U, uint4* stage, int64_t k0, int w) {
    const int c = wq0 + w;   // chunk of the row = code word index within the k-step
    stage[swz(brow, c)] = dequant8<kInvS>(U.words[w], U.step, U.zero,
                                          kInvS ? inv_s + k0 + 8 * c : nullptr);
  };
  // Wait until this wave's DMA into `stage` has landed (the compiler inserts
  // the exact vmcnt for a read of an object with a pending DMA write).
  auto own_dma_done = [&](const uint4* stage) {
    const uint32_t v = *(const uint32_t*)(stage + dma_slot);
    asm volatile("" ::"v"(v));
  };

  f32x16 acc[4][BJ];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < BJ; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.f;

  struct Frags {
    bf16x8 a[4], b[BJ];
  };
  auto read_frags = [&](Frags& F, const uint4* la, const uint4* lb, int s) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      F.a[i] = __builtin_bit_cast(bf16x8, la[swz(wm * 128 + i * 32 + lr, 2 * s + lk)]);
#pragma unroll
    for (int j = 0; j < BJ; ++j)
      F.b[j] = __builtin_bit_cast(bf16x8, lb[swz(wn * TN + j * 32 + lr, 2 * s + lk)]);
  };
  // Half of the wave's blocks (rows i = 2h, 2h+1).
  auto mfma_half = [&](const Frags& F, int h) {
#pragma unroll
    for (int i = 2 * h; i < 2 * h + 2; ++i)
#pragma unroll
      for (int j = 0; j < BJ; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(F.a[i], F.b[j], acc[i][j], 0, 0, 0);
  };

  const int64_t KT = K / BK;   // multiple of 4 (K is a multiple of 128)
  CodeRegs<WPT> C[2];
  Frags F0, F1;

  // Prologue: A(0..2) [and bf16 B(0..2)] in flight; INT4 B(0), B(1)
  // dequantized; stages 0 and 1 published; step 0's first fragments read.
  dma_tile(ra, SA[0], 0);
  dma_tile(ra, SA[1], BK);
  dma_tile(ra, SA[2], 2 * BK);
  if constexpr (kInt4) {
    load_codes(C[0], 0);
    load_codes(C[1], BK);
    {
      const Unpacked U0 = pin(C[0]);
#pragma unroll
      for (int w = 0; w < WPT; ++w) dequant_word(U0, SB[0], 0, w);
      const Unpacked U1 = pin(C[1]);
#pragma unroll
      for (int w = 0; w < WPT; ++w) dequant_word(U1, SB[1], BK, w);
    }
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

  // Interleave MFMAs with other work in the current scheduling region:
  // nm groups of {1 MFMA, v VALU, d DS-read}.
  auto interleave = [&](auto NM, auto V, auto D) {
    constexpr int nm = decltype(NM)::value, v = decltype(V)::value, d = decltype(D)::value;
#pragma unroll
    for (int q = 0; q < nm; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);                          // MFMA
      if constexpr (v > 0) __builtin_amdgcn_sched_group_barrier(0x002, v, 0);   // VALU
      if constexpr (d > 0) __builtin_amdgcn_sched_group_barrier(0x100, d, 0);   // DS read
    }
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using IH = std::integral_constant<int, 2 * BJ>;        // MFMAs per half substep
  using IS = std::integral_constant<int, 4 * BJ>;        // MFMAs per substep
  // VALU per MFMA for the dequant words placed in a region
  using IV1 = std::integral_constant<int, (WPT / 2) * 40 / (4 * BJ)>;
  using IV2 = std::integral_constant<int, (WPT / 2) * 40 / (2 * BJ)>;

  // One k-step.  The loads are issued unconditionally so the compiler's wait
  // counts are exact on every path; the prefetches of the three steps past
  // the end of K are clamped to the last k-step (they fill stages that are
  // never read), which keeps every address inside its row.
  auto step = [&](int64_t k, auto I) {
    constexpr int i = decltype(I)::value;      // k % 4
    const int64_t kpre = min(k + 3, KT - 1) * BK;
    dma_tile(ra, SA[(i + 3) & 3], kpre);
    if constexpr (kInt4) {
      uint4* const bq = SB[(i + 2) & 3];
      const int64_t kq = (k + 2) * BK;
      const Unpacked U = pin(C[i & 1]);      // codes of step k+2
      load_codes(C[(i + 1) & 1], kpre);
      read_frags(F1, SA[i], SB[i], 1);
      mfma_half(F0, 0);
      mfma_half(F0, 1);
#pragma unroll
      for (int w = 0; w < WPT / 2; ++w) dequant_word(U, bq, kq, w);
      interleave(IS{}, IV1{}, I0{});
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F1, 0);
#pragma unroll
      for (int w = WPT / 2; w < WPT; ++w) dequant_word(U, bq, kq, w);
      own_dma_done(SA[(i + 2) & 3]);
      interleave(IH{}, IV2{}, I0{});
      // Every LDS write and DMA-completion read of this step is issued above;
      // the fragment reads below are the wave's youngest LDS operations.
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F1, 1);
      read_frags(F0, SA[(i + 1) & 3], SB[(i + 1) & 3], 0);
      interleave(IH{}, I0{}, I1{});
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds_keep<C_::kFragReads>();
    } else {
      dma_tile(rb, SB[(i + 3) & 3], kpre);
      read_frags(F1, SA[i], SB[i], 1);
      mfma_half(F0, 0);
      mfma_half(F0, 1);
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F1, 0);
      // This wave's copies into stage k+2 were issued one step ago; only this
      // step's 2 x DPW copies may still be in flight.  (An explicit count: a
      // dummy LDS read of the stage would also wait for every LDS read.)
      static_assert(DPW == 2, "the count below assumes 2 copies per operand per step");
      asm volatile("s_waitcnt vmcnt(4)");
      __builtin_amdgcn_sched_barrier(0);
      mfma_half(F1, 1);
      read_frags(F0, SA[(i + 1) & 3], SB[(i + 1) & 3], 0);
      interleave(IH{}, I0{}, I1{});
      __builtin_amdgcn_sched_barrier(0);
      barrier_lds_keep<0>();
    }
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
  if constexpr (kStoreY) {
    // Rows past M fall outside the buffer resource and are dropped.
    const rsrc_t ro = make_rsrc(p.y + m0 * N + n0, ((uint64_t)(M - m0) * N - n0) * 4);
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      if (n0 + wn * TN + j * 32 + lr < N) {
        const uint32_t cbase = (uint32_t)((row0 * N + wn * TN + j * 32 + lr) * 4);
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
  if constexpr (kSse) {
    // Sum of (acc - y_ref)^2.  The wave's 128 x TN block of y_ref is staged
    // through LDS (the k-loop's stage buffers are free now) by the buffer
    // unit, 64 rows at a time, so a whole half-block is in flight at once;
    // each wave copies and reads only its own rows, so no barrier is needed
    // between the copy and the reads.  Rows past M read 0 through the buffer
    // resource (their accumulators are 0 too); columns past N are masked.
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");   // stray prefetches into LDS
    barrier_lds();                                      // every wave is done with the stages
    // The wave's 16 KiB (8 waves) or 2 x 16 KiB (4 waves) of LDS for a phase.
    constexpr int kArrs = 8 / NW;
    auto arr = [&](int a) -> float* {
      switch (a & 7) {
        case 0: return (float*)sa0;
        case 1: return (float*)sa1;
        case 2: return (float*)sa2;
        case 3: return (float*)sa3;
        case 4: return (float*)sb0;
        case 5: return (float*)sb1;
        case 6: return (float*)sb2;
        default: return (float*)sb3;
      }
    };
    float* const mine0 = arr(wave * kArrs);
    float* const mine1 = arr(wave * kArrs + kArrs - 1);
    constexpr int kRowsPerArr = 16384 / 4 / TN;         // rows of a wave's block per array
    constexpr int kLanesPerRow = TN / 4;                // 16-byte pieces per row
    constexpr int kRowsPerDma = 64 / kLanesPerRow;
    constexpr int kDmaPerPhase = 64 / kRowsPerDma;
    const rsrc_t ry = make_rsrc(p.y_ref + m0 * N + n0, ((uint64_t)(M - m0) * N - n0) * 4);
    const uint32_t ybase = (uint32_t)((((int64_t)wm * 128 + lane / kLanesPerRow) * N + wn * TN +
                                       4 * (lane % kLanesPerRow)) * 4);
    bool col_ok[BJ];
#pragma unroll
    for (int j = 0; j < BJ; ++j) col_ok[j] = n0 + wn * TN + j * 32 + lr < N;
    double sse = 0.0;
#pragma unroll
    for (int phase = 0; phase < 2; ++phase) {
      if (phase == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // reads of phase 0 done
#pragma unroll
      for (int q = 0; q < kDmaPerPhase; ++q) {
        const int rr = q * kRowsPerDma;                   // first row of this DMA within the phase
        float* dst = (rr < kRowsPerArr ? mine0 : mine1) + (rr % kRowsPerArr) * TN;
        const uint32_t roff = (uint32_t)(((int64_t)phase * 64 + rr) * N * 4);
        dma16(ry, dst, ybase + roff);
      }
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
      for (int ii = 0; ii < 2; ++ii) {
        const int i = 2 * phase + ii;
        double dpart = 0.0;
#pragma unroll
        for (int j = 0; j < BJ; ++j) {
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int rho = ii * 32 + 8 * (r >> 2) + 4 * lk + (r & 3);   // row within the phase
            const float yv = (rho < kRowsPerArr ? mine0 : mine1)[(rho % kRowsPerArr) * TN + j * 32 + lr];
            if constexpr (kDot) {
              const double prod = (double)acc[i][j][r] * (double)yv;   // exact
              dpart += col_ok[j] ? prod : 0.0;
            } else {
              float d = acc[i][j][r] - yv;
              d = col_ok[j] ? d : 0.f;
              dpart += (double)d * (double)d;
            }
          }
        }
        sse += dpart;
      }
    }
    sse = wave_sum_f64(sse);
    __shared__ double wsum[NW];
    if (lane == 0) wsum[wave] = sse;
    __syncthreads();
    if (t == 0) {
      double tot = 0.0;
#pragma unroll
      for (int w = 0; w < NW; ++w) tot += wsum[w];
      p.partials[tm * p.tiles_n + tn] = tot;
    }
  }
#endif  // __HIP_DEVICE_COMPILE__
}

// Epilogues of mfma16_kernel beside the optional fp32 store of Y.
enum Epilogue { kEpiNone = 0, kEpiSq = 1, kEpiSse = 2, kEpiDot = 3 };

// The contractions with a bf16 weight operand, Y = X . B^T per 256x256 tile
// (B: the search's difference operand D, so Y is the candidate's output
// error itself, robotsatlas AWQ page, "How it works": the scale minimises the
// layer's output error; or W, a staged dequantized operand, a Gram factor).
// kStoreY writes fp32 Y; kEpi adds per tile the fp64 sum of Y^2 (kEpiSq), of
// (Y - Y_ref)^2 (kEpiSse) or of Y * Y_ref (kEpiDot) to a partial slot.  Same
// tiles, XCD-aware order, LDS layout, DMA ring and publication two k-steps
// ahead as gemm_kernel, but on v_mfma_f32_16x16x32_bf16: per k-step one k32
// substep of 8 A and 4 B fragments per wave (128x64) and 32 MFMAs.  Under the chip's power limit
// the 16x16x32 form sustains more flops than 32x32x16 on random operands
// (measured with operands in registers: 78% against 74% of the 2.5 PFLOP/s
// spec; zero operands reach 91% and 98%); on the search's operands this
// kernel is 4-5% faster than gemm_kernel's 32x32x16 form.  The accumulators
// (128 per lane) stay in VGPRs; the next step's fragments are read into the
// registers each row block frees right after its MFMAs, so two fragment sets
// never coexist in full (230-236 VGPRs, two waves per SIMD, no spills).
template <bool kStoreY, int kEpi>
__global__ __launch_bounds__(512, 1) void mfma16_kernel(Params p) {
#if defined(__HIP_DEVICE_COMPILE__)
  constexpr int WN = 4, NW = 8, DPW = Cfg<WN>::kDma;
  static_assert(DPW == 2, "the vmcnt below assumes 2 copies per operand per step");
  __shared__ uint4 sa0[kSlots], sa1[kSlots], sa2[kSlots], sa3[kSlots];
  __shared__ uint4 sb0[kSlots], sb1[kSlots], sb2[kSlots], sb3[kSlots];
  uint4* const SA[4] = {sa0, sa1, sa2, sa3};
  uint4* const SB[4] = {sb0, sb1, sb2, sb3};
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int wave = t >> 6;
  const int wm = wave / WN, wn = wave % WN;
  // 16x16x32 operand layout: lane l holds row (l & 15) of a 16-row block and
  // k = 8 (l >> 4) .. 8 (l >> 4) + 7 of the k32 step, i.e. logical chunk l >> 4.
  const int l16 = lane & 15, lq = lane >> 4;

  int64_t tm, tn;
  tile_coords(blockIdx.x, p.tiles_m, p.tiles_n, tm, tn);
  const int64_t m0 = tm * BM, n0 = tn * BN;
  const int64_t M = p.M, N = p.N, K = p.K;
  uint32_t dma_off[DPW];
#pragma unroll
  for (int i = 0; i < DPW; ++i) {
    const int row = 16 * (DPW * wave + i) + (lane >> 2);
    const int chunk = (lane & 3) ^ chunk_swz(row);
    dma_off[i] = (uint32_t)(row * K * 2 + chunk * 16);
  }
  const int dma_slot = wave * (DPW * 64);
  // Rows past M / N read as zero, so their products add nothing.
  const rsrc_t ra = make_rsrc(p.x + m0 * K, (uint64_t)(M - m0) * K * 2);
  const rsrc_t rb = make_rsrc(p.w + n0 * K, (uint64_t)(N - n0) * K * 2);
  auto dma_tile = [&](rsrc_t r, uint4* stage, int64_t k0) {
    dma_tile_wave<DPW>(r, stage + dma_slot, dma_off, (uint32_t)(k0 * 2));
  };
  auto own_dma_done = [&](const uint4* stage) {
    const uint32_t v = *(const uint32_t*)(stage + dma_slot);
    asm volatile("" ::"v"(v));
  };

  f32x4 acc[8][4];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
  struct Frags {
    bf16x8 a[8], b[4];
  };
  auto read_a = [&](const uint4* la, int r) {
    return __builtin_bit_cast(bf16x8, la[swz(wm * 128 + r * 16 + l16, lq)]);
  };
  auto read_b = [&](const uint4* lb, int j) {
    return __builtin_bit_cast(bf16x8, lb[swz(wn * 64 + j * 16 + l16, lq)]);
  };
  auto mfma_block = [&](const Frags& F, int r) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
      acc[r][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(F.a[r], F.b[j], acc[r][j], 0, 0, 0);
  };

  const int64_t KT = K / BK;   // multiple of 4 (K is a multiple of 128)
  Frags Fr[2];
  // Prologue: stages 0..2 in flight, 0 and 1 published, step 0's fragments read.
  dma_tile(ra, SA[0], 0);
  dma_tile(ra, SA[1], BK);
  dma_tile(ra, SA[2], 2 * BK);
  dma_tile(rb, SB[0], 0);
  dma_tile(rb, SB[1], BK);
  dma_tile(rb, SB[2], 2 * BK);
  own_dma_done(SB[0]);
  own_dma_done(SB[1]);
  own_dma_done(SA[0]);
  own_dma_done(SA[1]);
  barrier_lds();
#pragma unroll
  for (int j = 0; j < 4; ++j) Fr[0].b[j] = read_b(SB[0], j);
#pragma unroll
  for (int r = 0; r < 8; ++r) Fr[0].a[r] = read_a(SA[0], r);

  // One k-step: the copies of step k+3 are issued (clamped to the last step
  // past the end, into stages never read); the next step's fragments come
  // from stage k+1, published at the end of step k-1: its B fragments first,
  // then A row block r right after the MFMAs of row block r.  Before the
  // barrier each wave waits for its own copies into stage k+2 (issued one
  // step ago; only this step's 2 x DPW may still be in flight).
  auto step = [&](int64_t k, auto I) {
    constexpr int i = decltype(I)::value;      // k % 4
    const int64_t kpre = min(k + 3, KT - 1) * BK;
    dma_tile(ra, SA[(i + 3) & 3], kpre);
    dma_tile(rb, SB[(i + 3) & 3], kpre);
    Frags& Fc = Fr[i & 1];
    Frags& Fn = Fr[(i + 1) & 1];
    const uint4* la = SA[(i + 1) & 3];
    const uint4* lb = SB[(i + 1) & 3];
#pragma unroll
    for (int j = 0; j < 4; ++j) Fn.b[j] = read_b(lb, j);
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      mfma_block(Fc, r);
      Fn.a[r] = read_a(la, r);
    }
    __builtin_amdgcn_sched_group_barrier(0x100, 4, 0);     // DS reads: the B fragments
#pragma unroll
    for (int q = 0; q < 8; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);   // MFMA: one row block
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);   // DS read: its next A fragment
    }
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_waitcnt vmcnt(4)");
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
  };
  for (int64_t k = 0; k < KT; k += 4) {
    step(k, std::integral_constant<int, 0>{});
    step(k + 1, std::integral_constant<int, 1>{});
    step(k + 2, std::integral_constant<int, 2>{});
    step(k + 3, std::integral_constant<int, 3>{});
  }

  // Lane holds column l16 of each 16x16 block (r, j) and its rows 4*lq + e,
  // e = 0..3: tile row wm*128 + 16r + 4lq + e, tile column wn*64 + 16j + l16.
  // Rows past M fall outside the buffer resources (stores dropped, Y_ref
  // reads 0; their accumulators are 0); columns past N are masked.
  const uint32_t lane_off = (uint32_t)(((int64_t)(wm * 128 + 4 * lq) * N + wn * 64 + l16) * 4);
  if constexpr (kStoreY) {
    // The wave's 128 x 64 block goes out through LDS, 64 rows at a time, so
    // that each store writes 4 whole rows of 256 bytes (one 16-byte piece per
    // lane) instead of 4 x 64 scattered bytes.  The k-loop's stage arrays are
    // free once every wave has passed the barrier and the prefetches past the
    // last step have landed; each wave then uses one 16 KiB array of its own.
    // Inside a row the 16-column block index is XOR-ed with the row's quad
    // ((row >> 2) & 3), so the fragment-order writes hit 64 distinct banks.
    asm volatile("s_waitcnt vmcnt(0) lgkmcnt(0)" ::: "memory");
    __syncthreads();
    float* lw;
    switch (wave) {                       // a switch keeps every pointer in LDS space
      case 0: lw = (float*)sa0; break;
      case 1: lw = (float*)sa1; break;
      case 2: lw = (float*)sa2; break;
      case 3: lw = (float*)sa3; break;
      case 4: lw = (float*)sb0; break;
      case 5: lw = (float*)sb1; break;
      case 6: lw = (float*)sb2; break;
      default: lw = (float*)sb3; break;
    }
    const rsrc_t ro = make_rsrc(p.y + m0 * N + n0, ((uint64_t)(M - m0) * N - n0) * 4);
    const int pc = lane & 15, pr = lane >> 4;             // piece column, row in a group of 4
    const int64_t col = wn * 64 + 4 * pc;                 // within the tile
#pragma unroll
    for (int ph = 0; ph < 2; ++ph) {
      if (ph == 1) asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");   // phase 0's reads done
#pragma unroll
      for (int rr = 0; rr < 4; ++rr)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int row = 16 * rr + 4 * lq + e;         // within the phase
            lw[row * 64 + 16 * (j ^ lq) + l16] = acc[4 * ph + rr][j][e];
          }
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int row = 4 * q + pr;
        const float4 v = *(const float4*)&lw[row * 64 + 16 * ((pc >> 2) ^ ((row >> 2) & 3)) +
                                             4 * (pc & 3)];
        const uint32_t off =
            (uint32_t)((((int64_t)wm * 128 + 64 * ph + row) * N + col) * 4);
        if (n0 + col + 3 < N) {
          __builtin_amdgcn_raw_buffer_store_b128(
              u32x4{__float_as_uint(v.x), __float_as_uint(v.y), __float_as_uint(v.z),
                    __float_as_uint(v.w)}, ro, off, 0, 0);
        } else {
          const float vs[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (n0 + col + i < N)
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(vs[i]), ro, off + 4 * i, 0, 0);
        }
      }
    }
  }
  if constexpr (kEpi == kEpiNone) return;
  // fp64 sums: each square and each product of two fp32 values is exact.
  double sse = 0.0;
  if constexpr (kEpi == kEpiSq) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = n0 + wn * 64 + j * 16 + l16 < N;
      double dpart = 0.0;
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const double a = (double)acc[r][j][e];
          dpart = fma(a, a, dpart);
        }
      sse += ok ? dpart : 0.0;
    }
  } else {
    const rsrc_t ry = make_rsrc(p.y_ref + m0 * N + n0, ((uint64_t)(M - m0) * N - n0) * 4);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const bool ok = n0 + wn * 64 + j * 16 + l16 < N;
      float yv[8][4];
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          yv[r][e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
              ry, lane_off + (uint32_t)(((int64_t)(16 * r + e) * N + 16 * j) * 4), 0, 0));
      double dpart = 0.0;
#pragma unroll
      for (int r = 0; r < 8; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (kEpi == kEpiDot) {
            dpart = fma((double)acc[r][j][e], (double)yv[r][e], dpart);
          } else {
            const double d = (double)(acc[r][j][e] - yv[r][e]);
            dpart = fma(d, d, dpart);
          }
        }
      sse += ok ? dpart : 0.0;
    }
  }
  sse = wave_sum_f64(sse);
  __shared__ double wsq[NW];
  if (lane == 0) wsq[wave] = sse;
  __syncthreads();
  if (t == 0) {
    double tot = 0.0;
#pragma unroll
    for (int w = 0; w < NW; ++w) tot += wsq[w];
    p.partials[tm * p.tiles_n + tn] = tot;
  }
#endif  // __HIP_DEVICE_COMPILE__
}

}  // namespace gemm_detail

using namespace gemm_detail;

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
  // bf16 operand: 8 waves (two per SIMD) measured faster; INT4: the dequant
  // VALU work favours 4 waves with 128x128 tiles each.
  const bool y = op.y != nullptr, sse = op.partials != nullptr;
  constexpr unsigned kThreads16 = 512;
  if (op.qweight == nullptr && op.sq) {
    mfma16_kernel<false, kEpiSq><<<blocks, kThreads16, 0, stream>>>(p);
  } else if (op.qweight == nullptr && op.dot) {
    mfma16_kernel<false, kEpiDot><<<blocks, kThreads16, 0, stream>>>(p);
  } else if (op.qweight == nullptr) {
    if (y && sse)
      mfma16_kernel<true, kEpiSse><<<blocks, kThreads16, 0, stream>>>(p);
    else if (sse)
      mfma16_kernel<false, kEpiSse><<<blocks, kThreads16, 0, stream>>>(p);
    else
      mfma16_kernel<true, kEpiNone><<<blocks, kThreads16, 0, stream>>>(p);
  } else {
    auto go = [&](auto kInv, auto kI3c) {
      constexpr bool inv = decltype(kInv)::value, i3 = decltype(kI3c)::value;
      const float* is = inv ? op.inv_s : nullptr;
      if (y && sse)
        gemm_kernel<true, inv, 2, true, true, false, i3><<<blocks, Cfg<2>::kThreads, 0, stream>>>(p, is);
      else if (sse)
        gemm_kernel<true, inv, 2, false, true, false, i3><<<blocks, Cfg<2>::kThreads, 0, stream>>>(p, is);
      else
        gemm_kernel<true, inv, 2, true, false, false, i3><<<blocks, Cfg<2>::kThreads, 0, stream>>>(p, is);
    };
    if (op.inv_s != nullptr && op.int3_dense)
      go(std::true_type{}, std::true_type{});
    else if (op.inv_s != nullptr)
      go(std::true_type{}, std::false_type{});
    else if (op.int3_dense)
      go(std::false_type{}, std::true_type{});
    else
      go(std::false_type{}, std::false_type{});
  }
  return hipGetLastError();
}

}  // namespace awq
