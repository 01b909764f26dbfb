// Int4 / int8 expert FFN as grouped GEMMs on the matrix cores (prefill).
//
// With ~80 tokens per expert (4096 tokens, top-10 of 512) each expert's
// weights are a real dense contraction, so they run on MFMA
// (v_mfma_f32_32x32x16_f16, fp32 accumulate).  Experts are MLX affine int4
// or int8 group-quantised (relationship-to-TurboFieldfare section of the
// Swiftlet pages); SwiGLU and group 64 are this library's readings.
//
// Dequantisation: a 4-bit code word's nibbles i and i+4 (an 8-bit word
// pair's bytes (0,2) and (1,3), which hold inputs i and i+4 of the block)
// become the fp16 pair (1024+q_i, 1024+q_{i+4}) by OR-ing them into 0x6400
// (fp16 1024.0 has a mantissa step of 1, exact for q < 1024), a packed
// subtract gives q exactly, and one packed fma gives s*q + b rounded once to
// fp16 (11-bit significand: |rel err| <= 2^-11).
// bf16 (8-bit significand) rounding of the weights would spend most of the
// 2e-3 output tolerance; fp16 keeps it small.  Activations enter as fp16.
// The k order inside every 8-column block is (0,4,1,5,2,6,3,7) in both
// operands, which the dot product does not see, so no nibble shuffles.
//
// gate/up: item = (bucket chunk of <=128 tokens, 64 intermediate rows); the
// block computes both gate and up for those rows (4 waves x 32 tokens x
// 2 x 64 columns) and writes h = silu(g) * u in fp16.  down: item = (bucket
// chunk, 128 output rows); unweighted outputs per (token, rank) pair go to
// the partial buffer, combined later in rank order.
#include "internal.h"
#include "device.h"

namespace moe {
namespace {

constexpr int kPM = 128;        // tokens per bucket chunk (m-tile)

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float float16_t __attribute__((ext_vector_type(16)));

struct PInst {                  // bucket chunk
  int32_t expert;               // -1 = shared expert
  int32_t start;                // routed: offset into pair_ids; shared: first token
  int32_t n;                    // tokens (1..kPM)
};

struct PrefillArgs {
  PoolView pool;
  const uint8_t* shared_blob;
  int d, I, Ish, Imax, T, k;
  const uint16_t* xh;           // fp16 x [T][d], k order permuted per 8
  const PInst* inst;
  const int32_t* n_routed;
  int n_shared_inst;
  const int32_t* pair_ids;
  uint16_t* hh;                 // fp16 h [T*k + T][Imax], permuted per 8
  float* partial;               // [T*k][d]
  float* shared_out;            // [T][d]
};

// 8 nibbles -> 8 fp16 weights s*q + b, in (0,4,1,5,2,6,3,7) order.
__device__ __forceinline__ uint4 dequant8(uint32_t w, half2_t s2, half2_t b2) {
  const half2_t m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p = ((w >> (4 * i)) & 0x000F000Fu) | 0x64006400u;
    const half2_t q = __builtin_bit_cast(half2_t, p) + m1024;
    o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// 8-bit codes of one 8-input block (words wa = inputs (0,1,4,5), wb =
// inputs (2,3,6,7), a byte each) -> 8 fp16 weights in (0,4,1,5,2,6,3,7) order.
__device__ __forceinline__ uint4 dequant8_b(uint32_t wa, uint32_t wb, half2_t s2, half2_t b2) {
  const half2_t m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const uint32_t w[2] = {wa, wb};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p = ((w[i >> 1] >> (8 * (i & 1))) & 0x00FF00FFu) | 0x64006400u;
    const half2_t q = __builtin_bit_cast(half2_t, p) + m1024;
    o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

__device__ __forceinline__ void resolve_p(const PrefillArgs& a, int ii, bool routed, const uint8_t** blob,
                                          int* Iinst, bool* missing) {
  PInst in = a.inst[ii];
  in.expert = __builtin_amdgcn_readfirstlane(in.expert);
  *missing = false;
  if (routed) {
    const int e = in.expert;
    // uniform across the block: keeps the blob descriptor in scalar registers
    const int slot = __builtin_amdgcn_readfirstlane((e >= 0 && e < a.pool.E) ? a.pool.slot_table[e] : -1);
    *missing = slot < 0;
    *blob = a.pool.slab + (uint64_t)(slot < 0 ? 0 : slot) * a.pool.stride;
    *Iinst = a.I;
  } else {
    *blob = a.shared_blob;
    *Iinst = a.Ish;
  }
}

// Pipeline of both GEMMs (one block = 4 waves, a chunk of <= 128 tokens x
// 128 weight rows, k in steps of 64 = one quantisation group): every wave
// owns 32 weight rows and all 128 tokens (up to four 32x32 MFMA tiles).
// Each step's operands go global -> LDS by the buffer unit itself (LDS DMA,
// no registers), three stages in flight: the activation tile (128 rows x
// 128 B), every wave's codes (lanes 0-31 hold the first 32 k of the step for
// their row, lanes 32-63 the second: one 16-byte piece per lane for 4-bit
// codes, two for 8-bit) and its (scale, bias) words.  A wave dequantises its
// own codes straight into the MFMA B operand, so each weight is dequantised
// once.  The k order inside a step is (lane half, 8-input block, the
// (0,4,1,5,2,6,3,7) order) on both operands.
//
// Synchronisation is explicit: every step issues the same DMAs per wave (six
// for 4-bit codes, seven for 8-bit), waits until at most the next stage's
// are in flight (s_waitcnt vmcnt),
// then meets the other waves at a bare s_barrier.  The DMA destinations are
// passed as opaque LDS addresses, so the compiler adds no waits of its own
// (a __syncthreads fence, or its alias tracking, would wait for every DMA in
// flight and serialise the pipeline); empty asm statements with a memory
// clobber keep it from moving LDS accesses across the wait and barrier.
constexpr int kKS = 64;                         // k per step
constexpr int kStA = kPM * 128;                 // activation tile bytes
constexpr int kStS = 4 * 256;                   // (scale, bias), 256 B per wave
// per code width: 16-byte code DMAs per lane, codes bytes (1 KB per wave per
// DMA), stage bytes and DMA instructions per wave per stage
template <int BITS> constexpr int kCodeDma = BITS / 4;
template <int BITS> constexpr int kStB = 4 * 1024 * kCodeDma<BITS>;
template <int BITS> constexpr int kStage = kStA + kStB<BITS> + kStS;
template <int BITS> constexpr int kDmaPerStage = 5 + kCodeDma<BITS>;

// s_waitcnt vmcnt <= N, lgkmcnt == 0, then s_barrier; no code motion of
// memory accesses across it.
template <int N>
__device__ __forceinline__ void stage_barrier() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (0 << 8));
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// LDS position of the 16-byte piece `cc` (0..7) of activation row r: pieces
// are XOR-swizzled by r mod 8 so the MFMA reads (32 rows, one piece) hit 32
// distinct banks.
__device__ __forceinline__ int a_pos(int r, int cc) { return r * 128 + 16 * (cc ^ (r & 7)); }

// Grouped-GEMM main loop: C steps of 64 along k.
//   S0, S1, S2: the stages, kStage bytes each (distinct arrays, used in a
//                 fixed rotation).
//   rA / a_vo[i]: activation rows; a_vo[i] = byte offset of the row this
//                 lane fetches for DMA i (row 8*(4*wave+i) + lane/8), plus
//                 16 * the swizzled piece.  Rows past the chunk fetch row 0:
//                 MFMA row r of C depends on row r of A only, and those
//                 output rows are never stored.
//   rB: the expert blob; codes_off / sb_off: the matrix's sections in it;
//   rows: the matrix's output rows; row: this lane's weight row.
// MT: live 32-token tiles of the chunk (a template so the inner loop has no
// branches and LDS reads overlap the MFMAs).
template <int MT, int BITS>
__device__ __forceinline__ void gemm_loop(uint8_t* S0, uint8_t* S1, uint8_t* S2, rsrc_t rA, const uint32_t* a_vo,
                                          rsrc_t rB, uint32_t codes_off, uint32_t sb_off, uint32_t rows,
                                          uint32_t row, int C, float16_t* acc) {
  constexpr int ND = kCodeDma<BITS>;            // 16-byte code pieces per lane per step
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // piece (ND h + j) of the step's 2 ND pieces of this lane's row
  uint32_t b_vo[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) b_vo[j] = ((ND * h + j) * rows + row) * 16;
  const uint32_t s_vo = row * 4;
  // Stages past the end read through a zero-size descriptor: no memory
  // traffic, zeros land in a stage nobody reads, and the count stays six.
  const rsrc_t rN = make_rsrc(nullptr, 0);
  // Wave w fetches activation rows 32w..32w+31 (tile w): the waves past the
  // live tiles fetch through the zero-size descriptor as well.
  const bool a_live = wave < MT;
  auto issue = [&](int s, uint8_t* st) {
    const bool live = s < C;
    const rsrc_t ra = (live && a_live) ? rA : rN, rb = live ? rB : rN;
    const uint32_t ao = __builtin_amdgcn_readfirstlane(s * 128);
    const uint32_t co = __builtin_amdgcn_readfirstlane(codes_off + (uint32_t)(2 * ND) * s * rows * 16);
    const uint32_t so = __builtin_amdgcn_readfirstlane(sb_off + (uint32_t)s * rows * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_opaque(st + (4 * wave + i) * 1024), 16, a_vo[i], ao, 0, 0);
#pragma unroll
    for (int j = 0; j < ND; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, lds_opaque(st + kStA + (ND * wave + j) * 1024), 16, b_vo[j], co,
                                               0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, lds_opaque(st + kStA + kStB<BITS> + wave * 256), 4, s_vo, so, 0, 0);
  };
  // One step on stage `st` while stage s+2 refills `nx` (the stage read in
  // the previous step).
  auto step = [&](int s, const uint8_t* st, uint8_t* nx) {
    // stage s landed for this wave (stage s+1 may be in flight) and this
    // wave's reads of the previous stage are done; then the block meets
    stage_barrier<kDmaPerStage<BITS>>();
    issue(s + 2, nx);
    const uint32_t sb = *reinterpret_cast<const uint32_t*>(st + kStA + kStB<BITS> + wave * 256 + 4 * (lane & 31));
    const half2_t s2 = __builtin_bit_cast(half2_t, (sb & 0xFFFFu) * 0x10001u);
    const half2_t b2 = __builtin_bit_cast(half2_t, (sb >> 16) * 0x10001u);
    half8_t bv[4];
    if constexpr (BITS == 4) {
      const uint4 cw = *reinterpret_cast<const uint4*>(st + kStA + wave * 1024 + 16 * lane);
      bv[0] = __builtin_bit_cast(half8_t, dequant8(cw.x, s2, b2));
      bv[1] = __builtin_bit_cast(half8_t, dequant8(cw.y, s2, b2));
      bv[2] = __builtin_bit_cast(half8_t, dequant8(cw.z, s2, b2));
      bv[3] = __builtin_bit_cast(half8_t, dequant8(cw.w, s2, b2));
    } else {
      const uint4 c0 = *reinterpret_cast<const uint4*>(st + kStA + (2 * wave) * 1024 + 16 * lane);
      const uint4 c1 = *reinterpret_cast<const uint4*>(st + kStA + (2 * wave + 1) * 1024 + 16 * lane);
      bv[0] = __builtin_bit_cast(half8_t, dequant8_b(c0.x, c0.y, s2, b2));
      bv[1] = __builtin_bit_cast(half8_t, dequant8_b(c0.z, c0.w, s2, b2));
      bv[2] = __builtin_bit_cast(half8_t, dequant8_b(c1.x, c1.y, s2, b2));
      bv[3] = __builtin_bit_cast(half8_t, dequant8_b(c1.z, c1.w, s2, b2));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      half8_t av[MT];
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        av[mt] = *reinterpret_cast<const half8_t*>(st + a_pos(32 * mt + (lane & 31), 4 * h + j));
#pragma unroll
      for (int mt = 0; mt < MT; ++mt)
        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[mt], bv[j], acc[mt], 0, 0, 0);
    }
  };
  // earlier stores / DMAs of this block are done and every wave is past its
  // last reads of the stages before they refill
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
  issue(0, S0);
  issue(1, S1);
  for (int s = 0; s < C; s += 3) {
    step(s, S0, S2);
    if (s + 1 >= C) break;
    step(s + 1, S1, S0);
    if (s + 2 >= C) break;
    step(s + 2, S2, S1);
  }
  // the (empty) DMAs still in flight land before anyone reuses the stages
  stage_barrier<0>();
}

// The same GEMM for chunks of at most 32 tokens (one m-tile), with more
// steps in flight: a stage holds only the live 32 activation rows (4 KB, one
// 1 KB DMA per wave), the codes and the (scale, bias) words, so the LDS of
// the three full stages takes NS of these and NS - 1 steps are in flight.
// Used for 8-bit codes (batched 80B shape: gate/up 236 -> 219 us, down
// 141 -> 121 us); with 4-bit codes it measured slower than the full-stage
// loop (gate/up 131 -> 193 us at any depth from 3 to 7 stages), not yet
// understood, so 4-bit keeps that loop.
// a_vo_n: this lane's activation offset for row 8 * wave + lane / 8.
template <int BITS> constexpr int kNarrowStage = 4096 + 4096 * kCodeDma<BITS> + 1024;
template <int BITS> constexpr int kNarrowNS = (3 * kStage<BITS>) / kNarrowStage<BITS>;

template <int BITS>
__device__ __forceinline__ void gemm_loop_narrow(uint8_t* SM, rsrc_t rA, uint32_t a_vo_n, rsrc_t rB,
                                                 uint32_t codes_off, uint32_t sb_off, uint32_t rows, uint32_t row,
                                                 int C, float16_t* acc) {
  constexpr int ND = kCodeDma<BITS>;
  constexpr int kA = 4096, kB = 4096 * ND, kSt = kNarrowStage<BITS>, NS = kNarrowNS<BITS>;
  constexpr int kPer = 2 + ND;                  // DMAs per wave per stage
  static_assert(NS >= 3 && NS <= 7 && (NS - 2) * kPer < 64, "stages in flight");
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  uint32_t b_vo[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) b_vo[j] = ((ND * h + j) * rows + row) * 16;
  const uint32_t s_vo = row * 4;
  const rsrc_t rN = make_rsrc(nullptr, 0);
  auto issue = [&](int s) {
    uint8_t* st = SM + (s % NS) * kSt;
    const bool live = s < C;
    const rsrc_t ra = live ? rA : rN, rb = live ? rB : rN;
    const uint32_t ao = __builtin_amdgcn_readfirstlane(s * 128);
    const uint32_t co = __builtin_amdgcn_readfirstlane(codes_off + (uint32_t)(2 * ND) * s * rows * 16);
    const uint32_t so = __builtin_amdgcn_readfirstlane(sb_off + (uint32_t)s * rows * 4);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_opaque(st + wave * 1024), 16, a_vo_n, ao, 0, 0);
#pragma unroll
    for (int j = 0; j < ND; ++j)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, lds_opaque(st + kA + (ND * wave + j) * 1024), 16, b_vo[j], co,
                                               0, 0);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rb, lds_opaque(st + kA + kB + wave * 256), 4, s_vo, so, 0, 0);
  };
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
#pragma unroll
  for (int q = 0; q < NS - 1; ++q)
    if (q < C) issue(q);
  for (int s = 0; s < C; ++s) {
    // stage s landed for this wave (the stages issued after it, at most
    // NS - 2, may still be in flight; no stage past the end is issued) and
    // every wave is done with stage s - 1, which the next issue refills
    const int behind = C - 1 - s < NS - 2 ? C - 1 - s : NS - 2;
    switch (behind) {
      case 0: stage_barrier<0>(); break;
      case 1: stage_barrier<kPer>(); break;
      case 2: stage_barrier<2 * kPer>(); break;
      case 3: stage_barrier<3 * kPer>(); break;
      case 4: stage_barrier<(NS - 2 >= 4 ? 4 : 0) * kPer>(); break;
      default: stage_barrier<(NS - 2 >= 5 ? 5 : 0) * kPer>(); break;
    }
    if (s + NS - 1 < C) issue(s + NS - 1);
    const uint8_t* st = SM + (s % NS) * kSt;
    const uint32_t sb = *reinterpret_cast<const uint32_t*>(st + kA + kB + wave * 256 + 4 * (lane & 31));
    const half2_t s2 = __builtin_bit_cast(half2_t, (sb & 0xFFFFu) * 0x10001u);
    const half2_t b2 = __builtin_bit_cast(half2_t, (sb >> 16) * 0x10001u);
    half8_t bv[4];
    if constexpr (BITS == 4) {
      const uint4 cw = *reinterpret_cast<const uint4*>(st + kA + wave * 1024 + 16 * lane);
      bv[0] = __builtin_bit_cast(half8_t, dequant8(cw.x, s2, b2));
      bv[1] = __builtin_bit_cast(half8_t, dequant8(cw.y, s2, b2));
      bv[2] = __builtin_bit_cast(half8_t, dequant8(cw.z, s2, b2));
      bv[3] = __builtin_bit_cast(half8_t, dequant8(cw.w, s2, b2));
    } else {
      const uint4 c0 = *reinterpret_cast<const uint4*>(st + kA + (2 * wave) * 1024 + 16 * lane);
      const uint4 c1 = *reinterpret_cast<const uint4*>(st + kA + (2 * wave + 1) * 1024 + 16 * lane);
      bv[0] = __builtin_bit_cast(half8_t, dequant8_b(c0.x, c0.y, s2, b2));
      bv[1] = __builtin_bit_cast(half8_t, dequant8_b(c0.z, c0.w, s2, b2));
      bv[2] = __builtin_bit_cast(half8_t, dequant8_b(c1.x, c1.y, s2, b2));
      bv[3] = __builtin_bit_cast(half8_t, dequant8_b(c1.z, c1.w, s2, b2));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const half8_t av = *reinterpret_cast<const half8_t*>(st + a_pos(lane & 31, 4 * h + j));
      acc[0] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv[j], acc[0], 0, 0, 0);
    }
  }
  stage_barrier<0>();
}

template <int BITS>
__device__ __forceinline__ void gemm_tiles(int n_tok, uint8_t* S0, uint8_t* S1, uint8_t* S2, rsrc_t rA,
                                           const uint32_t* a_vo, uint32_t a_vo_n,
                                           rsrc_t rB, uint32_t codes_off, uint32_t sb_off, uint32_t rows,
                                           uint32_t row, int C, float16_t* acc) {
  switch ((n_tok + 31) >> 5) {
    case 1:
      // 8-bit: the narrow stages (measured faster on one-tile chunks); 4-bit
      // stays on the full-stage loop, which measured faster there
      if constexpr (BITS == 8) gemm_loop_narrow<BITS>(S0, rA, a_vo_n, rB, codes_off, sb_off, rows, row, C, acc);
      else gemm_loop<1, BITS>(S0, S1, S2, rA, a_vo, rB, codes_off, sb_off, rows, row, C, acc);
      break;
    case 2: gemm_loop<2, BITS>(S0, S1, S2, rA, a_vo, rB, codes_off, sb_off, rows, row, C, acc); break;
    case 3: gemm_loop<3, BITS>(S0, S1, S2, rA, a_vo, rB, codes_off, sb_off, rows, row, C, acc); break;
    default: gemm_loop<4, BITS>(S0, S1, S2, rA, a_vo, rB, codes_off, sb_off, rows, row, C, acc); break;
  }
}

// Work item L -> (chunk, tile).  Workgroups are handed to the 8 XCDs in
// turn, so workgroups L, L+8, L+16, ... run on one XCD and share its L2; they
// take the tiles of one chunk one after another, so the chunk's activation
// rows come from HBM once instead of once per XCD.  Grids are multiples of 8.
constexpr int kXcd = 8;
__device__ __forceinline__ bool xcd_item(long L, int nch, int nt, int* chunk, int* tile) {
  const long j = L / kXcd;
  *tile = (int)(j % nt);
  *chunk = (int)(kXcd * (j / nt) + L % kXcd);
  return *chunk < nch;
}

template <int BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_gate_up_kernel(PrefillArgs a) {
  // three stages, contiguous (chunks of <= 32 tokens use the space as more, smaller stages)
  __shared__ __attribute__((aligned(16))) uint8_t SM[3 * kStage<BITS>];
  uint8_t* S0 = SM;
  uint8_t* S1 = SM + kStage<BITS>;
  uint8_t* S2 = SM + 2 * kStage<BITS>;
  __shared__ int tok_s[kPM], hrow_s[kPM];
  // up tiles handed to the gate waves after the GEMM, one m-tile at a time;
  // they reuse stage 0 (no DMA is in flight and no wave reads the stages
  // once the GEMM has ended)
  static_assert(sizeof(float) * 2 * 16 * 64 <= kStage<BITS>, "exchange fits a stage");
  float (*xch)[16][64] = reinterpret_cast<float (*)[16][64]>(S0);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nR = __builtin_amdgcn_readfirstlane(*a.n_routed);
  const int ntR = a.I / 64, ntS = a.Ish / 64;
  const int nt = ntR > ntS ? ntR : ntS;
  const int nch = nR + a.n_shared_inst;
  const long Lend = (long)((nch + kXcd - 1) / kXcd) * kXcd * nt;
  const int C = a.d / kKS;
  const rsrc_t rX = make_rsrc(a.xh, (uint32_t)a.T * a.d * 2);
  const int mat = wave >> 1;                    // waves 0,1: gate rows; 2,3: up rows
  const int colb = 32 * (wave & 1);

  for (long wi = blockIdx.x; wi < Lend; wi += gridDim.x) {
    int ii, tile;
    if (!xcd_item(wi, nch, nt, &ii, &tile)) continue;
    const bool routed = ii < nR;
    if (tile >= (routed ? ntR : ntS)) continue;
    const int o0 = tile * 64;
    const uint8_t* blob;
    int Iinst;
    bool missing;
    resolve_p(a, ii, routed, &blob, &Iinst, &missing);
    PInst in = a.inst[ii];
    in.start = __builtin_amdgcn_readfirstlane(in.start);
    in.n = __builtin_amdgcn_readfirstlane(in.n);
    if (tid < kPM) {
      int t = -1, h = -1;
      if (tid < in.n) {
        if (routed) {
          const int p = a.pair_ids[in.start + tid];
          t = p / a.k;
          h = p;
        } else {
          t = in.start + tid;
          h = a.T * a.k + t;
        }
      }
      tok_s[tid] = t;
      hrow_s[tid] = h;
    }
    __syncthreads();
    const BlobLayout L = blob_layout(a.d, Iinst, BITS);
    uint32_t a_vo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * (4 * wave + i) + (lane >> 3);
      const int t = tok_s[r];
      a_vo[i] = (uint32_t)(t >= 0 ? t : 0) * a.d * 2 + 16 * ((lane & 7) ^ (r & 7));
    }
    uint32_t a_vo_n;                            // one-tile chunks: row 8 * wave + lane / 8
    {
      const int r = 8 * wave + (lane >> 3);
      const int t = tok_s[r];
      a_vo_n = (uint32_t)(t >= 0 ? t : 0) * a.d * 2 + 16 * ((lane & 7) ^ (r & 7));
    }
    float16_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
    const uint32_t mc = (uint32_t)(mat ? L.m[1].codes : L.m[0].codes);
    const uint32_t ms = (uint32_t)(mat ? L.m[1].sb : L.m[0].sb);
    gemm_tiles<BITS>(in.n, S0, S1, S2, rX, a_vo, a_vo_n, make_rsrc(blob, (uint32_t)L.bytes), mc, ms, (uint32_t)Iinst,
                     (uint32_t)(o0 + colb + (lane & 31)), C, acc);
    // epilogue: up waves hand their tiles to the gate waves, one m-tile at a time
    const int mt_live = (in.n + 31) >> 5;
    bool ovf = false;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt >= mt_live) break;
      if (mat == 1) {
#pragma unroll
        for (int i = 0; i < 16; ++i) xch[wave & 1][i][lane] = acc[mt][i];
      }
      __syncthreads();
      if (mat == 0) {
        const int o = o0 + colb + (lane & 31);
        const int po = (o & ~7) | (2 * (o & 3) + ((o >> 2) & 1));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * mt + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
          if (r < in.n) {
            const float g = acc[mt][i], u = xch[wave & 1][i][lane];
            const float h = missing ? 0.f : g / (1.0f + expf(-g)) * u;
            ovf |= !(fabsf(h) <= 65504.0f);
            a.hh[(size_t)hrow_s[r] * a.Imax + po] = __builtin_bit_cast(uint16_t, (_Float16)h);
          }
        }
      }
      __syncthreads();
    }
    if (ovf) atomicOr(a.pool.err, 2);
    if (missing && tid == 0) atomicOr(a.pool.err, 1);
  }
}

template <int BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void prefill_down_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t SM[3 * kStage<BITS>];
  uint8_t* S0 = SM;
  uint8_t* S1 = SM + kStage<BITS>;
  uint8_t* S2 = SM + 2 * kStage<BITS>;
  __shared__ int hrow_s[kPM], tok_s[kPM];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nR = __builtin_amdgcn_readfirstlane(*a.n_routed);
  const int nt = a.d / 128;
  const int nch = nR + a.n_shared_inst;
  const long Lend = (long)((nch + kXcd - 1) / kXcd) * kXcd * nt;
  const rsrc_t rH = make_rsrc(a.hh, (uint32_t)(a.T * a.k + a.T) * a.Imax * 2);

  for (long wi = blockIdx.x; wi < Lend; wi += gridDim.x) {
    int ii, tile;
    if (!xcd_item(wi, nch, nt, &ii, &tile)) continue;
    const int n0 = tile * 128;
    const bool routed = ii < nR;
    const uint8_t* blob;
    int Iinst;
    bool missing;
    resolve_p(a, ii, routed, &blob, &Iinst, &missing);
    PInst in = a.inst[ii];
    in.start = __builtin_amdgcn_readfirstlane(in.start);
    in.n = __builtin_amdgcn_readfirstlane(in.n);
    if (tid < kPM) {
      int h = -1, t = -1;
      if (tid < in.n) {
        if (routed) {
          h = a.pair_ids[in.start + tid];
        } else {
          t = in.start + tid;
          h = a.T * a.k + t;
        }
      }
      hrow_s[tid] = h;
      tok_s[tid] = t;
    }
    __syncthreads();
    const BlobLayout L = blob_layout(a.d, Iinst, BITS);
    uint32_t a_vo[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = 8 * (4 * wave + i) + (lane >> 3);
      const int hr = hrow_s[r];
      a_vo[i] = (uint32_t)(hr >= 0 ? hr : 0) * a.Imax * 2 + 16 * ((lane & 7) ^ (r & 7));
    }
    uint32_t a_vo_n;                            // one-tile chunks: row 8 * wave + lane / 8
    {
      const int r = 8 * wave + (lane >> 3);
      const int hr = hrow_s[r];
      a_vo_n = (uint32_t)(hr >= 0 ? hr : 0) * a.Imax * 2 + 16 * ((lane & 7) ^ (r & 7));
    }
    float16_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
    gemm_tiles<BITS>(in.n, S0, S1, S2, rH, a_vo, a_vo_n, make_rsrc(blob, (uint32_t)L.bytes), (uint32_t)L.m[2].codes,
                     (uint32_t)L.m[2].sb, (uint32_t)a.d, (uint32_t)(n0 + 32 * wave + (lane & 31)), Iinst / kKS, acc);
    const int n = n0 + 32 * wave + (lane & 31);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = 32 * mt + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (r < in.n) {
          const float v = missing ? 0.f : acc[mt][i];
          if (routed) a.partial[(size_t)hrow_s[r] * a.d + n] = v;
          else a.shared_out[(size_t)tok_s[r] * a.d + n] = v;
        }
      }
    }
    __syncthreads();
  }
}

// x (bf16) -> fp16 with the k order permuted per 8 columns; flags values
// outside the fp16 range.
__global__ __launch_bounds__(256) void prefill_xprep_kernel(const uint16_t* __restrict__ x, long n8,
                                                            uint16_t* __restrict__ xh, int32_t* err) {
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= n8) return;
  const uint4 v = reinterpret_cast<const uint4*>(x)[id];
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
  float f[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = bf16_lo(w[i]);
    f[2 * i + 1] = bf16_hi(w[i]);
  }
  bool ovf = false;
  uint16_t h[8];
  const int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const float t = f[order[s]];
    ovf |= !(fabsf(t) <= 65504.0f);
    h[s] = __builtin_bit_cast(uint16_t, (_Float16)t);
  }
  uint4 o;
  o.x = h[0] | ((uint32_t)h[1] << 16);
  o.y = h[2] | ((uint32_t)h[3] << 16);
  o.z = h[4] | ((uint32_t)h[5] << 16);
  o.w = h[6] | ((uint32_t)h[7] << 16);
  reinterpret_cast<uint4*>(xh)[id] = o;
  if (ovf) atomicOr(err, 2);
}

// Bucket chunks of up to kPM tokens per expert, in expert order, then the
// shared expert's chunks.  One block.
__global__ __launch_bounds__(1024) void prefill_plan_kernel(const int32_t* __restrict__ offsets, int E, int T,
                                                            PInst* __restrict__ inst, int32_t* __restrict__ n_routed) {
  __shared__ int sums[1024];
  const int tid = threadIdx.x;
  const int c = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
  const int nch = (c + kPM - 1) / kPM;
  sums[tid] = nch;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {
    const int v = tid >= off ? sums[tid - off] : 0;
    __syncthreads();
    sums[tid] += v;
    __syncthreads();
  }
  const int base = sums[tid] - nch;
  for (int q = 0; q < nch; ++q) {
    PInst in;
    in.expert = tid;
    in.start = offsets[tid] + q * kPM;
    in.n = min(kPM, c - q * kPM);
    inst[base + q] = in;
  }
  const int total = sums[1023];
  if (tid == 0) *n_routed = total;
  const int nsh = (T + kPM - 1) / kPM;
  for (int q = tid; q < nsh; q += 1024) {
    PInst in;
    in.expert = -1;
    in.start = q * kPM;
    in.n = min(kPM, T - q * kPM);
    inst[total + q] = in;
  }
}

struct PrefillWs {
  uint16_t* xh; uint16_t* hh; PInst* inst; int32_t* n_routed;
};

bool carve_prefill(Carver& c, int d, int Imax, int T, int k, int E, PrefillWs* w) {
  w->xh = c.take<uint16_t>((size_t)T * d);
  w->hh = c.take<uint16_t>(((size_t)T * k + T) * Imax);
  w->inst = c.take<PInst>((size_t)((long)T * k + E) / 1 + (T + kPM - 1) / kPM + 1);
  w->n_routed = c.take<int32_t>(64);
  return c.ok();
}

}  // namespace

size_t prefill_ws_bytes(int d, int I, int Ish, int T, int k, int E) {
  Carver c(nullptr, (size_t)-1);
  PrefillWs w;
  carve_prefill(c, d, I > Ish ? I : Ish, T, k, E, &w);
  return c.off + 256;
}

int prefill_launch(const FfnArgs& f, void* ws, size_t ws_bytes, hipStream_t s) {
  const int Imax = f.I > f.Ish ? f.I : f.Ish;
  Carver c(ws, ws_bytes);
  PrefillWs w;
  if (!carve_prefill(c, f.d, Imax, f.T, f.k, f.pool.E, &w)) return MOE_ERR_INVALID_ARG;
  if (!f.offsets || !f.pair_ids || !f.partial || !f.shared_out) return MOE_ERR_INVALID_ARG;
  const long n8 = (long)f.T * f.d / 8;
  prefill_xprep_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(f.x, n8, w.xh, f.pool.err);
  MOE_HIP(hipGetLastError());
  prefill_plan_kernel<<<1, 1024, 0, s>>>(f.offsets, f.pool.E, f.T, w.inst, w.n_routed);
  MOE_HIP(hipGetLastError());
  PrefillArgs a{};
  a.pool = f.pool; a.shared_blob = f.shared_blob;
  a.d = f.d; a.I = f.I; a.Ish = f.Ish; a.Imax = Imax; a.T = f.T; a.k = f.k;
  a.xh = w.xh; a.inst = w.inst; a.n_routed = w.n_routed;
  a.n_shared_inst = (f.T + kPM - 1) / kPM;
  a.pair_ids = f.pair_ids;
  a.hh = w.hh; a.partial = f.partial; a.shared_out = f.shared_out;
  // upper bounds on the work items; kernels stride over the device count
  long chunks = ((long)f.T * f.k + kPM - 1) / kPM + f.pool.E + a.n_shared_inst;
  chunks = (chunks + kXcd - 1) / kXcd * kXcd;   // grids stay multiples of 8
  const long gu_items = chunks * (Imax / 64);
  const long dn_items = chunks * (f.d / 128);
  if (f.d % 128 != 0) return MOE_ERR_UNSUPPORTED;
  const int gu_grid = (int)(gu_items < 4096 ? gu_items : 4096);
  const int dn_grid = (int)(dn_items < 4096 ? dn_items : 4096);
  void* args[] = {&a};
  void* gu = f.bits == 8 ? (void*)prefill_gate_up_kernel<8> : (void*)prefill_gate_up_kernel<4>;
  void* dn = f.bits == 8 ? (void*)prefill_down_kernel<8> : (void*)prefill_down_kernel<4>;
  MOE_HIP(hipLaunchKernel(gu, dim3(gu_grid), dim3(256), args, 0, s));
  MOE_HIP(hipLaunchKernel(dn, dim3(dn_grid), dim3(256), args, 0, s));
  return MOE_OK;
}

}  // namespace moe
