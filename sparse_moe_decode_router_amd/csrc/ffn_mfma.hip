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
// become an fp16 pair (c+q_i, c+q_{i+4}) by OR-ing them into the mantissa of
// an fp16 constant c whose mantissa step at that bit position is 1: 0x6400
// (1024.0, step 1) for codes at bits 0.. of each half, 0x5400 (64.0, step
// 1/16) for nibbles at bits 4..7, so a word needs one shift (by 8) rather
// than three.  A packed subtract gives q exactly, and one packed fma gives
// s*q + b rounded once to fp16 (11-bit significand: |rel err| <= 2^-11).
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
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

struct PInst {                  // bucket chunk
  int32_t expert;               // -1 = shared expert
  int32_t start;                // routed: offset into pair_ids; shared: first token
  int32_t n;                    // tokens (1..kPM)
};

struct PrefillArgs {
  PoolView pool;
  const uint8_t* shared_blob;
  int d, I, Ish, Imax, T, k;
  const uint16_t* x;            // bf16 x [T][d] (the streaming kernels convert it themselves)
  const uint16_t* xh;           // fp16 x [T][d], k order permuted per 8
  const PInst* inst;
  const int32_t* n_routed;
  int n_shared_inst;
  const int32_t* pair_ids;
  uint16_t* hh;                 // fp16 h [T*k + T][Imax], permuted per 8
  float* partial;               // [T*k][d]
  float* shared_out;            // [T][d]
};

// The masks and the fp16 constants enter through empty asm statements, so the
// compiler keeps them in registers and forms each (code & mask) | constant as
// one v_and_or_b32 (a VOP3 instruction takes no literal operand here; with
// literals it emits a v_and and a v_or).
struct DqConst {
  uint32_t m4lo, m4hi, m8;        // nibble masks at bits 0.. / 4.. of each half; byte mask
  uint32_t c1024, c64;            // 0x6400 (1024.0), 0x5400 (64.0) in both halves
};
__device__ __forceinline__ DqConst dq_const() {
  DqConst k{0x000F000Fu, 0x00F000F0u, 0x00FF00FFu, 0x64006400u, 0x54005400u};
  asm("" : "+s"(k.m4lo), "+s"(k.m4hi), "+s"(k.m8));
  asm("" : "+v"(k.c1024), "+v"(k.c64));
  return k;
}

// 8 nibbles -> 8 fp16 weights s*q + b, in (0,4,1,5,2,6,3,7) order.
__device__ __forceinline__ uint4 dequant8(uint32_t w, half2_t s2, half2_t b2, const DqConst& k) {
  const half2_t m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const half2_t m64 = {(_Float16)-64.0f, (_Float16)-64.0f};
  const uint32_t w8 = w >> 8;
  const uint32_t p[4] = {(w & k.m4lo) | k.c1024, (w & k.m4hi) | k.c64, (w8 & k.m4lo) | k.c1024,
                         (w8 & k.m4hi) | k.c64};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const half2_t q = __builtin_bit_cast(half2_t, p[i]) + ((i & 1) ? m64 : m1024);
    o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// 8-bit codes of one 8-input block (words wa = inputs (0,1,4,5), wb =
// inputs (2,3,6,7), a byte each) -> 8 fp16 weights in (0,4,1,5,2,6,3,7) order.
__device__ __forceinline__ uint4 dequant8_b(uint32_t wa, uint32_t wb, half2_t s2, half2_t b2, const DqConst& k) {
  const half2_t m1024 = {(_Float16)-1024.0f, (_Float16)-1024.0f};
  const uint32_t w[2] = {wa, wb};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t p = ((w[i >> 1] >> (8 * (i & 1))) & k.m8) | k.c1024;
    const half2_t q = __builtin_bit_cast(half2_t, p) + m1024;
    o[i] = __builtin_bit_cast(uint32_t, __builtin_elementwise_fma(q, s2, b2));
  }
  return make_uint4(o[0], o[1], o[2], o[3]);
}

// h = silu(g) u = g / (1 + e^-g) * u in fp32 (the caller then rounds it to
// fp16), from the hardware's base-2 exponential (v_exp_f32 of -g log2 e) and
// reciprocal (v_rcp_f32), each within about one fp32 ulp: a few ulp in all,
// far below the fp16 rounding of h (2^-11 relative).  Large |g| goes to the
// right limits (e^-g -> inf: h -> 0; e^-g -> 0: h -> g u).  The empty asm
// pins the fp32 value: without it the compiler may fold the last multiply
// into the fp16 conversion (v_fma_mixlo_f16, one rounding straight to fp16)
// in one kernel and not in another, and the two roundings differ for values
// next to an fp16 midpoint (about one h in 10^4); the tiled and streaming
// kernels must agree bit for bit.
__device__ __forceinline__ float swiglu(float g, float u) {
  const float e = __builtin_amdgcn_exp2f(g * -1.44269504088896341f);
  float h = g * __builtin_amdgcn_rcpf(1.0f + e) * u;
  asm volatile("" : "+v"(h));
  return h;
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
// Each step's activation tile (128 rows x 128 B) goes global -> LDS by the
// buffer unit itself (LDS DMA, no registers), three stages in flight; every
// wave's codes (lanes 0-31 hold the first 32 k of the step for their row,
// lanes 32-63 the second: one 16-byte piece per lane for 4-bit codes, two
// for 8-bit) and its (scale, bias) words go straight into registers, a ring
// of three steps beside the stages.  A wave dequantises its own codes into
// the MFMA B operand, so each weight is dequantised once.  The k order
// inside a step is (lane half, 8-input block, the (0,4,1,5,2,6,3,7) order)
// on both operands.  A stage is the activation tile alone (16 KB), so three
// blocks share a CU (3 x 49 KB of LDS, 168 VGPRs a wave): against two blocks
// with 21-25 KB stages, the 4096-token expert FFN went 581-591 -> 547-554 us
// (8-bit 646-667 -> 630-634).
//
// Synchronisation is explicit: every step issues the same loads per wave
// (four DMAs, then the codes and the (scale, bias) word: six for 4-bit
// codes, seven for 8-bit), waits until at most the next step's are in
// flight (s_waitcnt vmcnt),
// then meets the other waves at a bare s_barrier.  The DMA destinations are
// passed as opaque LDS addresses, so the compiler adds no waits of its own
// (a __syncthreads fence, or its alias tracking, would wait for every DMA in
// flight and serialise the pipeline); empty asm statements with a memory
// clobber keep it from moving LDS accesses across the wait and barrier.
constexpr int kKS = 64;                         // k per step
constexpr int kStA = kPM * 128;                 // activation tile bytes
// per code width: 16-byte code loads per lane, stage bytes and loads per
// wave per step (four activation DMAs, the codes, the (scale, bias) word)
template <int BITS> constexpr int kCodeDma = BITS / 4;
template <int BITS> constexpr int kStage = kStA;
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

// LDS position of the 16-byte piece `cc` (0..7) of activation row r (rows
// of 128 B): pieces are XOR-swizzled by a_swz(r) = (r mod 8) ^ bit 3 of r,
// so that an MFMA operand read (one piece of consecutive rows) hits distinct
// banks both in any 8 consecutive rows (one 128-byte bank line) and in any
// 16 (two rows per 256-byte bank line: plain r mod 8 made rows r and r + 8
// collide there).
__device__ __forceinline__ int a_swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__device__ __forceinline__ int a_pos(int r, int cc) { return r * 128 + 16 * (cc ^ a_swz(r)); }

// Grouped-GEMM main loop: C steps of 64 along k.
//   S0, S1, S2: the stages, kStage bytes each (distinct arrays, used in a
//                 fixed rotation).
//   rA / a_vo[i]: activation rows; a_vo[i] = byte offset of the row this
//                 lane fetches for DMA i (row 8*(4*wave+i) + lane/8), plus
//                 16 * the swizzled piece.  Rows past the chunk read from
//                 past the end of the buffer, i.e. zeros: MFMA row r of C
//                 depends on row r of A only, and those output rows are
//                 never stored (zeros rather than a copy of a real row: the
//                 matrix cores draw less power on them).
//   rB: the expert blob; codes_off / sb_off: the matrix's sections in it;
//   rows: the matrix's output rows; row: this lane's weight row.
// MT: live 32-token tiles of the chunk (a template so the inner loop has no
// branches and LDS reads overlap the MFMAs).
template <int BITS>
struct CodeSlot {                               // one step's codes and (scale, bias) word of a lane
  u32x4 c[BITS / 4];
  uint32_t sb;
};

template <int MT, int BITS>
__device__ __forceinline__ void gemm_loop(uint8_t* S0, uint8_t* S1, uint8_t* S2, rsrc_t rA, const uint32_t* a_vo,
                                          rsrc_t rB, uint32_t codes_off, uint32_t sb_off, uint32_t rows,
                                          uint32_t row, int C, float16_t* acc) {
  constexpr int ND = kCodeDma<BITS>;            // 16-byte code pieces per lane per step
  const DqConst dq = dq_const();
  const int tid = threadIdx.x, lane = tid & 63, h = lane >> 5;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  // piece (ND h + j) of the step's 2 ND pieces of this lane's row
  uint32_t b_vo[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) b_vo[j] = ((ND * h + j) * rows + row) * 16;
  const uint32_t s_vo = row * 4;
  // Stages past the end read through a zero-size descriptor: no memory
  // traffic, zeros land in a stage nobody reads, and the count stays the same.
  const rsrc_t rN = make_rsrc(nullptr, 0);
  // Wave w fetches activation rows 32w..32w+31 (tile w): the waves past the
  // live tiles fetch through the zero-size descriptor as well.
  const bool a_live = wave < MT;
  // The codes and (scale, bias) words are the wave's own: they go straight
  // into registers (a ring of three steps, as the stages), counted by the
  // same vmcnt as the activation DMAs.
  auto issue = [&](int s, uint8_t* st, CodeSlot<BITS>& cs) {
    const bool live = s < C;
    const rsrc_t ra = (live && a_live) ? rA : rN, rb = live ? rB : rN;
    const uint32_t ao = __builtin_amdgcn_readfirstlane(s * 128);
    const uint32_t co = __builtin_amdgcn_readfirstlane(codes_off + (uint32_t)(2 * ND) * s * rows * 16);
    const uint32_t so = __builtin_amdgcn_readfirstlane(sb_off + (uint32_t)s * rows * 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(ra, lds_opaque(st + (4 * wave + i) * 1024), 16, a_vo[i], ao, 0, 0);
#pragma unroll
    for (int j = 0; j < ND; ++j) cs.c[j] = __builtin_amdgcn_raw_buffer_load_b128(rb, b_vo[j], co, 0);
    cs.sb = __builtin_amdgcn_raw_buffer_load_b32(rb, s_vo, so, 0);
  };
  // One step on stage `st` with codes `cs` while stage s+2 refills `nx` and
  // `nxs` (the stage and codes used in the previous step).
  auto step = [&](int s, const uint8_t* st, const CodeSlot<BITS>& cs, uint8_t* nx, CodeSlot<BITS>& nxs) {
    // stage s landed for this wave (stage s+1 may be in flight) and this
    // wave's reads of the previous stage are done; then the block meets
    stage_barrier<kDmaPerStage<BITS>>();
    const CodeSlot<BITS> cur = cs;
    issue(s + 2, nx, nxs);
    const half2_t s2 = __builtin_bit_cast(half2_t, (cur.sb & 0xFFFFu) * 0x10001u);
    const half2_t b2 = __builtin_bit_cast(half2_t, (cur.sb >> 16) * 0x10001u);
    half8_t bv[4];
    if constexpr (BITS == 4) {
      const u32x4 cw = cur.c[0];
      bv[0] = __builtin_bit_cast(half8_t, dequant8(cw.x, s2, b2, dq));
      bv[1] = __builtin_bit_cast(half8_t, dequant8(cw.y, s2, b2, dq));
      bv[2] = __builtin_bit_cast(half8_t, dequant8(cw.z, s2, b2, dq));
      bv[3] = __builtin_bit_cast(half8_t, dequant8(cw.w, s2, b2, dq));
    } else {
      const u32x4 c0 = cur.c[0], c1 = cur.c[1];
      bv[0] = __builtin_bit_cast(half8_t, dequant8_b(c0.x, c0.y, s2, b2, dq));
      bv[1] = __builtin_bit_cast(half8_t, dequant8_b(c0.z, c0.w, s2, b2, dq));
      bv[2] = __builtin_bit_cast(half8_t, dequant8_b(c1.x, c1.y, s2, b2, dq));
      bv[3] = __builtin_bit_cast(half8_t, dequant8_b(c1.z, c1.w, s2, b2, dq));
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
  CodeSlot<BITS> r0, r1, r2;
  issue(0, S0, r0);
  issue(1, S1, r1);
  // Whole rounds of three steps, then the last C mod 3 after the loop: exits
  // from inside the round made the compiler give each of the three steps its
  // own copy of the accumulators (up to 192 registers), copied across once a
  // round while the MFMAs writing them drained.
  int s = 0;
  for (; s + 3 <= C; s += 3) {
    step(s, S0, r0, S2, r2);
    step(s + 1, S1, r1, S0, r0);
    step(s + 2, S2, r2, S1, r1);
  }
  if (s < C) step(s, S0, r0, S2, r2);
  if (s + 1 < C) step(s + 1, S1, r1, S0, r0);
  // the (empty) loads still in flight land before anyone reuses the stages
  stage_barrier<0>();
}

// The same GEMM for chunks of at most 32 tokens (one m-tile), with more
// steps in flight: a stage holds only the live 32 activation rows (4 KB, one
// 1 KB DMA per wave), the codes and the (scale, bias) words, so the LDS of
// the three full stages takes NS of these and NS - 1 steps are in flight
// (three stages, two in flight, since a full stage holds only the
// activation tile).  Used for 8-bit codes (batched 80B shape, with five of
// these stages in the larger full stages of before: gate/up 236 -> 219 us,
// down 141 -> 121 us); with 4-bit codes it measured slower than the
// full-stage loop (gate/up 131 -> 193 us at any depth from 3 to 7 stages),
// not yet understood, so 4-bit keeps that loop.
// a_vo_n: this lane's activation offset for row 8 * wave + lane / 8.
template <int BITS> constexpr int kNarrowStage = 4096 + 4096 * kCodeDma<BITS> + 1024;
template <int BITS> constexpr int kNarrowNS = (3 * kStage<BITS>) / kNarrowStage<BITS>;
static_assert(kNarrowNS<8> >= 3, "narrow stages in the LDS of three full stages");

template <int BITS>
__device__ __forceinline__ void gemm_loop_narrow(uint8_t* SM, rsrc_t rA, uint32_t a_vo_n, rsrc_t rB,
                                                 uint32_t codes_off, uint32_t sb_off, uint32_t rows, uint32_t row,
                                                 int C, float16_t* acc) {
  constexpr int ND = kCodeDma<BITS>;
  const DqConst dq = dq_const();
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
      bv[0] = __builtin_bit_cast(half8_t, dequant8(cw.x, s2, b2, dq));
      bv[1] = __builtin_bit_cast(half8_t, dequant8(cw.y, s2, b2, dq));
      bv[2] = __builtin_bit_cast(half8_t, dequant8(cw.z, s2, b2, dq));
      bv[3] = __builtin_bit_cast(half8_t, dequant8(cw.w, s2, b2, dq));
    } else {
      const uint4 c0 = *reinterpret_cast<const uint4*>(st + kA + (2 * wave) * 1024 + 16 * lane);
      const uint4 c1 = *reinterpret_cast<const uint4*>(st + kA + (2 * wave + 1) * 1024 + 16 * lane);
      bv[0] = __builtin_bit_cast(half8_t, dequant8_b(c0.x, c0.y, s2, b2, dq));
      bv[1] = __builtin_bit_cast(half8_t, dequant8_b(c0.z, c0.w, s2, b2, dq));
      bv[2] = __builtin_bit_cast(half8_t, dequant8_b(c1.x, c1.y, s2, b2, dq));
      bv[3] = __builtin_bit_cast(half8_t, dequant8_b(c1.z, c1.w, s2, b2, dq));
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

// three blocks a CU: 168 VGPRs a wave (a few spills, outside the k loop)
template <int BITS>
__global__ __launch_bounds__(256, 3) void prefill_gate_up_kernel(PrefillArgs a) {
  // three stages, contiguous (chunks of <= 32 tokens use the space as more, smaller stages)
  __shared__ __attribute__((aligned(16))) uint8_t SM[3 * kStage<BITS>];
  uint8_t* S0 = SM;
  uint8_t* S1 = SM + kStage<BITS>;
  uint8_t* S2 = SM + 2 * kStage<BITS>;
  __shared__ int tok_s[kPM], hrow_s[kPM];
  // half tiles swapped between gate and up waves after the GEMM, one m-tile
  // at a time; they reuse stage 0 (no DMA is in flight and no wave reads the
  // stages once the GEMM has ended)
  static_assert(sizeof(float) * 2 * 2 * 8 * 64 <= kStage<BITS>, "exchange fits a stage");
  float (*xch)[2][8][64] = reinterpret_cast<float (*)[2][8][64]>(S0);
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nR = __builtin_amdgcn_readfirstlane(*a.n_routed);
  const int ntR = a.I / 64, ntS = a.Ish / 64;
  const int nt = ntR > ntS ? ntR : ntS;
  const int nch = nR + a.n_shared_inst;
  const long Lend = (long)((nch + kXcd - 1) / kXcd) * kXcd * nt;
  const int C = a.d / kKS;
  const uint32_t xbytes = (uint32_t)((uint64_t)a.T * a.d * 2);               // < 4 GiB: prefill_fits
  const rsrc_t rX = make_rsrc(a.xh, xbytes);
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
      a_vo[i] = t >= 0 ? (uint32_t)t * a.d * 2 + 16 * ((lane & 7) ^ a_swz(r)) : xbytes;   // past the end: zeros
    }
    uint32_t a_vo_n;                            // one-tile chunks: row 8 * wave + lane / 8
    {
      const int r = 8 * wave + (lane >> 3);
      const int t = tok_s[r];
      a_vo_n = t >= 0 ? (uint32_t)t * a.d * 2 + 16 * ((lane & 7) ^ a_swz(r)) : xbytes;
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
    // epilogue, one m-tile at a time: a gate wave and the up wave with the same
    // 32 columns swap halves of their tiles through LDS (the gate wave gives
    // rows i = 8..15 of its accumulators, the up wave rows 0..7), then each
    // forms h for the half it kept
    const int mt_live = (in.n + 31) >> 5;
    const int o = o0 + colb + (lane & 31);
    const int po = (o & ~7) | (2 * (o & 3) + ((o >> 2) & 1));
    bool ovf = false;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      if (mt >= mt_live) break;
#pragma unroll
      for (int i = 0; i < 8; ++i) xch[mat][wave & 1][i][lane] = mat ? acc[mt][i] : acc[mt][8 + i];
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int ii = mat ? 8 + i : i;
        const int r = 32 * mt + (ii >> 2) * 8 + (lane >> 5) * 4 + (ii & 3);
        if (r < in.n) {
          const float mine = mat ? acc[mt][8 + i] : acc[mt][i];
          const float other = xch[1 - mat][wave & 1][i][lane];
          const float g = mat ? other : mine, u = mat ? mine : other;
          const float h = missing ? 0.f : swiglu(g, u);
          ovf |= !(fabsf(h) <= 65504.0f);
          a.hh[(size_t)hrow_s[r] * a.Imax + po] = __builtin_bit_cast(uint16_t, (_Float16)h);
        }
      }
      __syncthreads();
    }
    if (ovf) atomicOr(a.pool.err, 2);
    if (missing && tid == 0) atomicOr(a.pool.err, 1);
  }
}

// Output staging of the down kernel: 64 tokens x 128 outputs fp32 a pass,
// rows padded by 4 floats (the two token rows a store instruction writes
// fall in different banks); it fits the stages.
constexpr int kEpLd = 132;
static_assert(64 * kEpLd * 4 <= 3 * kStA, "down output staging in the stages");

template <int BITS>
__global__ __launch_bounds__(256, 3) void prefill_down_kernel(PrefillArgs a) {
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
  const uint32_t hbytes = (uint32_t)(((uint64_t)a.T * a.k + a.T) * a.Imax * 2);   // < 4 GiB: prefill_fits
  const rsrc_t rH = make_rsrc(a.hh, hbytes);

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
      a_vo[i] = hr >= 0 ? (uint32_t)hr * a.Imax * 2 + 16 * ((lane & 7) ^ a_swz(r)) : hbytes;   // past the end: zeros
    }
    uint32_t a_vo_n;                            // one-tile chunks: row 8 * wave + lane / 8
    {
      const int r = 8 * wave + (lane >> 3);
      const int hr = hrow_s[r];
      a_vo_n = hr >= 0 ? (uint32_t)hr * a.Imax * 2 + 16 * ((lane & 7) ^ a_swz(r)) : hbytes;
    }
    float16_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
    gemm_tiles<BITS>(in.n, S0, S1, S2, rH, a_vo, a_vo_n, make_rsrc(blob, (uint32_t)L.bytes), (uint32_t)L.m[2].codes,
                     (uint32_t)L.m[2].sb, (uint32_t)a.d, (uint32_t)(n0 + 32 * wave + (lane & 31)), Iinst / kKS, acc);
    // The outputs go out through LDS (the stages are idle now: every wave
    // is past its last stage read and every DMA has landed) in two passes of
    // 64 tokens, so each thread stores 16-byte pieces of one token's 128
    // outputs, a quarter of the store instructions and address computations
    // of storing the accumulators as they lie (one value a lane).
    float* E = reinterpret_cast<float*>(SM);
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      if (64 * p >= in.n) break;                // block-uniform
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int rl = 32 * h + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);   // token within the pass
          E[rl * kEpLd + 32 * wave + (lane & 31)] = missing ? 0.f : acc[2 * p + h][i];
        }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int q = tid + 256 * u, rl = q >> 5, pc = q & 31;
        const int r = 64 * p + rl;
        if (r < in.n) {
          const float4 v = *reinterpret_cast<const float4*>(&E[rl * kEpLd + 4 * pc]);
          float* dst = routed ? a.partial + (size_t)hrow_s[r] * a.d : a.shared_out + (size_t)tok_s[r] * a.d;
          *reinterpret_cast<float4*>(dst + n0 + 4 * pc) = v;
        }
      }
      __syncthreads();                          // the next pass rewrites E
    }
    __syncthreads();                            // every wave is past this item's hrow_s / tok_s reads
  }
}

// ---------------------------------------------------------------------------
// Streaming grouped GEMMs for buckets of a few tokens (batched decode: 64
// tokens over 512 experts is 1-10 tokens per bucket).  There the weights are
// read once per bucket and the step is bound by how many weight bytes are in
// flight, not by the matrix cores, so the activation side stays put and the
// weights stream:
//   * a chunk holds at most kSC tokens; its activation rows (gate/up: x in
//     fp16, converted from bf16 here; down: the chunk's h rows) sit in LDS for
//     the whole k range, loaded once per work item;
//   * every wave owns 32 weight rows (gate/up: the same 32 rows of both
//     matrices, so SwiGLU happens in registers) and streams their codes and
//     (scale, bias) words straight into registers through the buffer unit,
//     kSP steps of 64 inputs ahead, with no block barrier in the k loop;
//   * the MFMA tiles are the tiled path's (v_mfma_f32_32x32x16_f16, tokens
//     as the 32 rows of A, of which the first n are live; rows past the chunk
//     read a row of zeros kept after the chunk's rows and are never stored:
//     with at most 8 live rows, zeros instead of copies of live rows cut the
//     matrix cores' power, 153-154 -> 145-149 us for the 80B batched expert
//     FFN), with the same dequantised fp16 weights and k order, and h /
//     partial outputs in the same layouts.
// tokens per chunk on the streaming path: its activation rows take (kSC + 1)
// (d + 8) x 2 B of LDS, so 8 lets four gate/up blocks share a CU at d = 2048; measured
// on the 80B batched shape (1.9 tokens per active expert) against 16 and 4:
// expert FFN 146.6 against 151.1 and 149.0 us (8-bit unchanged)
constexpr int kSC = 8;
// steps of codes in flight per wave: 2 measured best on the 80B batched
// shape (expert FFN 157.5 us, 8-bit 220.4) against 1 (160.7, 219.0), 4
// (160.7, 228.7) and 8 (169.9, 241.7)
constexpr int kSP = 2;

// One k step (64 inputs) of a wave's NM matrices: this lane's code pieces and
// its row's (scale, bias) word.
template <int BITS, int NM>
struct SStep {
  u32x4 c[NM][BITS / 4];
  uint32_t sb[NM];
};

// Loads of step s (zeros through the zero-size descriptor past the end).
template <int BITS, int NM>
__device__ __forceinline__ void sstep_load(SStep<BITS, NM>& st, int s, bool live, rsrc_t rB, rsrc_t rN,
                                           const uint32_t (&b_vo)[BITS / 4], uint32_t s_vo,
                                           const uint32_t (&co)[NM], const uint32_t (&so)[NM], uint32_t rows) {
  constexpr int ND = BITS / 4;
  const rsrc_t r = live ? rB : rN;
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const uint32_t cs = __builtin_amdgcn_readfirstlane(co[m] + (uint32_t)(2 * ND) * (uint32_t)s * rows * 16);
    const uint32_t ss = __builtin_amdgcn_readfirstlane(so[m] + (uint32_t)s * rows * 4);
#pragma unroll
    for (int j = 0; j < ND; ++j) st.c[m][j] = __builtin_amdgcn_raw_buffer_load_b128(r, b_vo[j], cs, 0);
    st.sb[m] = __builtin_amdgcn_raw_buffer_load_b32(r, s_vo, ss, 0);
  }
}

// Dequantise step st's matrices and multiply them into acc against the four
// 8-input A pieces of this lane's row (arow: the row's fp16 values at the
// step's first input, k order permuted per 8).
template <int BITS, int NM>
__device__ __forceinline__ void sstep_mma(const SStep<BITS, NM>& st, const uint16_t* arow, int h,
                                          const DqConst& dq, float16_t (&acc)[NM]) {
  half8_t av[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) av[j] = *reinterpret_cast<const half8_t*>(arow + 32 * h + 8 * j);
#pragma unroll
  for (int m = 0; m < NM; ++m) {
    const uint32_t sb = st.sb[m];
    const half2_t s2 = __builtin_bit_cast(half2_t, (sb & 0xFFFFu) * 0x10001u);
    const half2_t b2 = __builtin_bit_cast(half2_t, (sb >> 16) * 0x10001u);
    half8_t bv[4];
    if constexpr (BITS == 4) {
      const u32x4 cw = st.c[m][0];
      bv[0] = __builtin_bit_cast(half8_t, dequant8(cw.x, s2, b2, dq));
      bv[1] = __builtin_bit_cast(half8_t, dequant8(cw.y, s2, b2, dq));
      bv[2] = __builtin_bit_cast(half8_t, dequant8(cw.z, s2, b2, dq));
      bv[3] = __builtin_bit_cast(half8_t, dequant8(cw.w, s2, b2, dq));
    } else {
      const u32x4 c0 = st.c[m][0], c1 = st.c[m][1];
      bv[0] = __builtin_bit_cast(half8_t, dequant8_b(c0.x, c0.y, s2, b2, dq));
      bv[1] = __builtin_bit_cast(half8_t, dequant8_b(c0.z, c0.w, s2, b2, dq));
      bv[2] = __builtin_bit_cast(half8_t, dequant8_b(c1.x, c1.y, s2, b2, dq));
      bv[3] = __builtin_bit_cast(half8_t, dequant8_b(c1.z, c1.w, s2, b2, dq));
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[m] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av[j], bv[j], acc[m], 0, 0, 0);
  }
}

// The k loop of one wave: C steps, a ring of kSP steps in flight.  live:
// whether the wave's 32 rows exist (a tile's last wave may be past the
// matrix); a dead wave loads zeros and its results are not stored.
template <int BITS, int NM>
__device__ __forceinline__ void stream_loop(const uint16_t* arow, rsrc_t rB, bool live, const uint32_t (&co)[NM],
                                            const uint32_t (&so)[NM], uint32_t rows, uint32_t row, int C,
                                            float16_t (&acc)[NM]) {
  constexpr int ND = BITS / 4;
  const int lane = threadIdx.x & 63, h = lane >> 5;
  const DqConst dq = dq_const();
  uint32_t b_vo[ND];
#pragma unroll
  for (int j = 0; j < ND; ++j) b_vo[j] = ((ND * h + j) * rows + row) * 16;
  const uint32_t s_vo = row * 4;
  const rsrc_t rN = make_rsrc(nullptr, 0);
  SStep<BITS, NM> ring[kSP];
#pragma unroll
  for (int p = 0; p < kSP; ++p) sstep_load<BITS, NM>(ring[p], p, live && p < C, rB, rN, b_vo, s_vo, co, so, rows);
  for (int s0 = 0; s0 < C; s0 += kSP) {
#pragma unroll
    for (int p = 0; p < kSP; ++p) {
      const int s = s0 + p;
      if (s < C) {
        const SStep<BITS, NM> cur = ring[p];
        sstep_load<BITS, NM>(ring[p], s + kSP, live && s + kSP < C, rB, rN, b_vo, s_vo, co, so, rows);
        sstep_mma<BITS, NM>(cur, arow + 64 * s, h, dq, acc);
      }
    }
  }
}

// Stage the fp16 rows of a chunk into LDS (row stride ld halfs): gate/up from
// bf16 x (converted, k order permuted per 8, values beyond fp16 range
// flagged), down from the fp16 h rows as they are.  All of a thread's loads
// are issued before its first store.
template <bool FROM_BF16>
__device__ __forceinline__ bool stage_rows(const uint16_t* __restrict__ src, size_t src_ld, const int* rows_s, int n,
                                           int width, uint16_t* dst, int ld) {
  const int npc = width / 8;
  const int total = n * npc;
  bool ovf = false;
  for (int q0 = threadIdx.x; q0 < total; q0 += 4 * 256) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * 256;
      const int qq = q < total ? q : 0;             // clamped: unconditional loads
      v[u] = reinterpret_cast<const uint4*>(src + (size_t)rows_s[qq / npc] * src_ld)[qq % npc];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int q = q0 + u * 256;
      if (q >= total) break;
      uint4 o = v[u];
      if constexpr (FROM_BF16) {
        const uint32_t w[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
        float f[8];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f[2 * i] = bf16_lo(w[i]);
          f[2 * i + 1] = bf16_hi(w[i]);
        }
        const int order[8] = {0, 4, 1, 5, 2, 6, 3, 7};
        uint16_t hv[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          const float x = f[order[t]];
          ovf |= !(fabsf(x) <= 65504.0f);
          hv[t] = __builtin_bit_cast(uint16_t, (_Float16)x);
        }
        o = make_uint4(hv[0] | ((uint32_t)hv[1] << 16), hv[2] | ((uint32_t)hv[3] << 16),
                       hv[4] | ((uint32_t)hv[5] << 16), hv[6] | ((uint32_t)hv[7] << 16));
      }
      *reinterpret_cast<uint4*>(dst + (q / npc) * ld + 8 * (q % npc)) = o;
    }
  }
  return ovf;
}

// gate/up: item = (chunk, 128 intermediate rows); wave w takes rows
// 32 w .. 32 w + 31 of both matrices.  LDS: the chunk's x rows.
template <int BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void stream_gate_up_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t xl[];   // [kSC + 1][d + 8] fp16, the last row zeros
  __shared__ int tok_s[kSC], hrow_s[kSC];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nR = __builtin_amdgcn_readfirstlane(*a.n_routed);
  const int ntR = (a.I + 127) / 128, ntS = (a.Ish + 127) / 128;
  const int nt = ntR > ntS ? ntR : ntS;
  const int nch = nR + a.n_shared_inst;
  const long Lend = (long)((nch + kXcd - 1) / kXcd) * kXcd * nt;
  const int ld = a.d + 8;
  const int C = a.d / kKS;
  for (int c = tid; c < ld / 8; c += 256) reinterpret_cast<uint4*>(xl + kSC * ld)[c] = make_uint4(0, 0, 0, 0);
  for (long wi = blockIdx.x; wi < Lend; wi += gridDim.x) {
    int ii, tile;
    if (!xcd_item(wi, nch, nt, &ii, &tile)) continue;
    const bool routed = ii < nR;
    if (tile >= (routed ? ntR : ntS)) continue;
    const uint8_t* blob;
    int Iinst;
    bool missing;
    resolve_p(a, ii, routed, &blob, &Iinst, &missing);
    PInst in = a.inst[ii];
    in.start = __builtin_amdgcn_readfirstlane(in.start);
    in.n = __builtin_amdgcn_readfirstlane(in.n);
    if (tid < kSC) {
      int t = 0, hr = 0;
      if (tid < in.n) {
        if (routed) {
          const int p = a.pair_ids[in.start + tid];
          t = p / a.k;
          hr = p;
        } else {
          t = in.start + tid;
          hr = a.T * a.k + t;
        }
      }
      tok_s[tid] = t;
      hrow_s[tid] = hr;
    }
    const BlobLayout L = blob_layout(a.d, Iinst, BITS);
    const int o = tile * 128 + 32 * wave + (lane & 31);
    const bool live = !missing && tile * 128 + 32 * wave < Iinst;
    const uint32_t co[2] = {(uint32_t)L.m[0].codes, (uint32_t)L.m[1].codes};
    const uint32_t so[2] = {(uint32_t)L.m[0].sb, (uint32_t)L.m[1].sb};
    __syncthreads();                            // tok_s; and every wave is past the previous item's LDS reads
    bool ovf = stage_rows<true>(a.x, (size_t)a.d, tok_s, in.n, a.d, xl, ld);
    __syncthreads();
    float16_t acc[2];
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[m][i] = 0.f;
    const uint16_t* arow = xl + ((lane & 31) < in.n ? (lane & 31) : kSC) * ld;
    stream_loop<BITS, 2>(arow, make_rsrc(blob, (uint32_t)L.bytes), live, co, so, (uint32_t)Iinst,
                         (uint32_t)(live ? o : 0), C, acc);
    if (live) {
      const int po = (o & ~7) | (2 * (o & 3) + ((o >> 2) & 1));
#pragma unroll
      for (int i = 0; i < 8; ++i) {              // token rows 0..15 of the tile
        const int r = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (r < in.n) {
          const float g = acc[0][i], u = acc[1][i];
          const float hv = swiglu(g, u);
          ovf |= !(fabsf(hv) <= 65504.0f);
          a.hh[(size_t)hrow_s[r] * a.Imax + po] = __builtin_bit_cast(uint16_t, (_Float16)hv);
        }
      }
    } else if (missing && tile * 128 + 32 * wave < Iinst) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        const int po = (o & ~7) | (2 * (o & 3) + ((o >> 2) & 1));
        if (r < in.n) a.hh[(size_t)hrow_s[r] * a.Imax + po] = 0;
      }
    }
    if (ovf) atomicOr(a.pool.err, 2);
    if (missing && tid == 0) atomicOr(a.pool.err, 1);
    // every wave is past this item's reads of tok_s / hrow_s / xl before the
    // next item rewrites them (a block takes several items when the grid is
    // smaller than the work)
    __syncthreads();
  }
}

// down: item = (chunk, 128 output rows); wave w takes rows 32 w .. 32 w + 31.
// LDS: the chunk's h rows.
template <int BITS>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2))) void stream_down_kernel(PrefillArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint16_t hl[];   // [kSC + 1][Imax + 8] fp16, the last row zeros
  __shared__ int hrow_s[kSC], tok_s[kSC];
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int nR = __builtin_amdgcn_readfirstlane(*a.n_routed);
  const int nt = (a.d + 127) / 128;
  const int nch = nR + a.n_shared_inst;
  const long Lend = (long)((nch + kXcd - 1) / kXcd) * kXcd * nt;
  const int ld = a.Imax + 8;
  for (int c = tid; c < ld / 8; c += 256) reinterpret_cast<uint4*>(hl + kSC * ld)[c] = make_uint4(0, 0, 0, 0);
  for (long wi = blockIdx.x; wi < Lend; wi += gridDim.x) {
    int ii, tile;
    if (!xcd_item(wi, nch, nt, &ii, &tile)) continue;
    const bool routed = ii < nR;
    const uint8_t* blob;
    int Iinst;
    bool missing;
    resolve_p(a, ii, routed, &blob, &Iinst, &missing);
    PInst in = a.inst[ii];
    in.start = __builtin_amdgcn_readfirstlane(in.start);
    in.n = __builtin_amdgcn_readfirstlane(in.n);
    if (tid < kSC) {
      int t = 0, hr = 0;
      if (tid < in.n) {
        if (routed) {
          hr = a.pair_ids[in.start + tid];
        } else {
          t = in.start + tid;
          hr = a.T * a.k + t;
        }
      }
      hrow_s[tid] = hr;
      tok_s[tid] = t;
    }
    const BlobLayout L = blob_layout(a.d, Iinst, BITS);
    const int n = tile * 128 + 32 * wave + (lane & 31);
    const bool live = !missing && tile * 128 + 32 * wave < a.d;
    const uint32_t co[1] = {(uint32_t)L.m[2].codes};
    const uint32_t so[1] = {(uint32_t)L.m[2].sb};
    __syncthreads();
    stage_rows<false>(a.hh, (size_t)a.Imax, hrow_s, in.n, Iinst, hl, ld);
    __syncthreads();
    float16_t acc[1];
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[0][i] = 0.f;
    const uint16_t* arow = hl + ((lane & 31) < in.n ? (lane & 31) : kSC) * ld;
    stream_loop<BITS, 1>(arow, make_rsrc(blob, (uint32_t)L.bytes), live, co, so, (uint32_t)a.d,
                         (uint32_t)(live ? n : 0), Iinst / kKS, acc);
    if (tile * 128 + 32 * wave < a.d) {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
        if (r < in.n) {
          const float v = live ? acc[0][i] : 0.f;
          if (routed) a.partial[(size_t)hrow_s[r] * a.d + n] = v;
          else a.shared_out[(size_t)tok_s[r] * a.d + n] = v;
        }
      }
    }
    // every wave is past this item's reads of hrow_s / tok_s / hl before the
    // next item rewrites them
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

// Bucket chunks of up to csz tokens per expert (kPM on the tiled path, kSC
// on the streaming path), in expert order, then the shared expert's chunks.
// One block.
__global__ __launch_bounds__(1024) void prefill_plan_kernel(const int32_t* __restrict__ offsets, int E, int T,
                                                            int csz, PInst* __restrict__ inst,
                                                            int32_t* __restrict__ n_routed) {
  __shared__ int sums[1024];
  const int tid = threadIdx.x;
  const int c = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
  const int nch = (c + csz - 1) / csz;
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
    in.start = offsets[tid] + q * csz;
    in.n = min(csz, c - q * csz);
    inst[base + q] = in;
  }
  const int total = sums[1023];
  if (tid == 0) *n_routed = total;
  const int nsh = (T + csz - 1) / csz;
  for (int q = tid; q < nsh; q += 1024) {
    PInst in;
    in.expert = -1;
    in.start = q * csz;
    in.n = min(csz, T - q * csz);
    inst[total + q] = in;
  }
}

struct PrefillWs {
  uint16_t* xh; uint16_t* hh; PInst* inst; int32_t* n_routed;
};

bool carve_prefill(Carver& c, int d, int Imax, int T, int k, int E, PrefillWs* w) {
  w->xh = c.take<uint16_t>((size_t)T * d);
  w->hh = c.take<uint16_t>(((size_t)T * k + T) * Imax);
  w->inst = c.take<PInst>((size_t)((long)T * k + E) + (T + kSC - 1) / kSC + 1);   // chunks on either path
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

int prefill_launch(const FfnArgs& f, int path, void* ws, size_t ws_bytes, hipStream_t s) {
  const int Imax = f.I > f.Ish ? f.I : f.Ish;
  if (!prefill_fits(f.T, f.d, f.k, Imax)) return MOE_ERR_UNSUPPORTED;
  if (f.d % 128 != 0) return MOE_ERR_UNSUPPORTED;
  Carver c(ws, ws_bytes);
  PrefillWs w;
  if (!carve_prefill(c, f.d, Imax, f.T, f.k, f.pool.E, &w)) return MOE_ERR_INVALID_ARG;
  if (!f.offsets || !f.pair_ids || !f.partial || !f.shared_out) return MOE_ERR_INVALID_ARG;
  // streaming GEMMs for a few tokens per expert (their activation rows stay
  // in LDS: kSC + 1 rows of d fp16 values must fit beside a second block)
  const bool stream_fits = f.d <= 4096;
  if (path == MOE_PATH_PREFILL_STREAM && !stream_fits) return MOE_ERR_UNSUPPORTED;
  const bool stream = path == MOE_PATH_PREFILL_STREAM ||
                      (path == MOE_PATH_PREFILL && stream_fits && (long)f.T * f.k <= 4L * f.pool.E);
  const int csz = stream ? kSC : kPM;
  if (!stream) {
    const long n8 = (long)f.T * f.d / 8;
    prefill_xprep_kernel<<<(unsigned)((n8 + 255) / 256), 256, 0, s>>>(f.x, n8, w.xh, f.pool.err);
    MOE_HIP(hipGetLastError());
  }
  prefill_plan_kernel<<<1, 1024, 0, s>>>(f.offsets, f.pool.E, f.T, csz, w.inst, w.n_routed);
  MOE_HIP(hipGetLastError());
  PrefillArgs a{};
  a.pool = f.pool; a.shared_blob = f.shared_blob;
  a.d = f.d; a.I = f.I; a.Ish = f.Ish; a.Imax = Imax; a.T = f.T; a.k = f.k;
  a.x = f.x; a.xh = w.xh; a.inst = w.inst; a.n_routed = w.n_routed;
  a.n_shared_inst = (f.T + csz - 1) / csz;
  a.pair_ids = f.pair_ids;
  a.hh = w.hh; a.partial = f.partial; a.shared_out = f.shared_out;
  // upper bounds on the work items; kernels stride over the device count
  long chunks = ((long)f.T * f.k + csz - 1) / csz + f.pool.E + a.n_shared_inst;
  chunks = (chunks + kXcd - 1) / kXcd * kXcd;   // grids stay multiples of 8
  void* args[] = {&a};
  if (stream) {
    const long gu_items = chunks * ((Imax + 127) / 128);
    const long dn_items = chunks * (f.d / 128);
    const int gu_grid = (int)(gu_items < 8192 ? gu_items : 8192);
    const int dn_grid = (int)(dn_items < 8192 ? dn_items : 8192);
    void* gu = f.bits == 8 ? (void*)stream_gate_up_kernel<8> : (void*)stream_gate_up_kernel<4>;
    void* dn = f.bits == 8 ? (void*)stream_down_kernel<8> : (void*)stream_down_kernel<4>;
    MOE_HIP(hipLaunchKernel(gu, dim3(gu_grid), dim3(256), args, (size_t)(kSC + 1) * (f.d + 8) * 2, s));
    MOE_HIP(hipLaunchKernel(dn, dim3(dn_grid), dim3(256), args, (size_t)(kSC + 1) * (Imax + 8) * 2, s));
    return MOE_OK;
  }
  const long gu_items = chunks * (Imax / 64);
  const long dn_items = chunks * (f.d / 128);
  const int gu_grid = (int)(gu_items < 4096 ? gu_items : 4096);
  const int dn_grid = (int)(dn_items < 4096 ? dn_items : 4096);
  void* gu = f.bits == 8 ? (void*)prefill_gate_up_kernel<8> : (void*)prefill_gate_up_kernel<4>;
  void* dn = f.bits == 8 ? (void*)prefill_down_kernel<8> : (void*)prefill_down_kernel<4>;
  MOE_HIP(hipLaunchKernel(gu, dim3(gu_grid), dim3(256), args, 0, s));
  MOE_HIP(hipLaunchKernel(dn, dim3(dn_grid), dim3(256), args, 0, s));
  return MOE_OK;
}

}  // namespace moe
