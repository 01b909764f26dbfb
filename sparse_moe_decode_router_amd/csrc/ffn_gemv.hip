// Int4 / int8 expert FFN as GEMVs (decode and batched decode).
//
// Experts are MLX affine int4 or int8 group-quantised (relationship-to-
// TurboFieldfare section of the Swiftlet pages), fetched from the slot pool
// through the slot table with 64-bit offsets; the SwiGLU form and group 64
// are this library's readings.  With W = s*q + b per group of 64 inputs, a
// group's dot product is  s * sum(q x) + b * sum(x).  The kernels form
// sum((c + q) x) with v_dot2c_f32_bf16 on bf16 pairs built by OR-ing nibbles
// into a bf16 constant, and fold the offset c into the bias term:
//     group = s * sum((c+q) x) + (b - c s) * sum(x).
//   4-bit: nibble q into 0x4300 (128.0, mantissa step 1) -> 128 + q, c = 128;
//   8-bit: low nibble into 0x4300 -> 128 + lo, high nibble into 0x4500
//          (2048.0, mantissa step 16) -> 2048 + 16 hi; both products go to
//          the same sums, so c = 2176 and q = lo + 16 hi.
// Products of bf16 values are exact in fp32; accumulation is fp32.
//
// gate/up: one work item = (instance, 8 rows).  Lane (row r, group g) loads
// the 2 x 16 B codes of its group for gate and up (8 rows x 8 groups per
// wave-load = eight 128 B segments), activations come from LDS, partial sums
// meet through a 3-step butterfly and LDS.  h = silu(g) * u is stored as bf16
// (hi, lo) pairs in the (x[8m+i], x[8m+i+4]) order plus per-8 sums, ready
// for the down GEMV.
// down (decode): one block = 8 output rows for every instance of every token,
// so the weighted combine sum_r w_r o_r + s o_shared runs in rank order in
// the block (no float atomics; bit-reproducible, independent of placement).
// down (batched): one work item = (instance, 32 rows), unweighted outputs
// written per (token, rank) pair for moe_combine.
#include "internal.h"
#include "device.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kTC = 4;          // tokens per batched instance
constexpr int kXPad = 36;       // LDS dwords per 32-dword group (bank spread)

struct Inst {                   // batched instance
  int32_t expert;               // -1 = shared expert
  int32_t start;                // routed: offset into pair_ids; shared: first token
  int32_t n;                    // tokens (1..kTC)
};

// Workgroups go to the 8 XCDs in turn (b, b+8, ... share one XCD and its
// L2).  With a grid that is a multiple of 8, workgroup b takes work index
// (b % 8) * (G / 8) + b / 8: each XCD walks a contiguous range, so rows that
// share a cache line (e.g. the (scale, bias) words of 32 consecutive rows)
// are fetched into one L2 once instead of once per XCD.
__device__ __forceinline__ int xcd_remap(int b, int G) {
  return (G & 7) ? b : (b & 7) * (G >> 3) + (b >> 3);
}

struct GateUpArgs {
  PoolView pool;
  const uint8_t* shared_blob;
  int d, I, Ish, Imax, T, k;
  int32_t* idx;                 // decode: [T*k] (input, or output when routing here)
  float* w;                     // decode: [T*k] output when routing here
  float* sgate;                 // decode: [T] output when routing here
  const float* logits;          // decode: [T][E+1] -> route in-kernel
  const float* bias;            // [E] or null
  uint32_t* usage;              // [E] or null
  int32_t* sel_slot;            // decode: [T*k] slot of each selection, for the down pass
  const uint32_t* xq;           // [T][d/2]
  const float* xs;              // [T][d/64]
  const uint16_t* x;            // [T][d] bf16 (the f32-expert kernels read it as is)
  const Inst* inst;             // batched: instances
  const int32_t* n_routed;      // batched: device count of routed instances
  int n_shared_inst;            // batched
  const int32_t* pair_ids;
  uint32_t* hq;                 // [hrows][Imax]: hi pairs then lo pairs
  float* hs8;                   // [hrows][Imax/8]
  int batched;
  // decode in two phases (expert streaming): phase 1 computes the resident
  // selections and defers the missing ones (pend[i] = their slot then, -1 =
  // deferred); phase 2, after the refill, computes only the deferred ones
  int phase;                    // 0: one pass
  int32_t* pend;                // [T*k]
};

// Resolve instance -> (blob, I, tokens, hrows).  Returns ntok (0 = skip).
template <int TC>
__device__ __forceinline__ int resolve(const GateUpArgs& a, bool routed, int i, const uint8_t** blob,
                                       int* Iinst, int (&tok)[TC], int (&hrow)[TC], bool* missing) {
  *missing = false;
  if (!a.batched) {
    if (routed) {
      const int e = a.idx[i];
      const int slot = (e >= 0 && e < a.pool.E) ? a.pool.slot_table[e] : -1;
      *missing = slot < 0;
      *blob = a.pool.slab + (uint64_t)(slot < 0 ? 0 : slot) * a.pool.stride;
      *Iinst = a.I;
      tok[0] = i / a.k;
      hrow[0] = i;
    } else {
      *blob = a.shared_blob;
      *Iinst = a.Ish;
      tok[0] = i;
      hrow[0] = a.T * a.k + i;
    }
    return 1;
  }
  // instances hold at most TC tokens; entries past in.n repeat the first
  // (every index constant, so tok and hrow stay in registers)
  const Inst in = a.inst[routed ? i : *a.n_routed + i];
  if (routed) {
    const int e = in.expert;
    const int slot = (e >= 0 && e < a.pool.E) ? a.pool.slot_table[e] : -1;
    *missing = slot < 0;
    *blob = a.pool.slab + (uint64_t)(slot < 0 ? 0 : slot) * a.pool.stride;
    *Iinst = a.I;
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      const int p = a.pair_ids[in.start + (j < in.n ? j : 0)];
      tok[j] = p / a.k;
      hrow[j] = p;
    }
  } else {
    *blob = a.shared_blob;
    *Iinst = a.Ish;
#pragma unroll
    for (int j = 0; j < TC; ++j) {
      tok[j] = in.start + (j < in.n ? j : 0);
      hrow[j] = a.T * a.k + tok[j];
    }
  }
  return in.n < TC ? in.n : TC;
}

// Decode gate/up: GPL groups of 64 inputs per lane (32 group lanes per row):
// 1 for d <= 2048, 2 for d <= 4096, 4 for d <= 8192.

// Code words of one 64-input group held as NP 16-byte pieces (4-bit: 2
// pieces, word m = inputs 8m..8m+7, nibble i = input 8m+i; 8-bit: 4 pieces,
// words 2m and 2m+1 = inputs (0,1,4,5) and (2,3,6,7) of block m, a byte
// each).
template <int NP>
__device__ __forceinline__ uint32_t qword(const uint4 (&q)[NP], int i) {
  const uint4 v = q[i >> 2];
  return (i & 3) == 0 ? v.x : (i & 3) == 1 ? v.y : (i & 3) == 2 ? v.z : v.w;
}

// Product u of 8-input block m as a bf16 pair (c + q terms), to be taken
// against x pair qx<BITS>(u) of the block, i.e. (x[8m+p], x[8m+p+4]).
//   4-bit: u = 0..3, nibbles u and u+4 of word m, pair p = u.
//   8-bit: u = 0..7, pair p = u/2: its inputs are bytes (0,2) (p even) or
//          (1,3) (p odd) of word 2m + p/2; u even takes their low nibbles
//          (128 + lo), u odd their high nibbles (2048 + 16 hi).
// The nibble mask and the two bf16 constants, held in registers (the mask in
// an SGPR, the constants in VGPRs) so that each (shifted word & mask) |
// constant is one v_and_or_b32: a VOP3 instruction takes no literal operand
// here, and with literals the compiler emits a v_and and a v_or.
struct QConst {
  uint32_t mask, mag, mag8;       // 0x000F000F; 0x4300 (128.0) and 0x4500 (2048.0) in both halves
};
__device__ __forceinline__ QConst q_const() {
  QConst k{0x000F000Fu, 0x43004300u, 0x45004500u};
  asm("" : "+s"(k.mask));
  asm("" : "+v"(k.mag), "+v"(k.mag8));
  return k;
}

template <int BITS, int NP>
__device__ __forceinline__ uint32_t qpair(const uint4 (&q)[NP], int m, int u, const QConst& k) {
  static_assert(NP >= BITS / 2, "code pieces");
  const uint32_t w = qword(q, (BITS / 4) * m + (u >> 2));
  const uint32_t mag = (BITS == 8 && (u & 1)) ? k.mag8 : k.mag;
  return ((w >> (4 * (u & 3))) & k.mask) | mag;
}
template <int BITS> __device__ __forceinline__ constexpr int qx(int u) { return BITS == 4 ? u : u >> 1; }
// The same from the group's code words: word index of product u of block m,
// and the pair from that word.
template <int BITS> __device__ __forceinline__ constexpr int qwi(int m, int u) { return (BITS / 4) * m + (u >> 2); }
template <int BITS>
__device__ __forceinline__ uint32_t qpw(uint32_t w, int u, const QConst& k) {
  const uint32_t mag = (BITS == 8 && (u & 1)) ? k.mag8 : k.mag;
  return ((w >> (4 * (u & 3))) & k.mask) | mag;
}
template <int BITS> __device__ __forceinline__ constexpr float qoff() { return BITS == 4 ? 128.0f : 2176.0f; }

// Activation pairs of ntok (<= TC) tokens into the LDS tile [TC][G][kXPad]
// by a 256-thread block: the pieces of all TC tokens are loaded before any is
// stored, so they are in flight together (a plain strided loop waits for
// each load before it issues the next).  Tokens past ntok load token 0's
// piece again and drop it (unconditional loads keep v in registers).
template <int TC>
__device__ __forceinline__ void stage_x(const uint32_t* __restrict__ xq, const int (&tok)[TC], int ntok, int d,
                                        uint32_t* xlds) {
  const int per = d / 8;
  for (int c4 = threadIdx.x; c4 < per; c4 += 256) {
    uint4 v[TC];
#pragma unroll
    for (int tt = 0; tt < TC; ++tt) {
      const int tk = tt < ntok ? tok[tt] : tok[0];
      v[tt] = reinterpret_cast<const uint4*>(xq + (size_t)tk * (d / 2))[c4];
    }
#pragma unroll
    for (int tt = 0; tt < TC; ++tt)
      *reinterpret_cast<uint4*>(&xlds[((tt < ntok ? tt : 0) * (d / 64) + (c4 >> 3)) * kXPad + 4 * (c4 & 7)]) = v[tt];
  }
}

// The same LDS tile from bf16 x itself: piece c4 (x[8 c4 .. 8 c4 + 7]) goes
// in as the pairs (x[i], x[i+4]) the GEMVs read, i = 0..3.
template <int TC>
__device__ __forceinline__ void stage_x_raw(const uint16_t* __restrict__ x, const int (&tok)[TC], int ntok, int d,
                                            uint32_t* xlds) {
  const int per = d / 8;
  for (int c4 = threadIdx.x; c4 < per; c4 += 256) {
    uint4 v[TC];
#pragma unroll
    for (int tt = 0; tt < TC; ++tt) {
      const int tk = tt < ntok ? tok[tt] : tok[0];
      v[tt] = reinterpret_cast<const uint4*>(x + (size_t)tk * d)[c4];
    }
#pragma unroll
    for (int tt = 0; tt < TC; ++tt) {
      uint4 p;
      p.x = (v[tt].x & 0xFFFFu) | (v[tt].z << 16);
      p.y = (v[tt].x >> 16) | (v[tt].z & 0xFFFF0000u);
      p.z = (v[tt].y & 0xFFFFu) | (v[tt].w << 16);
      p.w = (v[tt].y >> 16) | (v[tt].w & 0xFFFF0000u);
      *reinterpret_cast<uint4*>(&xlds[((tt < ntok ? tt : 0) * (d / 64) + (c4 >> 3)) * kXPad + 4 * (c4 & 7)]) = p;
    }
  }
}

// h of 8 consecutive intermediate rows (one 8-block m = rb) as bf16 (hi, lo)
// pairs (h[8m+i], h[8m+i+4]) plus the sum of hi + lo, for the down pass.
__device__ __forceinline__ void write_h8(const float* h, uint32_t* hq, float* hs8, int Imax, int hrow, int rb) {
  uint32_t hi[4], lo[4];
  float s8 = 0.f;
#pragma unroll
  for (int ii = 0; ii < 4; ++ii) {
    const uint32_t a0 = f32_to_bf16(h[ii]), a1 = f32_to_bf16(h[ii + 4]);
    const float r0 = h[ii] - __uint_as_float(a0 << 16);
    const float r1 = h[ii + 4] - __uint_as_float(a1 << 16);
    const uint32_t b0 = f32_to_bf16(r0), b1 = f32_to_bf16(r1);
    hi[ii] = a0 | (a1 << 16);
    lo[ii] = b0 | (b1 << 16);
  }
#pragma unroll
  for (int ii = 0; ii < 8; ++ii) {
    const int p = ii & 3;
    const float hv = ii < 4 ? __uint_as_float(hi[p] << 16) + __uint_as_float(lo[p] << 16)
                            : __uint_as_float(hi[p] & 0xFFFF0000u) + __uint_as_float(lo[p] & 0xFFFF0000u);
    s8 += hv;
  }
  uint32_t* dst = hq + (size_t)hrow * Imax;
  *reinterpret_cast<uint4*>(dst + 4 * rb) = make_uint4(hi[0], hi[1], hi[2], hi[3]);
  *reinterpret_cast<uint4*>(dst + Imax / 2 + 4 * rb) = make_uint4(lo[0], lo[1], lo[2], lo[3]);
  hs8[(size_t)hrow * (Imax / 8) + rb] = s8;
}

// Decode blocks of routed instances select their expert in-kernel: the
// token's logits (+ bias) and the slot table are staged in LDS, wave 0 runs
// the top-k, and the block of (rank 0, rows 0..7) publishes the token's
// indices, weights, shared gate and usage.  This trades a redundant ~1k-cycle
// selection per block for the dependent global loads of a separate top-k.
// RAW (routing given, no prepared activations): the block forms the bf16
// pairs from x and the group sums in the order the router's preparation
// uses, so the results are the same bits; the in-kernel selection is absent.
template <int TC, int NK, int GPL, int BITS, bool RAW>
__global__ __launch_bounds__(256) void gate_up_kernel(GateUpArgs a) {
  constexpr int kNP = BITS / 2;                 // 16-byte code pieces per group
  extern __shared__ uint32_t xlds[];            // [TC][G][kXPad] | routing area
  static_assert(TC * 8 <= 64, "the SwiGLU rows of all tokens sit in wave 0");
  __shared__ float red[4][2][TC][8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // lane = (row r, group lane): the 8 lanes of one row are consecutive so the
  // row's partial sums meet by DPP within groups of 8
  const int r = (tid >> 3) & 7, cpl = (tid & 7) + 8 * (tid >> 6);   // cpl: 0..31
  const int G = a.d / 64;
  const int rbR = a.I / 8, rbS = a.Ish / 8;
  const int nR = a.batched ? *a.n_routed : a.T * a.k;
  const int nS = a.batched ? a.n_shared_inst : a.T;
  const int items = nR * rbR + nS * rbS;
  const int E = a.pool.E;
  // routing area (decode): scratch | slots | sel_l | sel_e
  uint32_t* tscr = xlds + TC * G * kXPad;                          // topk scratch
  int32_t* rslot = reinterpret_cast<int32_t*>(tscr + topk_scratch_words(E));   // [E] slot table
  float* sel_l = reinterpret_cast<float*>(rslot + E);            // [k]
  int32_t* sel_e = reinterpret_cast<int32_t*>(sel_l + a.k);      // [k]

  for (int item = xcd_remap(blockIdx.x, gridDim.x); item < items; item += gridDim.x) {
    const bool routed = item < nR * rbR;
    const int rel = routed ? item : item - nR * rbR;
    const int rb_per = routed ? rbR : rbS;
    const int i = rel / rb_per, rb = rel % rb_per;
    if (a.phase == 2 && (!routed || a.pend[i] >= 0)) continue;   // done in phase 1
    const uint8_t* blob;
    int Iinst, tok[TC], hrow[TC];
    bool missing = false;
    int ntok;
    if (!RAW && !a.batched && routed && a.logits) {
      const int t = i / a.k, rank = i % a.k;
      const float* lrow = a.logits + (size_t)t * (E + 1);
      if (wave != 0) {
        // the slot table goes to LDS through waves 1-3 (E <= 1024: at most
        // six entries per thread, all loads in flight at once) while wave 0
        // selects
        constexpr int kSP = (1024 + 191) / 192;
        int32_t sv[kSP];
#pragma unroll
        for (int u = 0; u < kSP; ++u) {
          const int q = tid - 64 + 192 * u;
          sv[u] = a.pool.slot_table[q < E ? q : 0];     // clamped: loads stay unconditional
        }
#pragma unroll
        for (int u = 0; u < kSP; ++u) {
          const int q = tid - 64 + 192 * u;
          rslot[q < E ? q : 0] = sv[u];
        }
      }
      if (wave == 0) {
        // the logits (+ bias) go from memory straight into wave 0's registers
        topk_select<NK>(lrow, a.bias, E, a.k, sel_l, sel_e, tscr);
        if (rank == 0 && rb == 0) {
          topk_finish(sel_l, sel_e, a.k, a.idx + (size_t)t * a.k, a.w + (size_t)t * a.k, a.usage);
          if (lane == 0) a.sgate[t] = sigmoidf_(lrow[E]);
        }
      }
      __syncthreads();
      const int e = sel_e[rank];
      const int slot = rslot[e];
      missing = slot < 0;
      blob = a.pool.slab + (uint64_t)(missing ? 0 : slot) * a.pool.stride;
      Iinst = a.I;
      tok[0] = t;
      hrow[0] = i;
      ntok = 1;
      if (rb == 0 && tid == 0) a.sel_slot[i] = slot;
    } else {
      ntok = resolve(a, routed, i, &blob, &Iinst, tok, hrow, &missing);
      if (!a.batched && routed && rb == 0 && tid == 0) {
        const int32_t sl = missing ? -1 : (int32_t)((blob - a.pool.slab) / a.pool.stride);
        a.sel_slot[i] = sl;
        if (a.phase == 1) a.pend[i] = sl;
      }
      if (a.phase == 1 && missing) continue;    // deferred: its blob is still on the way
    }
    const BlobLayout L = blob_layout(a.d, Iinst, BITS);
    const int o0 = rb * 8;

    // 1. weight loads first: all of this lane's codes and (scale, bias) words
    uint4 cg[GPL][kNP], cu[GPL][kNP];
    uint32_t sbg[GPL], sbu[GPL];
    float sxv[GPL][TC];                       // group sums of x, loaded up front
#pragma unroll
    for (int gi = 0; gi < GPL; ++gi) {
      const int g = cpl + 32 * gi;
#pragma unroll
      for (int tt = 0; tt < TC; ++tt)
        sxv[gi][tt] = (!RAW && g < G && tt < ntok) ? a.xs[(size_t)tok[tt] * G + g] : 0.f;
    }
    if (!missing) {
      const uint64_t o = (uint64_t)(o0 + r);
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = cpl + 32 * gi;
        if (g < G) {
          const uint64_t c0 = ((uint64_t)(kNP * g) * Iinst + o) * 16;
#pragma unroll
          for (int p = 0; p < kNP; ++p) {
            const uint64_t c = c0 + (uint64_t)p * Iinst * 16;
            cg[gi][p] = *reinterpret_cast<const uint4*>(blob + L.m[0].codes + c);
            cu[gi][p] = *reinterpret_cast<const uint4*>(blob + L.m[1].codes + c);
          }
          sbg[gi] = *reinterpret_cast<const uint32_t*>(blob + L.m[0].sb + ((uint64_t)g * Iinst + o) * 4);
          sbu[gi] = *reinterpret_cast<const uint32_t*>(blob + L.m[1].sb + ((uint64_t)g * Iinst + o) * 4);
        }
      }
    }
    // 2. stage activations (bf16 pairs) while the weights are in flight
    if constexpr (RAW) stage_x_raw<TC>(a.x, tok, ntok, a.d, xlds);
    else stage_x<TC>(a.xq, tok, ntok, a.d, xlds);
    __syncthreads();

    float vg[TC], vu[TC];
#pragma unroll
    for (int tt = 0; tt < TC; ++tt) { vg[tt] = 0.f; vu[tt] = 0.f; }
    const QConst qk = q_const();
    if (!missing) {
#pragma unroll
      for (int gi = 0; gi < GPL; ++gi) {
        const int g = cpl + 32 * gi;
        if (g >= G) continue;
        const float sg = f16_to_f32(sbg[gi]), bg = f16_to_f32(sbg[gi] >> 16);
        const float su = f16_to_f32(sbu[gi]), bu = f16_to_f32(sbu[gi] >> 16);
#pragma unroll
        for (int tt = 0; tt < TC; ++tt) {
          if (tt < ntok) {
            const uint32_t* xp = &xlds[(tt * G + g) * kXPad];
            float sxl = 0.f;                  // RAW: the group sum
            float ag0 = 0.f, au0 = 0.f, ag1 = 0.f, au1 = 0.f;   // two chains each
#pragma unroll
            for (int m = 0; m < 8; ++m) {
              const uint4 xv = *reinterpret_cast<const uint4*>(xp + 4 * m);
              const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
              if constexpr (RAW) {            // x[8m .. 8m+7] in column order
                sxl += bf16_lo(xv.x); sxl += bf16_lo(xv.y); sxl += bf16_lo(xv.z); sxl += bf16_lo(xv.w);
                sxl += bf16_hi(xv.x); sxl += bf16_hi(xv.y); sxl += bf16_hi(xv.z); sxl += bf16_hi(xv.w);
              }
#pragma unroll
              for (int s2 = 0; s2 < BITS / 2; ++s2) {     // products u = 2 s2 and 2 s2 + 1
                const int u0 = 2 * s2, u1 = 2 * s2 + 1;
                ag0 = dot2_bf16(qpair<BITS>(cg[gi], m, u0, qk), xw[qx<BITS>(u0)], ag0);
                au0 = dot2_bf16(qpair<BITS>(cu[gi], m, u0, qk), xw[qx<BITS>(u0)], au0);
                ag1 = dot2_bf16(qpair<BITS>(cg[gi], m, u1, qk), xw[qx<BITS>(u1)], ag1);
                au1 = dot2_bf16(qpair<BITS>(cu[gi], m, u1, qk), xw[qx<BITS>(u1)], au1);
              }
            }
            const float ag = ag0 + ag1, au = au0 + au1;
            const float sx = RAW ? sxl : sxv[gi][tt];
            // explicit roundings: every instance of this kernel (with or
            // without in-kernel selection, RAW or not) does the same arithmetic
            const float cg = __fmaf_rn(-qoff<BITS>(), sg, bg), cu = __fmaf_rn(-qoff<BITS>(), su, bu);
            vg[tt] = __fmaf_rn(sg, ag, __fmaf_rn(cg, sx, vg[tt]));
            vu[tt] = __fmaf_rn(su, au, __fmaf_rn(cu, sx, vu[tt]));
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < TC; ++tt) {
      const float x1 = sum8_dpp(vg[tt]), x2 = sum8_dpp(vu[tt]);
      if ((lane & 7) == 0) { red[wave][0][tt][r] = x1; red[wave][1][tt][r] = x2; }
    }
    __syncthreads();
    if (tid < TC * 8) {                       // lanes 8 tt + rr of wave 0: one row each
      const int tt = tid / 8, rr = tid % 8;
      const float g = ((red[0][0][tt][rr] + red[1][0][tt][rr]) + red[2][0][tt][rr]) + red[3][0][tt][rr];
      const float u = ((red[0][1][tt][rr] + red[1][1][tt][rr]) + red[2][1][tt][rr]) + red[3][1][tt][rr];
      const float hv = missing ? 0.0f : g / (1.0f + expf(-g)) * u;
      float h[8];
#pragma unroll
      for (int q = 0; q < 8; ++q) h[q] = __shfl(hv, 8 * tt + q, 64);
      if (rr == 0 && tt < ntok) write_h8(h, a.hq, a.hs8, a.Imax, hrow[tt], rb);
    }
    if (missing && tid == 0) atomicOr(a.pool.err, 1);
    __syncthreads();
  }
}

// Batched gate/up: item = (bucket chunk of <= kTC tokens, 32 rows).  Each
// wave computes one 8-row sub-block on its own (8 rows x 8 group lanes, GPL
// groups per lane; rows meet by DPP without block barriers); its codes are
// all in flight before the chunk's activations are staged in LDS.
template <int GPL, int BITS>
__global__ __launch_bounds__(256, (GPL <= 4 && BITS == 4) ? 3 : 1) void gate_up_batched_kernel(GateUpArgs a) {
  constexpr int kNP = BITS / 2;                 // 16-byte code pieces per group
  extern __shared__ uint32_t xlds[];            // [kTC][G][kXPad] | xs [kTC][G] | hbuf [4][kTC][8]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane >> 3, gl = lane & 7;
  const int G = a.d / 64;
  float* xsl = reinterpret_cast<float*>(xlds + kTC * G * kXPad);
  float* hbuf = xsl + kTC * G + wave * kTC * 8;
  const int nbR = a.I / 32, nbS = a.Ish / 32;   // items of 32 rows
  const int nR = *a.n_routed;
  const int items = nR * nbR + a.n_shared_inst * nbS;
  const QConst qk = q_const();
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const bool routed = item < nR * nbR;
    const int rel = routed ? item : item - nR * nbR;
    const int nb = routed ? nbR : nbS;
    const int i = rel / nb, ob = rel % nb;
    const uint8_t* blob;
    int Iinst, tok[kTC], hrow[kTC];
    bool missing;
    const int ntok = resolve(a, routed, i, &blob, &Iinst, tok, hrow, &missing);
    const BlobLayout L = blob_layout(a.d, Iinst, BITS);
    // 1. the codes of both of this wave's 8-row sub-blocks, all in flight
    //    before the activations are staged
    constexpr int kSub = 1;                     // sub-blocks per wave (4 per item / 4 waves)
    uint4 cg[kSub][GPL][kNP], cu[kSub][GPL][kNP];
    uint32_t sbg[kSub][GPL], sbu[kSub][GPL];
    if (!missing) {
#pragma unroll
      for (int it = 0; it < kSub; ++it) {
        const uint64_t o = (uint64_t)((ob * 4 + wave + 4 * it) * 8 + r);
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = gl + 8 * gi;
          if (g < G) {
#pragma unroll
            for (int p = 0; p < kNP; ++p) {
              const uint64_t c = ((uint64_t)(kNP * g + p) * Iinst + o) * 16;
              cg[it][gi][p] = *reinterpret_cast<const uint4*>(blob + L.m[0].codes + c);
              cu[it][gi][p] = *reinterpret_cast<const uint4*>(blob + L.m[1].codes + c);
            }
            sbg[it][gi] = *reinterpret_cast<const uint32_t*>(blob + L.m[0].sb + ((uint64_t)g * Iinst + o) * 4);
            sbu[it][gi] = *reinterpret_cast<const uint32_t*>(blob + L.m[1].sb + ((uint64_t)g * Iinst + o) * 4);
          }
        }
      }
    }
    // 2. activations (bf16 pairs) and group sums of the chunk's tokens
    stage_x<kTC>(a.xq, tok, ntok, a.d, xlds);
    for (int g = tid; g < G; g += 256) {
      float sv[kTC];
#pragma unroll
      for (int tt = 0; tt < kTC; ++tt) sv[tt] = a.xs[(size_t)(tt < ntok ? tok[tt] : tok[0]) * G + g];
#pragma unroll
      for (int tt = 0; tt < kTC; ++tt)
        xsl[(tt < ntok ? tt : 0) * G + g] = sv[tt];
    }
    __syncthreads();
    // 3. compute, SwiGLU and store per sub-block
#pragma unroll
    for (int it = 0; it < kSub; ++it) {
      const int rb = ob * 4 + wave + 4 * it;    // 8-row block index within the expert
      float vg[kTC], vu[kTC];
#pragma unroll
      for (int tt = 0; tt < kTC; ++tt) { vg[tt] = 0.f; vu[tt] = 0.f; }
      if (!missing) {
#pragma unroll
        for (int gi = 0; gi < GPL; ++gi) {
          const int g = gl + 8 * gi;
          if (g >= G) continue;
          const float sg = f16_to_f32(sbg[it][gi]), bg = f16_to_f32(sbg[it][gi] >> 16);
          const float su = f16_to_f32(sbu[it][gi]), bu = f16_to_f32(sbu[it][gi] >> 16);
          // tokens innermost: each code pair is formed once and applied to
          // every token of the chunk (per-token chains as in the decode GEMV)
          float ag0[kTC], au0[kTC], ag1[kTC], au1[kTC];
#pragma unroll
          for (int tt = 0; tt < kTC; ++tt) { ag0[tt] = au0[tt] = ag1[tt] = au1[tt] = 0.f; }
#pragma unroll
          for (int m = 0; m < 8; ++m) {
            uint4 xv[kTC];
#pragma unroll
            for (int tt = 0; tt < kTC; ++tt)
              xv[tt] = tt < ntok ? *reinterpret_cast<const uint4*>(&xlds[(tt * G + g) * kXPad + 4 * m])
                                 : make_uint4(0, 0, 0, 0);
#pragma unroll
            for (int s2 = 0; s2 < BITS / 2; ++s2) {       // products u = 2 s2 and 2 s2 + 1
              const uint32_t qg0 = qpair<BITS>(cg[it][gi], m, 2 * s2, qk), qu0 = qpair<BITS>(cu[it][gi], m, 2 * s2, qk);
              const uint32_t qg1 = qpair<BITS>(cg[it][gi], m, 2 * s2 + 1, qk);
              const uint32_t qu1 = qpair<BITS>(cu[it][gi], m, 2 * s2 + 1, qk);
#pragma unroll
              for (int tt = 0; tt < kTC; ++tt) {
                if (tt < ntok) {
                  const uint32_t xw[4] = {xv[tt].x, xv[tt].y, xv[tt].z, xv[tt].w};
                  ag0[tt] = dot2_bf16(qg0, xw[qx<BITS>(2 * s2)], ag0[tt]);
                  au0[tt] = dot2_bf16(qu0, xw[qx<BITS>(2 * s2)], au0[tt]);
                  ag1[tt] = dot2_bf16(qg1, xw[qx<BITS>(2 * s2 + 1)], ag1[tt]);
                  au1[tt] = dot2_bf16(qu1, xw[qx<BITS>(2 * s2 + 1)], au1[tt]);
                }
              }
            }
          }
#pragma unroll
          for (int tt = 0; tt < kTC; ++tt) {
            if (tt < ntok) {
              const float sx = xsl[tt * G + g];
              vg[tt] += sg * (ag0[tt] + ag1[tt]) + (bg - qoff<BITS>() * sg) * sx;
              vu[tt] += su * (au0[tt] + au1[tt]) + (bu - qoff<BITS>() * su) * sx;
            }
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < kTC; ++tt) {
        const float gg = sum8_dpp(vg[tt]), uu = sum8_dpp(vu[tt]);
        if (gl == 0) hbuf[tt * 8 + r] = missing ? 0.f : gg / (1.0f + expf(-gg)) * uu;
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (lane < ntok) {
        float h[8];
#pragma unroll
        for (int rr = 0; rr < 8; ++rr) h[rr] = hbuf[lane * 8 + rr];
        int hr = hrow[0];
#pragma unroll
        for (int tt = 1; tt < kTC; ++tt)
          if (lane == tt) hr = hrow[tt];
        write_h8(h, a.hq, a.hs8, a.Imax, hr, rb);
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
    if (missing && tid == 0) atomicOr(a.pool.err, 1);
    __syncthreads();
  }
}

// One group (64 inputs) of one down row: s*sum((128+q)h) + (b-128s)*sum(h),
// LDS image of one h record (bf16 hi pairs, bf16 lo pairs, per-8 sums): the
// 32 dwords of each 64-row group are padded to kHG = 36, so the 8 group lanes
// of a wave (groups g = 0..7 read together) hit distinct banks; the per-8
// sums follow.  hrec_pos maps a dword of the record as stored in HBM (hi
// pairs [0, Imax/2), lo pairs [Imax/2, Imax), sums [Imax, Imax + Imax/8)).
constexpr int kHG = 36;
__host__ __device__ inline int hrec_words(int Imax) { return 2 * (Imax / 64) * kHG + Imax / 8; }
__device__ __forceinline__ int hrec_pos(int j, int Imax) {
  if (j >= Imax) return 2 * (Imax / 64) * kHG + (j - Imax);
  const int part = j >= Imax / 2, jj = part ? j - Imax / 2 : j;
  return (part * (Imax / 64) + (jj >> 5)) * kHG + (jj & 31);
}
__device__ __forceinline__ const float* hrec_sums(const uint32_t* hrec, int Imax) {
  return reinterpret_cast<const float*>(hrec + 2 * (Imax / 64) * kHG);
}

// h record rows: consecutive (decode rounds) or a short list (bucket chunks).
struct RowsFrom {
  int base;
  __device__ int operator()(int r) const { return base + r; }
};
struct Rows4 {                                  // up to four rows, named (no array to index)
  int v0, v1, v2, v3;
  __device__ int operator()(int r) const { return r == 0 ? v0 : r == 1 ? v1 : r == 2 ? v2 : v3; }
};

// Stage nrec h records (rows rows(0..nrec-1) of hq / hs8) into their LDS
// images by an NT-thread block.  Per pass every thread loads four 16-byte
// pair pieces and one sum piece before it stores any, with branch-free
// addressing (so the compiler neither waits per piece nor sinks the loads
// to their stores); pieces past the end reload and rewrite piece 0 of
// record 0 (same value, same place).
// One pass of it: the pieces in registers with their LDS destinations.
struct HPass {
  uint4 vp[4], vs;
  int dp[4], ds;
};
template <int NT, class Rows>
__device__ __forceinline__ void stage_h_load(const uint32_t* __restrict__ hq, const float* __restrict__ hs8, int Imax,
                                             int nrec, Rows rows, int rec, int it, HPass& p) {
  const int pp = Imax / 4, sp = Imax / 32;      // pair pieces and sum pieces per record
  const int np = nrec * pp, ns = nrec * sp;
#pragma unroll
  for (int uu = 0; uu < 4; ++uu) {
    int q = it * 4 * NT + NT * uu + (int)threadIdx.x;
    q = q < np ? q : 0;
    const int r = q / pp, c = q % pp;
    p.vp[uu] = reinterpret_cast<const uint4*>(hq + (size_t)rows(r) * Imax)[c];
    const int j = 4 * c, part = j >= Imax / 2 ? 1 : 0, jj = j - part * (Imax / 2);
    p.dp[uu] = r * rec + (part * (Imax / 64) + (jj >> 5)) * kHG + (jj & 31);
  }
  int q = it * NT + (int)threadIdx.x;
  q = q < ns ? q : 0;
  const int r = q / sp, c = q % sp;
  p.vs = reinterpret_cast<const uint4*>(hs8 + (size_t)rows(r) * (Imax / 8))[c];
  p.ds = r * rec + 2 * (Imax / 64) * kHG + 4 * c;
}
__device__ __forceinline__ void stage_h_store(uint32_t* hst, const HPass& p) {
#pragma unroll
  for (int uu = 0; uu < 4; ++uu) *reinterpret_cast<uint4*>(hst + p.dp[uu]) = p.vp[uu];
  *reinterpret_cast<uint4*>(hst + p.ds) = p.vs;
}
// Passes needed for nrec records by NT threads.
template <int NT>
__host__ __device__ inline int stage_h_passes(int nrec, int Imax) {
  const int np = nrec * (Imax / 4), ns = nrec * (Imax / 32);
  const int a = (np + 4 * NT - 1) / (4 * NT), b = (ns + NT - 1) / NT;
  return a > b ? a : b;
}
template <int NT, class Rows>
__device__ __forceinline__ void stage_h(const uint32_t* __restrict__ hq, const float* __restrict__ hs8, int Imax,
                                        int nrec, Rows rows, uint32_t* hst, int rec) {
  const int K = stage_h_passes<NT>(nrec, Imax);
  for (int it = 0; it < K; ++it) {
    HPass p;
    stage_h_load<NT>(hq, hs8, Imax, nrec, rows, rec, it, p);
    stage_h_store(hst, p);
  }
}

// h given as the LDS record above (hs: its per-8 sums); q0..q3: the
// group's code pieces (4-bit: q0, q1; 8-bit: q0..q3), qpair layout.
template <int BITS>
__device__ __forceinline__ float down_group_regs(uint4 q0, uint4 q1, uint4 q2, uint4 q3, uint32_t sb, int g,
                                                 const uint32_t* hrec, int Imax, const float* hs) {
  const float s = f16_to_f32(sb);
  const float b = f16_to_f32(sb >> 16);
  const uint32_t qw[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                           q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
  const QConst qk = q_const();
  const uint4* hh = reinterpret_cast<const uint4*>(hrec + g * kHG);
  const uint4* hl = reinterpret_cast<const uint4*>(hrec + (Imax / 64 + g) * kHG);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;      // four independent chains
#pragma unroll
  for (int m = 0; m < 8; ++m) {
    const uint4 vh = hh[m], vl = hl[m];
    const uint32_t ph[4] = {vh.x, vh.y, vh.z, vh.w};
    const uint32_t pl[4] = {vl.x, vl.y, vl.z, vl.w};
#pragma unroll
    for (int s2 = 0; s2 < BITS / 2; ++s2) {         // products u = 2 s2 and 2 s2 + 1
      const uint32_t c0 = qpw<BITS>(qw[qwi<BITS>(m, 2 * s2)], 2 * s2, qk);
      const uint32_t c1 = qpw<BITS>(qw[qwi<BITS>(m, 2 * s2 + 1)], 2 * s2 + 1, qk);
      a0 = dot2_bf16(c0, ph[qx<BITS>(2 * s2)], a0);
      a1 = dot2_bf16(c0, pl[qx<BITS>(2 * s2)], a1);
      a2 = dot2_bf16(c1, ph[qx<BITS>(2 * s2 + 1)], a2);
      a3 = dot2_bf16(c1, pl[qx<BITS>(2 * s2 + 1)], a3);
    }
  }
  const float acc = (a0 + a2) + (a1 + a3);
  float sh = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) sh += hs[8 * g + m];
  return s * acc + (b - qoff<BITS>() * s) * sh;
}

// Code pieces of group g of down row j (qpair layout).
template <int BITS>
__device__ __forceinline__ void down_load(const uint8_t* blob, const BlobLayout& L, int d, int j, int g,
                                          uint4 (&q)[BITS / 2], uint32_t* sb) {
#pragma unroll
  for (int p = 0; p < BITS / 2; ++p)
    q[p] = *reinterpret_cast<const uint4*>(blob + L.m[2].codes + ((uint64_t)((BITS / 2) * g + p) * d + j) * 16);
  *sb = *reinterpret_cast<const uint32_t*>(blob + L.m[2].sb + ((uint64_t)g * d + j) * 4);
}

template <int BITS>
__device__ __forceinline__ float down_group(const uint8_t* blob, const BlobLayout& L, int d, int j,
                                            int g, const uint32_t* __restrict__ hrec, int Imax,
                                            const float* __restrict__ hs) {
  uint4 q[BITS / 2];
  uint32_t sb;
  down_load<BITS>(blob, L, d, j, g, q, &sb);
  return down_group_regs<BITS>(q[0], q[1], q[BITS / 2 > 2 ? 2 : 0], q[BITS / 2 > 3 ? 3 : 0], sb, g, hrec, Imax, hs);
}

struct DownArgs {
  PoolView pool;
  const uint8_t* shared_blob;
  int d, I, Ish, Imax, T, k;
  const int32_t* sel_slot;      // decode: slot of each (token, rank) selection
  const float* w;
  const float* sgate;
  const uint32_t* hq;
  const float* hs8;
  float* y;
  // batched
  const Inst* inst;
  const int32_t* n_routed;
  int n_shared_inst;
  const int32_t* pair_ids;
  float* partial;
  float* shared_out;
  // decode, chains of layers: x_{l+1} = bf16(res_in + y) and the sums of
  // squares of each 8 output rows
  const uint16_t* res_in;
  uint16_t* res_out;
  float* ssp_out;
  // decode in two phases (expert streaming): phase 1 writes every
  // instance's outputs for these rows to oi_buf [T*(k+1)][d] (deferred
  // selections as 0) and stops; phase 2 computes the deferred selections
  // (pend[i] < 0), takes the others from oi_buf and combines
  int phase;
  const int32_t* pend;
  float* oi_buf;
};

// Decode: block = 8 output rows, all T*(k+1) instances, fused rank-order
// combine.  16 waves; instances are taken in rounds of 16 (one per wave):
// the round's code loads are issued first, its h records are staged in LDS
// meanwhile.  (down_decode_pipe_kernel below is used whenever its two
// record buffers fit the LDS; this one otherwise.)
constexpr int kDnWaves = 16;
constexpr int kDnRound = kDnWaves;
template <int BITS>
__global__ __launch_bounds__(64 * kDnWaves) void down_decode_kernel(DownArgs a) {
  constexpr int kNP = BITS / 2;                 // 16-byte code pieces per group
  extern __shared__ float dyn[];                // oi[nI][8] | wk[nI] | hst[kDnRound][hrec_words]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane >> 3, gl = lane & 7;       // group lanes of a row are consecutive
  const int jb = xcd_remap(blockIdx.x, gridDim.x);   // this block's 8 output rows
  const int j = jb * 8 + r;
  const int nR = a.T * a.k, nI = nR + a.T;
  const int rec = hrec_words(a.Imax);           // dwords per staged record
  float* oi = dyn;
  float* wk = dyn + nI * 8;                     // combine weights: w[T*k] then sgate[T]
  uint32_t* hst = reinterpret_cast<uint32_t*>(dyn + ((nI * 9 + 3) & ~3));
  // a chain's residual rows, loaded now (they depend on nothing here) so
  // the hand-over at the end does not wait for them
  const uint32_t res_pre = (a.res_out && tid < 8 * a.T) ? a.res_in[(size_t)(tid / 8) * a.d + jb * 8 + tid % 8] : 0u;
  for (int base = 0; base < nI; base += kDnRound) {
    const int nr = min(kDnRound, nI - base);
    const int i = base + wave;
    const bool active = wave < nr;
    // 1. the wave's selection slot (issued first: the code addresses wait
    //    for it), in the first round the combine weights (read now, their
    //    latency would otherwise land at the very end; nI <= 2048: two per
    //    thread, clamped so the loads stay unconditional), then the codes
    //    (no load of this round is conditional before the slot is used, so
    //    the wait for it is exact; the weights are loaded every round, the
    //    first round's are the ones stored)
    const int slot_ld = a.sel_slot[(active && i < nR) ? i : 0];
    float wkv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int qw = tid + 64 * kDnWaves * u < nI ? tid + 64 * kDnWaves * u : 0;
      wkv[u] = *(qw < nR ? a.w + qw : a.sgate + (qw - nR));
    }
    // phase 2 of a streamed step: instances done in phase 1 come from oi_buf
    bool from_buf = false;
    float obuf = 0.f;
    if (a.phase == 2 && active) {
      from_buf = i >= nR || a.pend[i] >= 0;
      if (from_buf) obuf = a.oi_buf[(size_t)i * a.d + j];
    }
    uint4 q[kNP];
    uint32_t sb = 0;
    bool miss = true;
    int Iinst = 0;
    const uint8_t* blob = nullptr;
    if (active && !from_buf) {
      if (i < nR) {
        const int slot = slot_ld;
        miss = slot < 0;
        blob = a.pool.slab + (uint64_t)(miss ? 0 : slot) * a.pool.stride;
        Iinst = a.I;
      } else {
        miss = false;
        blob = a.shared_blob;
        Iinst = a.Ish;
      }
      if (!miss && gl < Iinst / 64) {
        const BlobLayout L = blob_layout(a.d, Iinst, BITS);
#pragma unroll
        for (int p = 0; p < kNP; ++p)
          q[p] = *reinterpret_cast<const uint4*>(blob + L.m[2].codes + ((uint64_t)(kNP * gl + p) * a.d + j) * 16);
        sb = *reinterpret_cast<const uint32_t*>(blob + L.m[2].sb + ((uint64_t)gl * a.d + j) * 4);
      }
    }
    // 2. stage the round's h records (pairs + per-8 sums) in LDS; the
    //    weights go to LDS after them (a store before the h loads would wait
    //    for the code loads issued ahead of it)
    stage_h<64 * kDnWaves>(a.hq, a.hs8, a.Imax, nr, RowsFrom{base}, hst, rec);
    if (base == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        wk[tid + 64 * kDnWaves * u < nI ? tid + 64 * kDnWaves * u : 0] = wkv[u];
    }
    __syncthreads();
    // 3. compute
    if (active) {
      const uint32_t* hrec = hst + wave * rec;
      const float* hs = hrec_sums(hrec, a.Imax);
      float acc = 0.f;
      if (!miss) {
        if (gl < Iinst / 64) acc = down_group_regs<BITS>(q[0], q[1], q[kNP > 2 ? 2 : 0], q[kNP > 3 ? 3 : 0], sb, gl, hrec, a.Imax, hs);
        if (Iinst > 512) {                    // wider intermediates: further groups
          const BlobLayout L = blob_layout(a.d, Iinst, BITS);
          for (int g = gl + 8; g < Iinst / 64; g += 8) acc += down_group<BITS>(blob, L, a.d, j, g, hrec, a.Imax, hs);
        }
      }
      acc = sum8_dpp(acc);
      if (gl == 0) oi[i * 8 + r] = from_buf ? obuf : acc;
    }
    __syncthreads();
  }
  if (a.phase == 1) {                           // streamed step: hand the outputs to phase 2
    for (int q2 = tid; q2 < nI * 8; q2 += 64 * kDnWaves)
      a.oi_buf[(size_t)(q2 / 8) * a.d + jb * 8 + (q2 % 8)] = oi[q2];
    return;
  }
  if (tid < 8 * a.T) {
    const int t = tid / 8, rr = tid % 8;
    float y = 0.f;
    for (int q2 = 0; q2 < a.k; ++q2) y += wk[t * a.k + q2] * oi[(t * a.k + q2) * 8 + rr];
    y += wk[nR + t] * oi[(nR + t) * 8 + rr];
    const size_t yi = (size_t)t * a.d + jb * 8 + rr;
    a.y[yi] = y;
    if (a.res_out) {                            // chain hand-over (all 8 lanes of a token active)
      const uint32_t b = f32_to_bf16(__uint_as_float(res_pre << 16) + y);
      a.res_out[yi] = (uint16_t)b;
      const float r = __uint_as_float(b << 16);
      const float p = sum8_dpp(__fmul_rn(r, r));
      if (rr == 0) a.ssp_out[(size_t)t * (a.d / 8) + jb] = p;
    }
  }
}

// Decode down (the kernel used whenever its two record buffers fit the
// LDS): down_decode_kernel's arithmetic, with the h records fetched by LDS
// DMA and, over several rounds of instances, the next round's inputs in
// flight while the current round computes.
// Every selection slot is staged in LDS at the start (so no round's code
// loads wait for a slot); the next round's codes go to registers and its h
// records to the second of two LDS buffers by LDS DMA (no registers).  The
// record there: the hi pairs, then the lo pairs, as groups of 32 words whose
// 16-byte pieces are XOR-swizzled by the group (piece m of group g at word
// 32 g + 4 (m ^ (g & 7)): the reads of one piece by 8 group lanes hit 8
// different bank quads), then the per-8 sums.
__host__ __device__ inline int hrec_sw_words(int Imax) { return (Imax / 64) * 64 + Imax / 8; }

template <int BITS>
struct DnInst {                                 // a wave's instance in one round
  uint4 q[BITS / 2];
  uint32_t sb;
  bool miss, from_buf;
  float obuf;
  int Iinst;
  const uint8_t* blob;
};
template <int BITS>
__device__ __forceinline__ void dn_inst_load(const DownArgs& a, int i, bool active, int slot, int j, int gl,
                                             DnInst<BITS>& s) {
  constexpr int kNP = BITS / 2;
  const int nR = a.T * a.k;
  s.from_buf = false; s.obuf = 0.f; s.miss = true; s.Iinst = 0; s.blob = nullptr; s.sb = 0;
  if (a.phase == 2 && active) {
    s.from_buf = i >= nR || a.pend[i] >= 0;
    if (s.from_buf) s.obuf = a.oi_buf[(size_t)i * a.d + j];
  }
  if (active && !s.from_buf) {
    if (i < nR) {
      s.miss = slot < 0;
      s.blob = a.pool.slab + (uint64_t)(s.miss ? 0 : slot) * a.pool.stride;
      s.Iinst = a.I;
    } else {
      s.miss = false;
      s.blob = a.shared_blob;
      s.Iinst = a.Ish;
    }
    if (!s.miss && gl < s.Iinst / 64) {
      const BlobLayout L = blob_layout(a.d, s.Iinst, BITS);
#pragma unroll
      for (int p = 0; p < kNP; ++p)
        s.q[p] = *reinterpret_cast<const uint4*>(s.blob + L.m[2].codes + ((uint64_t)(kNP * gl + p) * a.d + j) * 16);
      s.sb = *reinterpret_cast<const uint32_t*>(s.blob + L.m[2].sb + ((uint64_t)gl * a.d + j) * 4);
    }
  }
}

// Record of h row hr into LDS at rec (swizzled layout) by one wave's DMAs.
__device__ __forceinline__ void h_record_dma(rsrc_t rq, rsrc_t rs, int hr, int Imax, uint32_t* rec, int lane) {
  const int npc = Imax / 8;                     // 16-byte pieces per part
#pragma unroll
  for (int part = 0; part < 2; ++part)
    for (int p0 = 0; p0 < npc; p0 += 64) {
      const int L = p0 + lane;
      if (L < npc) {
        const int g = L >> 3, m = (L & 7) ^ (g & 7);
        const uint32_t src = ((uint32_t)hr * Imax + part * (Imax / 2) + 32 * g + 4 * m) * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rq, lds_opaque(rec + part * (Imax / 64) * 32 + 4 * p0), 16, src, 0,
                                                 0, 0);
      }
    }
  for (int p0 = 0; p0 < Imax / 8; p0 += 64) {   // the sums, a word per lane
    const int L = p0 + lane;
    if (L < Imax / 8)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, lds_opaque(rec + 2 * (Imax / 64) * 32 + p0), 4,
                                               ((uint32_t)hr * (Imax / 8) + L) * 4, 0, 0, 0);
  }
}

// down_group_regs on the swizzled record.
template <int BITS>
__device__ __forceinline__ float down_group_sw(uint4 q0, uint4 q1, uint4 q2, uint4 q3, uint32_t sb, int g,
                                               const uint32_t* hrec, int Imax) {
  const float s = f16_to_f32(sb);
  const float b = f16_to_f32(sb >> 16);
  const uint32_t qw[16] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w,
                           q2.x, q2.y, q2.z, q2.w, q3.x, q3.y, q3.z, q3.w};
  const QConst qk = q_const();
  const uint32_t* gh = hrec + 32 * g;
  const uint32_t* glo = hrec + (Imax / 64 + g) * 32;
  const float* hs = reinterpret_cast<const float*>(hrec + 2 * (Imax / 64) * 32);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;      // four independent chains
#pragma unroll 2
  for (int m = 0; m < 8; ++m) {
    const int pm = 4 * (m ^ (g & 7));
    const uint4 vh = *reinterpret_cast<const uint4*>(gh + pm), vl = *reinterpret_cast<const uint4*>(glo + pm);
    const uint32_t ph[4] = {vh.x, vh.y, vh.z, vh.w};
    const uint32_t pl[4] = {vl.x, vl.y, vl.z, vl.w};
#pragma unroll
    for (int s2 = 0; s2 < BITS / 2; ++s2) {         // products u = 2 s2 and 2 s2 + 1
      const uint32_t c0 = qpw<BITS>(qw[qwi<BITS>(m, 2 * s2)], 2 * s2, qk);
      const uint32_t c1 = qpw<BITS>(qw[qwi<BITS>(m, 2 * s2 + 1)], 2 * s2 + 1, qk);
      a0 = dot2_bf16(c0, ph[qx<BITS>(2 * s2)], a0);
      a1 = dot2_bf16(c0, pl[qx<BITS>(2 * s2)], a1);
      a2 = dot2_bf16(c1, ph[qx<BITS>(2 * s2 + 1)], a2);
      a3 = dot2_bf16(c1, pl[qx<BITS>(2 * s2 + 1)], a3);
    }
  }
  const float acc = (a0 + a2) + (a1 + a3);
  float sh = 0.f;
#pragma unroll
  for (int m = 0; m < 8; ++m) sh += hs[8 * g + m];
  return s * acc + (b - qoff<BITS>() * s) * sh;
}

// every DMA and load of this wave landed, then the block meets (no memory
// access moves across)
__device__ __forceinline__ void wait_all_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int BITS>
__global__ __launch_bounds__(64 * kDnWaves) void down_decode_pipe_kernel(DownArgs a) {
  constexpr int kNP = BITS / 2;
  extern __shared__ float dyn[];                // oi[nI][8] | wk[nI] | slots[nR] | hst[2][kDnRound][rec]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane >> 3, gl = lane & 7;
  const int jb = xcd_remap(blockIdx.x, gridDim.x);
  const int j = jb * 8 + r;
  const int nR = a.T * a.k, nI = nR + a.T;
  const int rec = hrec_sw_words(a.Imax);
  float* oi = dyn;
  float* wk = dyn + nI * 8;
  int32_t* sl = reinterpret_cast<int32_t*>(wk + nI);
  uint32_t* hst = reinterpret_cast<uint32_t*>(dyn + ((nI * 9 + nR + 3) & ~3));
  const rsrc_t rq = make_rsrc(a.hq, (uint32_t)nI * a.Imax * 4);
  const rsrc_t rs = make_rsrc(a.hs8, (uint32_t)nI * (a.Imax / 8) * 4);
  // a chain's residual rows, loaded now (they depend on nothing here) so
  // the hand-over at the end does not wait for them
  const uint32_t res_pre = (a.res_out && tid < 8 * a.T) ? a.res_in[(size_t)(tid / 8) * a.d + jb * 8 + tid % 8] : 0u;
  DnInst<BITS> cur;
  {
    // round 0: its slot straight from memory and its records by DMA; the
    // combine weights and every routed slot (nR <= 2048: two per thread,
    // clamped) go to LDS
    const bool active = wave < kDnRound && wave < nI;
    const int slot0 = a.sel_slot[(active && wave < nR) ? wave : 0];
    float wkv[2];
    int32_t sv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 64 * kDnWaves * u;
      const int qw = q < nI ? q : 0;
      wkv[u] = *(qw < nR ? a.w + qw : a.sgate + (qw - nR));
      sv[u] = a.sel_slot[q < nR ? q : 0];
    }
    if (active) h_record_dma(rq, rs, wave, a.Imax, hst + wave * rec, lane);
    dn_inst_load<BITS>(a, wave, active, slot0, j, gl, cur);
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int q = tid + 64 * kDnWaves * u;
      wk[q < nI ? q : 0] = wkv[u];
      sl[q < nR ? q : 0] = sv[u];
    }
  }
  wait_all_barrier();
  int buf = 0;
  for (int base = 0; base < nI; base += kDnRound) {
    const int nr = min(kDnRound, nI - base);
    const int i = base + wave;
    const bool active = wave < nr;
    const int nb = base + kDnRound, nnr = min(kDnRound, nI - nb);
    // 1. the next round's records (into the other buffer: every wave is past
    //    its reads of it, the barrier that ended the previous round) and codes
    DnInst<BITS> nxt;
    if (nnr > 0) {
      const int i2 = nb + wave;
      const bool act2 = wave < nnr;
      if (act2) h_record_dma(rq, rs, i2, a.Imax, hst + ((buf ^ 1) * kDnRound + wave) * rec, lane);
      dn_inst_load<BITS>(a, i2, act2, sl[(act2 && i2 < nR) ? i2 : 0], j, gl, nxt);
    }
    // 2. this round
    if (active) {
      const uint32_t* hrec = hst + (buf * kDnRound + wave) * rec;
      float acc = 0.f;
      if (!cur.miss) {
        if (gl < cur.Iinst / 64)
          acc = down_group_sw<BITS>(cur.q[0], cur.q[1], cur.q[kNP > 2 ? 2 : 0], cur.q[kNP > 3 ? 3 : 0], cur.sb, gl,
                                    hrec, a.Imax);
        if (cur.Iinst > 512) {                  // wider intermediates: further groups
          const BlobLayout L = blob_layout(a.d, cur.Iinst, BITS);
          for (int g = gl + 8; g < cur.Iinst / 64; g += 8) {
            uint4 q[kNP];
            uint32_t sb;
            down_load<BITS>(cur.blob, L, a.d, j, g, q, &sb);
            acc += down_group_sw<BITS>(q[0], q[1], q[kNP > 2 ? 2 : 0], q[kNP > 3 ? 3 : 0], sb, g, hrec, a.Imax);
          }
        }
      }
      acc = sum8_dpp(acc);
      if (gl == 0) oi[i * 8 + r] = cur.from_buf ? cur.obuf : acc;
    }
    if (nnr > 0) cur = nxt;
    buf ^= 1;
    wait_all_barrier();
  }
  if (a.phase == 1) {                           // streamed step: hand the outputs to phase 2
    for (int q2 = tid; q2 < nI * 8; q2 += 64 * kDnWaves)
      a.oi_buf[(size_t)(q2 / 8) * a.d + jb * 8 + (q2 % 8)] = oi[q2];
    return;
  }
  if (tid < 8 * a.T) {
    const int t = tid / 8, rr = tid % 8;
    float y = 0.f;
    for (int q2 = 0; q2 < a.k; ++q2) y += wk[t * a.k + q2] * oi[(t * a.k + q2) * 8 + rr];
    y += wk[nR + t] * oi[(nR + t) * 8 + rr];
    const size_t yi = (size_t)t * a.d + jb * 8 + rr;
    a.y[yi] = y;
    if (a.res_out) {                            // chain hand-over (all 8 lanes of a token active)
      const uint32_t b = f32_to_bf16(__uint_as_float(res_pre << 16) + y);
      a.res_out[yi] = (uint16_t)b;
      const float rv = __uint_as_float(b << 16);
      const float p = sum8_dpp(__fmul_rn(rv, rv));
      if (rr == 0) a.ssp_out[(size_t)t * (a.d / 8) + jb] = p;
    }
  }
}

// Sub-blocks of 8 rows per wave in the batched down GEMV: all their codes
// are in registers at once (4-bit: 8 x 32 B, 8-bit: 4 x 64 B).
template <int BITS> constexpr int kDnSub = BITS == 4 ? 8 : 4;

// Batched down: item = (bucket chunk, 256 (4-bit) or 128 (8-bit) output rows).  The chunk's h
// records are staged in LDS once; each wave takes 8-row sub-blocks (8 rows x
// 8 group lanes), loads the codes once and applies them to every token.
template <int BITS>
__global__ __launch_bounds__(256) void down_batched_kernel(DownArgs a) {
  constexpr int kNP = BITS / 2;                 // 16-byte code pieces per group
  extern __shared__ uint32_t hst[];            // [kTC][Imax + Imax/8]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane >> 3, gl = lane & 7;
  constexpr int kRows = 32 * kDnSub<BITS>;     // output rows per item
  const int nrb = (a.d + kRows - 1) / kRows;    // d is a multiple of 64: last block may be partial
  const int nR = *a.n_routed;
  const int items = (nR + a.n_shared_inst) * nrb;
  const int rec = hrec_words(a.Imax);
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int ii = item / nrb, j0 = (item % nrb) * kRows;
    const bool routed = ii < nR;
    const Inst in = a.inst[ii];
    const uint8_t* blob;
    int Iinst;
    bool missing = false;
    if (routed) {
      const int e = in.expert;
      const int slot = (e >= 0 && e < a.pool.E) ? a.pool.slot_table[e] : -1;
      missing = slot < 0;
      blob = a.pool.slab + (uint64_t)(slot < 0 ? 0 : slot) * a.pool.stride;
      Iinst = a.I;
    } else {
      blob = a.shared_blob;
      Iinst = a.Ish;
    }
    int hrow[kTC];
#pragma unroll
    for (int tt = 0; tt < kTC; ++tt)
      hrow[tt] = tt < in.n ? (routed ? a.pair_ids[in.start + tt] : a.T * a.k + in.start + tt) : 0;
    const BlobLayout L = blob_layout(a.d, Iinst, BITS);
    // 1. every code this wave needs (its 8 sub-blocks of 8 rows, group gl):
    //    all loads in flight at once, ahead of the h staging
    constexpr int kSub = kDnSub<BITS>;          // sub-blocks of 8 rows per wave
    uint4 q[kSub][kNP];
    uint32_t sbv[kSub];
    const bool gok = gl < Iinst / 64;
#pragma unroll
    for (int it = 0; it < kSub; ++it) {
      const int j = j0 + (wave + 4 * it) * 8 + r;
#pragma unroll
      for (int p = 0; p < kNP; ++p) q[it][p] = make_uint4(0, 0, 0, 0);
      sbv[it] = 0;
      if (!missing && gok && j < a.d) {
#pragma unroll
        for (int p = 0; p < kNP; ++p)
          q[it][p] = *reinterpret_cast<const uint4*>(blob + L.m[2].codes + ((uint64_t)(kNP * gl + p) * a.d + j) * 16);
        sbv[it] = *reinterpret_cast<const uint32_t*>(blob + L.m[2].sb + ((uint64_t)gl * a.d + j) * 4);
      }
    }
    // 2. the chunk's h records
    {
      static_assert(kTC == 4, "bucket chunks of four tokens");
      stage_h<256>(a.hq, a.hs8, a.Imax, in.n, Rows4{hrow[0], hrow[1], hrow[2], hrow[3]}, hst, rec);
    }
    __syncthreads();
    // 3. compute and store, sub-block by sub-block
#pragma unroll
    for (int it = 0; it < kSub; ++it) {
      const int j = j0 + (wave + 4 * it) * 8 + r;
      const bool jv = j < a.d;
      float acc[kTC];
#pragma unroll
      for (int tt = 0; tt < kTC; ++tt) acc[tt] = 0.f;
      if (!missing && jv) {
        if (gok) {
#pragma unroll
          for (int tt = 0; tt < kTC; ++tt) {
            if (tt < in.n) {
              const uint32_t* hrec = hst + tt * rec;
              acc[tt] += down_group_regs<BITS>(q[it][0], q[it][1], q[it][kNP > 2 ? 2 : 0], q[it][kNP > 3 ? 3 : 0], sbv[it],
                                                 gl, hrec, a.Imax, hrec_sums(hrec, a.Imax));
            }
          }
        }
        if (Iinst > 512) {                    // intermediates wider than 512: further groups
          for (int g = gl + 8; g < Iinst / 64; g += 8) {
            for (int tt = 0; tt < in.n; ++tt) {
              const uint32_t* hrec = hst + tt * rec;
              const float v = down_group<BITS>(blob, L, a.d, j, g, hrec, a.Imax, hrec_sums(hrec, a.Imax));
#pragma unroll
              for (int u = 0; u < kTC; ++u)
                if (u == tt) acc[u] += v;
            }
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < kTC; ++tt) {
        const float v = sum8_dpp(acc[tt]);
        if (gl == 0 && tt < in.n && jv) {
          if (routed) a.partial[(size_t)hrow[tt] * a.d + j] = v;
          else a.shared_out[(size_t)(in.start + tt) * a.d + j] = v;
        }
      }
    }
    if (missing && tid == 0) atomicOr(a.pool.err, 1);
    __syncthreads();
  }
}

// Batched instance list: per expert ceil(count/kTC) chunks in expert order,
// then ceil(T/kTC) shared chunks.  One block.
__global__ __launch_bounds__(1024) void plan_kernel(const int32_t* __restrict__ offsets, int E, int T,
                                                    Inst* __restrict__ inst, int32_t* __restrict__ n_routed) {
  __shared__ int sums[1024];
  const int tid = threadIdx.x;
  // E <= 1024: one expert per thread
  const int c = tid < E ? offsets[tid + 1] - offsets[tid] : 0;
  const int nch = (c + kTC - 1) / kTC;
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
    Inst in;
    in.expert = tid;
    in.start = offsets[tid] + q * kTC;
    in.n = min(kTC, c - q * kTC);
    inst[base + q] = in;
  }
  const int total = sums[1023];
  if (tid == 0) *n_routed = total;
  const int nsh = (T + kTC - 1) / kTC;
  for (int q = tid; q < nsh; q += 1024) {
    Inst in;
    in.expert = -1;
    in.start = q * kTC;
    in.n = min(kTC, T - q * kTC);
    inst[total + q] = in;
  }
}


// ------------------------------------------------------------- f32 experts
// Unquantised fp32 experts (row-major [out][in] matrices, gate | up | down).
// gate/up: one wave per weight row, its 64 lanes striding over d in float4
// pieces (a row is one contiguous read), both matrices, every token of the
// instance; x is staged in LDS as bf16 and widened on use.  down: 8 lanes
// per output row (as in the quantised kernels), h staged in LDS.  Products
// and sums in fp32; h kept in fp32.
constexpr int kF32Pass = 2048;                  // inputs of a gate/up row per register pass

__device__ __forceinline__ float4 bf16x4_to_f32(uint2 v) {
  return make_float4(bf16_lo(v.x), bf16_hi(v.x), bf16_lo(v.y), bf16_hi(v.y));
}
__device__ __forceinline__ float dot4(float4 a, float4 b, float acc) {
  acc = fmaf(a.x, b.x, acc);
  acc = fmaf(a.y, b.y, acc);
  acc = fmaf(a.z, b.z, acc);
  return fmaf(a.w, b.w, acc);
}

// item = (instance, 4 rows): wave w takes row 4 rb + w of gate and up.
template <int TC>
__global__ __launch_bounds__(256, 4) void gate_up_f32_kernel(GateUpArgs a) {
  extern __shared__ uint16_t xb[];              // [TC][d] bf16
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int rbR = a.I / 4, rbS = a.Ish / 4;
  const int nR = a.batched ? *a.n_routed : a.T * a.k;
  const int nS = a.batched ? a.n_shared_inst : a.T;
  const int items = nR * rbR + nS * rbS;
  const int d4 = a.d / 4;
  constexpr int NV = kF32Pass / 256;            // float4 per lane per matrix per pass
  for (int item = xcd_remap(blockIdx.x, gridDim.x); item < items; item += gridDim.x) {
    const bool routed = item < nR * rbR;
    const int rel = routed ? item : item - nR * rbR;
    const int rb_per = routed ? rbR : rbS;
    const int i = rel / rb_per, rb = rel % rb_per;
    const uint8_t* blob;
    int Iinst, tok[TC], hrow[TC];
    bool missing;
    const int ntok = resolve(a, routed, i, &blob, &Iinst, tok, hrow, &missing);
    if (!a.batched && routed && rb == 0 && tid == 0)
      a.sel_slot[i] = missing ? -1 : (int32_t)((blob - a.pool.slab) / a.pool.stride);
    const BlobLayout L = blob_layout(a.d, Iinst, 32);
    const int o = rb * 4 + wave;
    const float4* wg = reinterpret_cast<const float4*>(blob + L.m[0].codes) + (size_t)o * d4;
    const float4* wu = reinterpret_cast<const float4*>(blob + L.m[1].codes) + (size_t)o * d4;
    float g[TC], u[TC];
#pragma unroll
    for (int tt = 0; tt < TC; ++tt) { g[tt] = 0.f; u[tt] = 0.f; }
    for (int p0 = 0; p0 < d4; p0 += kF32Pass / 4) {
      // this pass's weights first, then (first pass) the activations
      float4 gv[NV], uv[NV];
#pragma unroll
      for (int v = 0; v < NV; ++v) {
        const int f = p0 + 64 * v + lane;
        const bool ok = !missing && f < d4 && 64 * v < kF32Pass / 4;
        gv[v] = ok ? wg[f] : make_float4(0.f, 0.f, 0.f, 0.f);
        uv[v] = ok ? wu[f] : make_float4(0.f, 0.f, 0.f, 0.f);
      }
      if (p0 == 0) {
        for (int c8 = tid; c8 < a.d / 8; c8 += 256) {   // all tokens' pieces in flight together
          uint4 v4[TC];
#pragma unroll
          for (int tt = 0; tt < TC; ++tt)
            v4[tt] = reinterpret_cast<const uint4*>(a.x + (size_t)(tt < ntok ? tok[tt] : tok[0]) * a.d)[c8];
#pragma unroll
          for (int tt = 0; tt < TC; ++tt)
            reinterpret_cast<uint4*>(xb + (size_t)(tt < ntok ? tt : 0) * a.d)[c8] = v4[tt];
        }
        __syncthreads();
      }
#pragma unroll
      for (int tt = 0; tt < TC; ++tt) {
        if (tt < ntok) {
#pragma unroll
          for (int v = 0; v < NV; ++v) {
            const int f = p0 + 64 * v + lane;
            if (f < d4) {
              const float4 xv = bf16x4_to_f32(reinterpret_cast<const uint2*>(xb + (size_t)tt * a.d)[f]);
              g[tt] = dot4(gv[v], xv, g[tt]);
              u[tt] = dot4(uv[v], xv, u[tt]);
            }
          }
        }
      }
    }
    float hv = 0.f;
    int hr = 0;
#pragma unroll
    for (int tt = 0; tt < TC; ++tt) {
      const float gg = wave_sum(g[tt]), uu = wave_sum(u[tt]);
      if (lane == tt) {
        hv = missing ? 0.f : gg / (1.0f + expf(-gg)) * uu;
        hr = hrow[tt];
      }
    }
    if (lane < ntok) reinterpret_cast<float*>(a.hq)[(size_t)hr * a.Imax + o] = hv;
    if (missing && tid == 0) atomicOr(a.pool.err, 1);
    __syncthreads();
  }
}

// down row j of an f32 expert against an fp32 h held in LDS: lane gl of the
// row's 8 takes float4 pieces gl, gl+8, ...; returns this lane's part.
template <int NW>
__device__ __forceinline__ float down_f32_part(const float4 (&wv)[NW], const float* hl, int gl, int I4) {
  float acc = 0.f;
#pragma unroll
  for (int v = 0; v < NW; ++v) {
    const int f = gl + 8 * v;
    if (f < I4) acc = dot4(wv[v], reinterpret_cast<const float4*>(hl)[f], acc);
  }
  return acc;
}

constexpr int kF32DnW = 16;                     // float4 per lane per register pass (I <= 512)

// Decode: block = 8 output rows, all T*(k+1) instances in rounds of 16 (one
// per wave), fused rank-order combine (as down_decode_kernel).
__global__ __launch_bounds__(64 * kDnWaves) void down_decode_f32_kernel(DownArgs a) {
  extern __shared__ float dyn[];                // oi[nI][8] | wk[nI] | hst[kDnRound][Imax]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane >> 3, gl = lane & 7;
  const int jb = xcd_remap(blockIdx.x, gridDim.x);
  const int j = jb * 8 + r;
  const int nR = a.T * a.k, nI = nR + a.T;
  float* oi = dyn;
  float* wk = dyn + nI * 8;
  float* hst = dyn + ((nI * 9 + 3) & ~3);
  for (int base = 0; base < nI; base += kDnRound) {
    const int nr = min(kDnRound, nI - base);
    const int i = base + wave;
    const bool active = wave < nr;
    // the selection slot first, then the combine weights (every round,
    // unconditional; the first round's are stored), then the weights
    const int slot_ld = a.sel_slot[(active && i < nR) ? i : 0];
    float wkv[2];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int qw = tid + 64 * kDnWaves * u < nI ? tid + 64 * kDnWaves * u : 0;
      wkv[u] = *(qw < nR ? a.w + qw : a.sgate + (qw - nR));
    }
    bool miss = true;
    int Iinst = 0;
    const uint8_t* blob = nullptr;
    float4 wv[kF32DnW];
    if (active) {
      if (i < nR) {
        const int slot = slot_ld;
        miss = slot < 0;
        blob = a.pool.slab + (uint64_t)(miss ? 0 : slot) * a.pool.stride;
        Iinst = a.I;
      } else {
        miss = false;
        blob = a.shared_blob;
        Iinst = a.Ish;
      }
    }
    const int I4 = Iinst / 4;
    const float4* wd = nullptr;
    if (active && !miss) {
      const BlobLayout L = blob_layout(a.d, Iinst, 32);
      wd = reinterpret_cast<const float4*>(blob + L.m[2].codes) + (size_t)j * I4;
    }
#pragma unroll
    for (int v = 0; v < kF32DnW; ++v) {
      const int f = gl + 8 * v;
      wv[v] = (wd && f < I4) ? wd[f] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    // the round's h records, then the weights (see the quantised kernel)
    const int im4 = a.Imax / 4;
    for (int q0 = tid; q0 < nr * im4; q0 += 2 * 64 * kDnWaves) {   // two pieces per thread in flight
      float4 v4[2];
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int q4 = q0 + 64 * kDnWaves * uu < nr * im4 ? q0 + 64 * kDnWaves * uu : 0;   // clamped
        v4[uu] = reinterpret_cast<const float4*>(a.hq + (size_t)(base + q4 / im4) * a.Imax)[q4 % im4];
      }
#pragma unroll
      for (int uu = 0; uu < 2; ++uu) {
        const int q4 = q0 + 64 * kDnWaves * uu < nr * im4 ? q0 + 64 * kDnWaves * uu : 0;
        reinterpret_cast<float4*>(hst + (size_t)(q4 / im4) * a.Imax)[q4 % im4] = v4[uu];
      }
    }
    if (base == 0) {
#pragma unroll
      for (int u = 0; u < 2; ++u)
        wk[tid + 64 * kDnWaves * u < nI ? tid + 64 * kDnWaves * u : 0] = wkv[u];
    }
    __syncthreads();
    if (active) {
      const float* hl = hst + (size_t)wave * a.Imax;
      float acc = 0.f;
      if (wd) {
        acc = down_f32_part<kF32DnW>(wv, hl, gl, I4);
        for (int p0 = 8 * kF32DnW; p0 < I4; p0 += 8 * kF32DnW) {   // intermediates wider than 512
#pragma unroll
          for (int v = 0; v < kF32DnW; ++v) {
            const int f = p0 + gl + 8 * v;
            if (f < I4) acc = dot4(wd[f], reinterpret_cast<const float4*>(hl)[f], acc);
          }
        }
      }
      acc = sum8_dpp(acc);
      if (gl == 0) oi[i * 8 + r] = acc;
    }
    __syncthreads();
  }
  if (tid < 8 * a.T) {
    const int t = tid / 8, rr = tid % 8;
    float y = 0.f;
    for (int q2 = 0; q2 < a.k; ++q2) y += wk[t * a.k + q2] * oi[(t * a.k + q2) * 8 + rr];
    y += wk[nR + t] * oi[(nR + t) * 8 + rr];
    a.y[(size_t)t * a.d + jb * 8 + rr] = y;
  }
}

// Batched: item = (bucket chunk, 32 output rows): wave w takes rows
// j0 + 8 w .. + 7 (8 lanes each), the chunk's h records staged in LDS.
__global__ __launch_bounds__(256) void down_batched_f32_kernel(DownArgs a) {
  extern __shared__ float hsf[];                // [kTC][Imax]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r = lane >> 3, gl = lane & 7;
  const int nrb = (a.d + 31) / 32;
  const int nR = *a.n_routed;
  const int items = (nR + a.n_shared_inst) * nrb;
  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int ii = item / nrb, j0 = (item % nrb) * 32;
    const bool routed = ii < nR;
    const Inst in = a.inst[ii];
    const uint8_t* blob;
    int Iinst;
    bool missing = false;
    if (routed) {
      const int e = in.expert;
      const int slot = (e >= 0 && e < a.pool.E) ? a.pool.slot_table[e] : -1;
      missing = slot < 0;
      blob = a.pool.slab + (uint64_t)(slot < 0 ? 0 : slot) * a.pool.stride;
      Iinst = a.I;
    } else {
      blob = a.shared_blob;
      Iinst = a.Ish;
    }
    const int I4 = Iinst / 4;
    const int j = j0 + 8 * wave + r;
    const bool jv = j < a.d;
    const BlobLayout L = blob_layout(a.d, Iinst, 32);
    const float4* wd = reinterpret_cast<const float4*>(blob + L.m[2].codes) + (size_t)(jv ? j : 0) * I4;
    float4 wv[kF32DnW];
#pragma unroll
    for (int v = 0; v < kF32DnW; ++v) {
      const int f = gl + 8 * v;
      wv[v] = (!missing && jv && f < I4) ? wd[f] : make_float4(0.f, 0.f, 0.f, 0.f);
    }
    const int im4 = a.Imax / 4;
    int hrow[kTC];
#pragma unroll
    for (int tt = 0; tt < kTC; ++tt)
      hrow[tt] = tt < in.n ? (routed ? a.pair_ids[in.start + tt] : a.T * a.k + in.start + tt) : 0;
    for (int c = tid; c < im4; c += 256) {        // the kTC records' pieces in flight together
      float4 v4[kTC];
#pragma unroll
      for (int tt = 0; tt < kTC; ++tt)
        v4[tt] = reinterpret_cast<const float4*>(a.hq + (size_t)(tt < in.n ? hrow[tt] : hrow[0]) * a.Imax)[c];
#pragma unroll
      for (int tt = 0; tt < kTC; ++tt)
        reinterpret_cast<float4*>(hsf + (size_t)(tt < in.n ? tt : 0) * a.Imax)[c] = v4[tt];
    }
    __syncthreads();
    float acc[kTC];
#pragma unroll
    for (int tt = 0; tt < kTC; ++tt) {
      acc[tt] = 0.f;
      if (tt < in.n && !missing && jv) {
        const float* hl = hsf + (size_t)tt * a.Imax;
        acc[tt] = down_f32_part<kF32DnW>(wv, hl, gl, I4);
        for (int p0 = 8 * kF32DnW; p0 < I4; p0 += 8 * kF32DnW) {
          for (int v = 0; v < kF32DnW; ++v) {
            const int f = p0 + gl + 8 * v;
            if (f < I4) acc[tt] = dot4(wd[f], reinterpret_cast<const float4*>(hl)[f], acc[tt]);
          }
        }
      }
    }
#pragma unroll
    for (int tt = 0; tt < kTC; ++tt) {
      const float v = sum8_dpp(acc[tt]);
      if (gl == 0 && tt < in.n && jv) {
        const int hr = routed ? a.pair_ids[in.start + tt] : 0;
        if (routed) a.partial[(size_t)hr * a.d + j] = v;
        else a.shared_out[(size_t)(in.start + tt) * a.d + j] = v;
      }
    }
    if (missing && tid == 0) atomicOr(a.pool.err, 1);
    __syncthreads();
  }
}

struct FfnWs {
  uint32_t* xq; float* xs;
  uint32_t* hq; float* hs8;
  int32_t* sel_slot;
  int32_t* pend; float* oi_buf;     // decode: two-phase steps
  Inst* inst; int32_t* n_routed;
};

bool carve_ffn(Carver& c, int d, int Imax, int T, int k, int path, FfnWs* w) {
  const size_t hrows = (size_t)T * k + T;
  w->xq = c.take<uint32_t>((size_t)T * d / 2);
  w->xs = c.take<float>((size_t)T * d / 64);
  w->hq = c.take<uint32_t>(hrows * Imax);
  w->hs8 = c.take<float>(hrows * Imax / 8);
  w->sel_slot = c.take<int32_t>((size_t)T * k);
  w->pend = nullptr;
  w->oi_buf = nullptr;
  if (path == MOE_PATH_DECODE) {
    w->pend = c.take<int32_t>((size_t)T * k);
    w->oi_buf = c.take<float>(hrows * d);
  }
  w->inst = nullptr;
  w->n_routed = nullptr;
  if (path != MOE_PATH_DECODE) {
    w->inst = c.take<Inst>((size_t)T * k + (T + kTC - 1) / kTC);
    w->n_routed = c.take<int32_t>(64);
  }
  return c.ok();
}

int grid_for(int items_upper) {
  return items_upper < 8192 ? (items_upper > 0 ? items_upper : 1) : 8192;
}

// Kernel instances for experts of BITS-bit codes.
template <int BITS>
struct GemvFns {
  template <int GPL>
  static void* gate_up_g(int nk) {
    switch (nk) {
      case 1: return (void*)gate_up_kernel<1, 1, GPL, BITS, false>;
      case 2: return (void*)gate_up_kernel<1, 2, GPL, BITS, false>;
      case 4: return (void*)gate_up_kernel<1, 4, GPL, BITS, false>;
      case 8: return (void*)gate_up_kernel<1, 8, GPL, BITS, false>;
      case 0: return (void*)gate_up_kernel<1, 1, GPL, BITS, true>;   // RAW (nk unused)
      default: return (void*)gate_up_kernel<1, 16, GPL, BITS, false>;
    }
  }
  // raw: routing given and no prepared activations (the blocks form them)
  static void* gate_up(int nk, int G, bool raw = false) {
    if (raw) nk = 0;
    return G <= 32 ? gate_up_g<1>(nk) : G <= 64 ? gate_up_g<2>(nk) : gate_up_g<4>(nk);
  }
  static void* gate_up_batched(int G) {
    return G <= 8 ? (void*)gate_up_batched_kernel<1, BITS> : G <= 16 ? (void*)gate_up_batched_kernel<2, BITS>
         : G <= 32 ? (void*)gate_up_batched_kernel<4, BITS> : G <= 64 ? (void*)gate_up_batched_kernel<8, BITS>
         : (void*)gate_up_batched_kernel<16, BITS>;
  }
  static void* down_decode() { return (void*)down_decode_kernel<BITS>; }
  static void* down_decode_pipe() { return (void*)down_decode_pipe_kernel<BITS>; }
  static void* down_batched() { return (void*)down_batched_kernel<BITS>; }
};

struct GemvSet {
  void* (*gate_up)(int, int, bool);
  void* (*gate_up_batched)(int);
  void* (*down_decode)();
  void* (*down_decode_pipe)();
  void* (*down_batched)();
};
template <int BITS>
GemvSet gemv_set() {
  return {GemvFns<BITS>::gate_up, GemvFns<BITS>::gate_up_batched, GemvFns<BITS>::down_decode,
          GemvFns<BITS>::down_decode_pipe, GemvFns<BITS>::down_batched};
}

}  // namespace

// AUTO: the per-token decode GEMVs up to 8 tokens; beyond that the grouped
// GEMMs on the matrix cores, which measured faster than the bucketed GEMVs
// from 2 tokens up (80B shape, 4- and 8-bit experts) even with a handful of
// tokens per bucket; the bucketed GEMVs where the GEMM tiles do not fit
// (d not a multiple of 128) and for unquantised f32 experts.
int resolve_path(int path, int T, int d, int k, int E, int bits, int Imax) {
  if (path != MOE_PATH_AUTO) return path;
  if (T <= 8 && (long)T * (k + 1) <= 2048) return MOE_PATH_DECODE;
  return (d % 128 == 0 && bits != 32 && prefill_fits(T, d, k, Imax)) ? MOE_PATH_PREFILL : MOE_PATH_BATCHED;
}

bool prefill_fits(int T, int d, int k, int Imax) {
  const uint64_t lim = (uint64_t)1 << 32;
  return (uint64_t)T * (uint64_t)d * 2 < lim && ((uint64_t)T * (uint64_t)k + (uint64_t)T) * (uint64_t)Imax * 2 < lim;
}

size_t ffn_ws_bytes(int d, int I, int Ish, int T, int k, int E, int path) {
  if (is_mfma_path(path))
    return prefill_fits(T, d, k, I > Ish ? I : Ish) ? prefill_ws_bytes(d, I, Ish, T, k, E) : 0;
  Carver c(nullptr, (size_t)-1);
  FfnWs w;
  carve_ffn(c, d, I > Ish ? I : Ish, T, k, path, &w);
  return c.off + 256;
}

int xprep_launch(const uint16_t* x, int T, int d, uint32_t* xq, float* xs, hipStream_t s);

namespace {
// f32 experts: decode (routing given: no in-kernel selection) or bucketed.
int f32_launch(const FfnArgs& f, int path, GateUpArgs& g, DownArgs& dn, const FfnWs& w, int Imax,
               hipStream_t s) {
  if (path == MOE_PATH_DECODE) {
    if (f.logits) return MOE_ERR_UNSUPPORTED;
    g.batched = 0;
    g.logits = nullptr;
    const int items = f.T * f.k * (f.I / 4) + f.T * (f.Ish / 4);
    void* args[] = {&g};
    MOE_HIP(hipLaunchKernel((void*)gate_up_f32_kernel<1>, dim3((items + 7) & ~7), dim3(256), args,
                            (size_t)f.d * 2, s));
    const int nI = f.T * (f.k + 1);
    void* dargs[] = {&dn};
    const size_t dlds = (size_t)(((nI * 9 + 3) & ~3) + kDnRound * Imax) * 4;
    MOE_HIP(hipLaunchKernel((void*)down_decode_f32_kernel, dim3(f.d / 8), dim3(64 * kDnWaves), dargs, dlds, s));
    return MOE_OK;
  }
  if (!f.offsets || !f.pair_ids || !f.partial || !f.shared_out) return MOE_ERR_INVALID_ARG;
  const int nsh = (f.T + kTC - 1) / kTC;
  plan_kernel<<<1, 1024, 0, s>>>(f.offsets, f.pool.E, f.T, w.inst, w.n_routed);
  MOE_HIP(hipGetLastError());
  g.batched = 1;
  g.inst = w.inst; g.n_routed = w.n_routed; g.n_shared_inst = nsh; g.pair_ids = f.pair_ids;
  const long upper = ((long)f.T * f.k + nsh) * (Imax / 4);
  void* args[] = {&g};
  MOE_HIP(hipLaunchKernel((void*)gate_up_f32_kernel<kTC>, dim3(grid_for((int)(upper < 65536 ? upper : 65536))),
                          dim3(256), args, (size_t)kTC * f.d * 2, s));
  dn.inst = w.inst; dn.n_routed = w.n_routed; dn.n_shared_inst = nsh; dn.pair_ids = f.pair_ids;
  dn.partial = f.partial; dn.shared_out = f.shared_out;
  const long dupper = ((long)f.T * f.k + nsh) * ((f.d + 31) / 32);
  void* dargs[] = {&dn};
  MOE_HIP(hipLaunchKernel((void*)down_batched_f32_kernel, dim3(grid_for((int)(dupper < 65536 ? dupper : 65536))),
                          dim3(256), dargs, (size_t)kTC * Imax * 4, s));
  return MOE_OK;
}
}  // namespace

int ffn_launch(const FfnArgs& f, int path, void* ws, size_t ws_bytes, hipStream_t s) {
  // one code width for routed and shared experts (4-bit, 8-bit or f32)
  if (f.bits != f.bits_sh || (f.bits != 4 && f.bits != 8 && f.bits != 32)) return MOE_ERR_UNSUPPORTED;
  if (is_mfma_path(path)) {
    if (f.bits == 32) return MOE_ERR_UNSUPPORTED;   // f32 experts: decode and bucketed GEMVs
    return prefill_launch(f, path, ws, ws_bytes, s);
  }
  if (path != MOE_PATH_DECODE && path != MOE_PATH_BATCHED) return MOE_ERR_INVALID_ARG;
  const int Imax = f.I > f.Ish ? f.I : f.Ish;
  Carver c(ws, ws_bytes);
  FfnWs w;
  if (!carve_ffn(c, f.d, Imax, f.T, f.k, path, &w)) return MOE_ERR_INVALID_ARG;
  const uint32_t* xq = f.xq;
  const float* xs = f.xs;
  // decode without prepared pairs: the gate/up blocks form them from x
  if (!xq && f.bits != 32 && path != MOE_PATH_DECODE) {
    MOE_TRY(xprep_launch(f.x, f.T, f.d, w.xq, w.xs, s));
    xq = w.xq;
    xs = w.xs;
  }
  const int G = f.d / 64;
  const GemvSet kf = f.bits == 8 ? gemv_set<8>() : gemv_set<4>();
  GateUpArgs g{};
  g.pool = f.pool; g.shared_blob = f.shared_blob;
  g.d = f.d; g.I = f.I; g.Ish = f.Ish; g.Imax = Imax; g.T = f.T; g.k = f.k;
  g.idx = f.idx; g.w = f.w; g.sgate = f.sgate; g.logits = f.logits; g.bias = f.bias; g.usage = f.usage;
  g.sel_slot = w.sel_slot;
  g.xq = xq; g.xs = xs; g.x = f.x;
  g.hq = w.hq; g.hs8 = w.hs8;
  DownArgs dn{};
  dn.pool = f.pool; dn.shared_blob = f.shared_blob;
  dn.d = f.d; dn.I = f.I; dn.Ish = f.Ish; dn.Imax = Imax; dn.T = f.T; dn.k = f.k;
  dn.sel_slot = w.sel_slot; dn.w = f.w; dn.sgate = f.sgate; dn.hq = w.hq; dn.hs8 = w.hs8; dn.y = f.y;
  dn.res_in = f.res_in; dn.res_out = f.res_out; dn.ssp_out = f.ssp_out;
  if (f.res_out && (path != MOE_PATH_DECODE || f.bits == 32)) return MOE_ERR_INVALID_ARG;
  // two-phase decode: routing given, quantised experts, no hand-over in phase 1
  if (f.phase != 0 && (path != MOE_PATH_DECODE || f.bits == 32 || f.logits || f.phase < 0 || f.phase > 2 ||
                       (f.phase == 1 && f.res_out)))
    return MOE_ERR_INVALID_ARG;
  g.phase = f.phase; g.pend = w.pend;
  dn.phase = f.phase; dn.pend = w.pend; dn.oi_buf = w.oi_buf;

  if (f.bits == 32) return f32_launch(f, path, g, dn, w, Imax, s);
  if (path == MOE_PATH_DECODE) {
    g.batched = 0;
    const int items = f.T * f.k * (f.I / 8) + f.T * (f.Ish / 8);
    const int E = f.pool.E;
    const size_t lds = (size_t)1 * G * kXPad * 4 +
                       (f.logits ? (size_t)(topk_scratch_words(E) + E + 2 * f.k) * 4 : 0);
    void* fn = kf.gate_up(f.logits ? nk_for(E) : 1, G, xq == nullptr);   // no selection: the smallest instance
    void* args[] = {&g};
    if (f.phase != 2 || f.pending > 0)   // multiple of 8: xcd_remap
      MOE_HIP(hipLaunchKernel(fn, dim3((items + 7) & ~7), dim3(256), args, lds, s));
    const int nI = f.T * (f.k + 1);
    void* dargs[] = {&dn};
    const size_t dlds = (size_t)(((nI * 9 + 3) & ~3) + kDnRound * hrec_words(Imax)) * 4;
    // the pipelined kernel when both record buffers fit the LDS (also for
    // one round: its DMA'd records measured faster than register staging)
    const size_t plds = (size_t)(((nI * 9 + f.T * f.k + 3) & ~3) + 2 * kDnRound * hrec_sw_words(Imax)) * 4;
    const bool pipe = plds <= 160 * 1024;
    if (f.phase == 2 && f.down_wait) MOE_HIP(hipStreamWaitEvent(s, f.down_wait, 0));
    MOE_HIP(hipLaunchKernel(pipe ? kf.down_decode_pipe() : kf.down_decode(), dim3(f.d / 8), dim3(64 * kDnWaves),
                            dargs, pipe ? plds : dlds, s));
    return MOE_OK;
  }
  // batched: bucketed instances of up to kTC tokens
  if (!f.offsets || !f.pair_ids || !f.partial || !f.shared_out) return MOE_ERR_INVALID_ARG;
  const int nsh = (f.T + kTC - 1) / kTC;
  plan_kernel<<<1, 1024, 0, s>>>(f.offsets, f.pool.E, f.T, w.inst, w.n_routed);
  MOE_HIP(hipGetLastError());
  g.batched = 1;
  g.inst = w.inst; g.n_routed = w.n_routed; g.n_shared_inst = nsh; g.pair_ids = f.pair_ids;
  const long upper = ((long)f.T * f.k + nsh) * (Imax / 32);
  const size_t lds = ((size_t)kTC * G * kXPad + kTC * G + 4 * kTC * 8) * 4;
  void* gfn = kf.gate_up_batched(G);
  void* args[] = {&g};
  MOE_HIP(hipLaunchKernel(gfn, dim3(grid_for((int)(upper < 65536 ? upper : 65536))), dim3(256), args, lds, s));
  dn.inst = w.inst; dn.n_routed = w.n_routed; dn.n_shared_inst = nsh; dn.pair_ids = f.pair_ids;
  dn.partial = f.partial; dn.shared_out = f.shared_out;
  const int drows = f.bits == 8 ? 128 : 256;   // output rows per item (32 * kDnSub)
  const long dupper = ((long)f.T * f.k + nsh) * ((f.d + drows - 1) / drows);
  void* dargs[] = {&dn};
  MOE_HIP(hipLaunchKernel(kf.down_batched(), dim3(grid_for((int)(dupper < 65536 ? dupper : 65536))),
                          dim3(256), dargs, (size_t)kTC * hrec_words(Imax) * 4, s));
  return MOE_OK;
}

}  // namespace moe
