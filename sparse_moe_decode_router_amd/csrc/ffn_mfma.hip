// Int4 expert FFN as grouped GEMMs on the matrix cores (prefill).
//
// With ~80 tokens per expert (4096 tokens, top-10 of 512) each expert's
// weights are a real dense contraction, so they run on MFMA
// (v_mfma_f32_32x32x16_f16, fp32 accumulate).  Experts are MLX affine int4
// group-quantised (relationship-to-TurboFieldfare section of the Swiftlet
// pages); SwiGLU and group 64 are this library's readings.
//
// Dequantisation: a code word's nibbles i and i+4 become the fp16 pair
// (1024+q_i, 1024+q_{i+4}) by OR-ing them into 0x6400 (fp16 1024.0 has a
// mantissa step of 1), a packed subtract gives q exactly, and one packed fma
// gives s*q + b rounded once to fp16 (11-bit significand: |rel err| <= 2^-11).
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
constexpr int kLdsRow = 40;     // fp16 per LDS row: 32 + 8 pad (80 B)

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

__device__ __forceinline__ void resolve_p(const PrefillArgs& a, int ii, bool routed, const uint8_t** blob,
                                          int* Iinst, bool* missing) {
  const PInst in = a.inst[ii];
  *missing = false;
  if (routed) {
    const int e = in.expert;
    const int slot = (e >= 0 && e < a.pool.E) ? a.pool.slot_table[e] : -1;
    *missing = slot < 0;
    *blob = a.pool.slab + (uint64_t)(slot < 0 ? 0 : slot) * a.pool.stride;
    *Iinst = a.I;
  } else {
    *blob = a.shared_blob;
    *Iinst = a.Ish;
  }
}

__global__ __launch_bounds__(256) void prefill_gate_up_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kPM * kLdsRow];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][kPM * kLdsRow];   // 64 gate + 64 up rows
  __shared__ int tok_s[kPM], hrow_s[kPM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nR = *a.n_routed;
  const int ntR = a.I / 64, ntS = a.Ish / 64;
  const int items = nR * ntR + a.n_shared_inst * ntS;
  const int C = a.d / 32;                       // k steps (blob chunks)
  const int lrow = tid >> 1, lhalf = tid & 1;   // loader: row, 16-column half

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const bool routed = item < nR * ntR;
    const int rel = routed ? item : item - nR * ntR;
    const int nt = routed ? ntR : ntS;
    const int ii = routed ? rel / nt : nR + rel / nt;
    const int o0 = (rel % nt) * 64;
    const uint8_t* blob;
    int Iinst;
    bool missing;
    resolve_p(a, ii, routed, &blob, &Iinst, &missing);
    const PInst in = a.inst[ii];
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
    const BlobLayout L = blob_layout(a.d, Iinst);
    // loader roles: A row lrow (token), B row lrow (0..63 gate, 64..127 up)
    const int my_tok = tok_s[lrow];
    const int mat = lrow >> 6;
    const uint64_t brow = (uint64_t)(o0 + (lrow & 63));
    const uint8_t* bcodes = blob + L.m[mat].codes;
    const uint8_t* bsb = blob + L.m[mat].sb;

    uint4 ra0, ra1;
    uint2 rb;
    uint32_t rsb;
    auto gload = [&](int c) {
      if (my_tok >= 0) {
        const uint4* src = reinterpret_cast<const uint4*>(a.xh + (size_t)my_tok * a.d + 32 * c + 16 * lhalf);
        ra0 = src[0];
        ra1 = src[1];
      } else {
        ra0 = make_uint4(0, 0, 0, 0);
        ra1 = ra0;
      }
      if (!missing) {
        rb = *reinterpret_cast<const uint2*>(bcodes + ((uint64_t)c * Iinst + brow) * 16 + 8 * lhalf);
        rsb = *reinterpret_cast<const uint32_t*>(bsb + ((uint64_t)(c >> 1) * Iinst + brow) * 4);
      } else {
        rb = make_uint2(0x88888888u, 0x88888888u);
        rsb = 0;
      }
    };
    auto lstore = [&](int buf) {
      _Float16* ad = &As[buf][lrow * kLdsRow + 16 * lhalf];
      *reinterpret_cast<uint4*>(ad) = ra0;
      *reinterpret_cast<uint4*>(ad + 8) = ra1;
      const half2_t s2 = __builtin_bit_cast(half2_t, (rsb & 0xFFFFu) * 0x10001u);
      const half2_t b2 = __builtin_bit_cast(half2_t, (rsb >> 16) * 0x10001u);
      _Float16* bd = &Bs[buf][lrow * kLdsRow + 16 * lhalf];
      *reinterpret_cast<uint4*>(bd) = dequant8(rb.x, s2, b2);
      *reinterpret_cast<uint4*>(bd + 8) = dequant8(rb.y, s2, b2);
    };

    float16_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
    const bool active = 32 * wave < in.n;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int c = 0; c < C; ++c) {
      const int buf = c & 1;
      if (c + 1 < C) gload(c + 1);
      if (active) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const half8_t av = *reinterpret_cast<const half8_t*>(
              &As[buf][(32 * wave + (lane & 31)) * kLdsRow + 16 * kh + 8 * (lane >> 5)]);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const half8_t bv = *reinterpret_cast<const half8_t*>(
                &Bs[buf][(32 * t + (lane & 31)) * kLdsRow + 16 * kh + 8 * (lane >> 5)]);
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[t], 0, 0, 0);
          }
        }
      }
      if (c + 1 < C) lstore(buf ^ 1);
      __syncthreads();
    }
    // epilogue: h = silu(g) * u (tiles 0/2 and 1/3 pair up), fp16, permuted
    if (active) {
      bool ovf = false;
#pragma unroll
      for (int half = 0; half < 2; ++half) {
        const int col = 32 * half + (lane & 31);
        const int o = o0 + col;
        const int po = (o & ~7) | (2 * (o & 3) + ((o >> 2) & 1));
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * wave + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
          if (r < in.n) {
            const float g = acc[half][i], u = acc[2 + half][i];
            const float h = missing ? 0.f : g / (1.0f + expf(-g)) * u;
            ovf |= !(fabsf(h) <= 65504.0f);
            a.hh[(size_t)hrow_s[r] * a.Imax + po] = __builtin_bit_cast(uint16_t, (_Float16)h);
          }
        }
      }
      if (ovf) atomicOr(a.pool.err, 2);
    }
    if (missing && tid == 0) atomicOr(a.pool.err, 1);
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void prefill_down_kernel(PrefillArgs a) {
  __shared__ __attribute__((aligned(16))) _Float16 As[2][kPM * kLdsRow];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[2][kPM * kLdsRow];   // 128 output rows
  __shared__ int hrow_s[kPM], tok_s[kPM];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int nR = *a.n_routed;
  const int nt = a.d / 128;
  const int items = (nR + a.n_shared_inst) * nt;
  const int lrow = tid >> 1, lhalf = tid & 1;

  for (int item = blockIdx.x; item < items; item += gridDim.x) {
    const int ii = item / nt;
    const int n0 = (item % nt) * 128;
    const bool routed = ii < nR;
    const uint8_t* blob;
    int Iinst;
    bool missing;
    resolve_p(a, ii, routed, &blob, &Iinst, &missing);
    const PInst in = a.inst[ii];
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
    const BlobLayout L = blob_layout(a.d, Iinst);
    const int C = Iinst / 32;
    const int my_h = hrow_s[lrow];
    const uint64_t brow = (uint64_t)(n0 + lrow);
    const uint8_t* bcodes = blob + L.m[2].codes;
    const uint8_t* bsb = blob + L.m[2].sb;

    uint4 ra0, ra1;
    uint2 rb;
    uint32_t rsb;
    auto gload = [&](int c) {
      if (my_h >= 0) {
        const uint4* src = reinterpret_cast<const uint4*>(a.hh + (size_t)my_h * a.Imax + 32 * c + 16 * lhalf);
        ra0 = src[0];
        ra1 = src[1];
      } else {
        ra0 = make_uint4(0, 0, 0, 0);
        ra1 = ra0;
      }
      if (!missing) {
        rb = *reinterpret_cast<const uint2*>(bcodes + ((uint64_t)c * a.d + brow) * 16 + 8 * lhalf);
        rsb = *reinterpret_cast<const uint32_t*>(bsb + ((uint64_t)(c >> 1) * a.d + brow) * 4);
      } else {
        rb = make_uint2(0x88888888u, 0x88888888u);
        rsb = 0;
      }
    };
    auto lstore = [&](int buf) {
      _Float16* ad = &As[buf][lrow * kLdsRow + 16 * lhalf];
      *reinterpret_cast<uint4*>(ad) = ra0;
      *reinterpret_cast<uint4*>(ad + 8) = ra1;
      const half2_t s2 = __builtin_bit_cast(half2_t, (rsb & 0xFFFFu) * 0x10001u);
      const half2_t b2 = __builtin_bit_cast(half2_t, (rsb >> 16) * 0x10001u);
      _Float16* bd = &Bs[buf][lrow * kLdsRow + 16 * lhalf];
      *reinterpret_cast<uint4*>(bd) = dequant8(rb.x, s2, b2);
      *reinterpret_cast<uint4*>(bd + 8) = dequant8(rb.y, s2, b2);
    };

    float16_t acc[4];
#pragma unroll
    for (int t = 0; t < 4; ++t)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[t][i] = 0.f;
    const bool active = 32 * wave < in.n;

    gload(0);
    lstore(0);
    __syncthreads();
    for (int c = 0; c < C; ++c) {
      const int buf = c & 1;
      if (c + 1 < C) gload(c + 1);
      if (active) {
#pragma unroll
        for (int kh = 0; kh < 2; ++kh) {
          const half8_t av = *reinterpret_cast<const half8_t*>(
              &As[buf][(32 * wave + (lane & 31)) * kLdsRow + 16 * kh + 8 * (lane >> 5)]);
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const half8_t bv = *reinterpret_cast<const half8_t*>(
                &Bs[buf][(32 * t + (lane & 31)) * kLdsRow + 16 * kh + 8 * (lane >> 5)]);
            acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_f16(av, bv, acc[t], 0, 0, 0);
          }
        }
      }
      if (c + 1 < C) lstore(buf ^ 1);
      __syncthreads();
    }
    if (active) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int n = n0 + 32 * t + (lane & 31);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int r = 32 * wave + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
          if (r < in.n) {
            const float v = missing ? 0.f : acc[t][i];
            if (routed) a.partial[(size_t)hrow_s[r] * a.d + n] = v;
            else a.shared_out[(size_t)tok_s[r] * a.d + n] = v;
          }
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
  const long chunks = ((long)f.T * f.k + kPM - 1) / kPM + f.pool.E + a.n_shared_inst;
  const long gu_items = chunks * (Imax / 64);
  const long dn_items = chunks * (f.d / 128);
  const int gu_grid = (int)(gu_items < 4096 ? gu_items : 4096);
  const int dn_grid = (int)(dn_items < 4096 ? dn_items : 4096);
  void* args[] = {&a};
  MOE_HIP(hipLaunchKernel((void*)prefill_gate_up_kernel, dim3(gu_grid), dim3(256), args, 0, s));
  MOE_HIP(hipLaunchKernel((void*)prefill_down_kernel, dim3(dn_grid), dim3(256), args, 0, s));
  return MOE_OK;
}

}  // namespace moe
