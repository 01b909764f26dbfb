// Router: logits, top-k selection, renormalised weights, shared-expert gate,
// usage counters (Swiftlet pages, "How it works": every token goes to k of E
// experts; the router is a resident dense weight).
//
// Selection is integer work on 64-bit keys (order-preserving fp32 logit bits
// in the high word, bit-inverted expert index in the low word), so equal
// logits go to the lower index and the rank order is logit descending, index
// ascending.  Weights are the softmax over the k chosen logits.
#include "internal.h"
#include "device.h"
#include "topk.h"

namespace moe {
namespace {

constexpr int kRouterThreads = 256;

// ---------------------------------------------------------------- x prep
// One (token, group of 64 columns): the bf16 pairs (x[8m+i], x[8m+i+4]) the
// int4 GEMVs consume, and the fp32 sum of the group (column order).  The
// group's eight loads are all issued before the first store.
__device__ void xprep_group(const uint16_t* __restrict__ x, int d, int t, int g,
                            uint32_t* __restrict__ xq, float* __restrict__ xs) {
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * d + 64 * g);
  uint4* dst = reinterpret_cast<uint4*>(xq + (size_t)t * (d / 2) + 32 * g);
  float s = 0.0f;
  uint4 vv[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) vv[q] = src[q];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 v = vv[q];
    uint4 p;
    p.x = (v.x & 0xFFFFu) | (v.z << 16);
    p.y = (v.x >> 16) | (v.z & 0xFFFF0000u);
    p.z = (v.y & 0xFFFFu) | (v.w << 16);
    p.w = (v.y >> 16) | (v.w & 0xFFFF0000u);
    dst[q] = p;
    s += bf16_lo(v.x); s += bf16_hi(v.x);
    s += bf16_lo(v.y); s += bf16_hi(v.y);
    s += bf16_lo(v.z); s += bf16_hi(v.z);
    s += bf16_lo(v.w); s += bf16_hi(v.w);
  }
  xs[(size_t)t * (d / 64) + g] = s;
}

// The same group of u = bf16(x * scale) (a chain's normalised layer input).
__device__ __forceinline__ uint32_t scaled_bf16(uint32_t xbits16, float scale) {
  return f32_to_bf16(__uint_as_float(xbits16 << 16) * scale);
}
__device__ void xprep_group_scaled(const uint16_t* __restrict__ x, float scale, int d, int t, int g,
                                   uint32_t* __restrict__ xq, float* __restrict__ xs) {
  const uint16_t* src = x + (size_t)t * d + 64 * g;
  uint4* dst = reinterpret_cast<uint4*>(xq + (size_t)t * (d / 2) + 32 * g);
  float s = 0.0f;
  uint4 vv[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) vv[q] = reinterpret_cast<const uint4*>(src)[q];   // all loads first
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const uint4 v = vv[q];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t e[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      e[2 * i] = scaled_bf16(w[i] & 0xFFFFu, scale);
      e[2 * i + 1] = scaled_bf16(w[i] >> 16, scale);
    }
    uint4 p;
    p.x = e[0] | (e[4] << 16);
    p.y = e[1] | (e[5] << 16);
    p.z = e[2] | (e[6] << 16);
    p.w = e[3] | (e[7] << 16);
    dst[q] = p;
#pragma unroll
    for (int i = 0; i < 8; ++i) s += __uint_as_float(e[i] << 16);
  }
  xs[(size_t)t * (d / 64) + g] = s;
}

__global__ __launch_bounds__(256) void xprep_kernel(const uint16_t* __restrict__ x, int T, int d,
                                                    uint32_t* __restrict__ xq, float* __restrict__ xs) {
  const int G = d / 64;
  const int id = blockIdx.x * blockDim.x + threadIdx.x;
  if (id < T * G) xprep_group(x, d, id / G, id % G, xq, xs);
}

}  // namespace

namespace {

// --------------------------------------------------------- decode router
// Logits for T <= TMAX tokens.  Block b computes logit row b (row E is the
// shared gate) with 256 threads, each summing d/256 products in column
// order, then a 64-lane butterfly and a two-level tree over the 4 waves:
// depth d/256 + 8, plus one for the bias (added by the top-k).  Blocks also
// prepare xq/xs, group q by thread (q / gridDim) % 256 of block q % gridDim
// (one group per block while T d / 64 <= E + 1).  No block waits for
// another.
struct DecodeArgs {
  const uint16_t* x; int T, d;
  const float* W; int E;
  float* logits; uint32_t* xq; float* xs;
  const float* ssp;             // chains: [T][d/8] partial sums of squares of x (or null)
  float eps;
};

template <int TMAX>
__global__ __launch_bounds__(kRouterThreads) void router_decode_kernel(DecodeArgs a) {
  __shared__ float red[4][TMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const int d = a.d, T = a.T, E = a.E;
  const bool chain = a.ssp != nullptr;
  const float4* Wr = reinterpret_cast<const float4*>(a.W + (size_t)row * d);
  // kRU pieces of 4 columns per thread a step.  The first step's weight and
  // activation loads (all of the row's for d <= 2048) go out first: the
  // chain's scale (a reduction of loaded partials) and the activation
  // preparation (loads, then stores that later loads may not pass) would
  // otherwise sit in front of them.
  constexpr int kRU = 2;
  float4 w_first[kRU];
  uint2 x_first[kRU][TMAX];
#pragma unroll
  for (int u = 0; u < kRU; ++u) {
    const int c = tid + u * kRouterThreads;
    const int cc = c < d / 4 ? c : 0;            // clamped: unconditional loads
    w_first[u] = Wr[cc];
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
      x_first[u][t] = *reinterpret_cast<const uint2*>(a.x + (size_t)(t < T ? t : 0) * d + 4 * cc);
  }
  float scale[TMAX];
  if (chain) {
    // x is a chain's residual stream: every block forms the same scale from
    // the partial sums of squares, added up in the same order as the chain
    // glue kernel adds its own (per-thread groups tid, tid + 256, ...; wave
    // butterfly; (w0 + w1) + (w2 + w3))
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      float ss = 0.f;
      if (t < T) {
        // d <= 8192: at most four partials per thread, all loads in flight at once
        float pv[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int g = tid + u * kRouterThreads;
          pv[u] = a.ssp[(size_t)t * (d / 8) + (g < d / 8 ? g : 0)];   // clamped: unconditional loads
        }
#pragma unroll
        for (int u = 0; u < 4; ++u)
          if (tid + u * kRouterThreads < d / 8) ss += pv[u];
      }
      ss = wave_sum(ss);
      if (lane == 0) red[wave][t] = ss;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < TMAX; ++t)
      scale[t] = 1.0f / sqrtf(((red[0][t] + red[1][t]) + (red[2][t] + red[3][t])) / (float)d + a.eps);
    __syncthreads();
  }
  {
    const int G = d / 64;
    // grid-stride: a grid of fewer than T d / 64 / 256 blocks (few experts,
    // wide d) still prepares every group
    for (int id = tid * gridDim.x + blockIdx.x; id < T * G; id += kRouterThreads * gridDim.x) {
      const int t = id / G;
      if (chain) {
        float sc = 1.f;
#pragma unroll
        for (int q = 0; q < TMAX; ++q)
          if (q == t) sc = scale[q];
        xprep_group_scaled(a.x, sc, d, t, id % G, a.xq, a.xs);
      } else {
        xprep_group(a.x, d, t, id % G, a.xq, a.xs);
      }
    }
  }
  float acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.0f;
  // a step's weight and activation loads are all issued before its first
  // product (a plain strided loop would wait for each piece's loads before
  // issuing the next); columns are still added in the order c = tid, tid +
  // 256, ...
  for (int c0 = tid; c0 < d / 4; c0 += kRU * kRouterThreads) {
    float4 wv[kRU];
    uint2 xv[kRU][TMAX];
#pragma unroll
    for (int u = 0; u < kRU; ++u) {
      const int c = c0 + u * kRouterThreads;
      const bool ok = c < d / 4;
      const int cc = ok ? c : 0;                 // clamped: unconditional loads
      wv[u] = c0 == tid ? w_first[u] : Wr[cc];
#pragma unroll
      for (int t = 0; t < TMAX; ++t)
        xv[u][t] = c0 == tid ? x_first[u][t]
                             : *reinterpret_cast<const uint2*>(a.x + (size_t)(t < T ? t : 0) * d + 4 * cc);
    }
#pragma unroll
    for (int u = 0; u < kRU; ++u) {
      if (c0 + u * kRouterThreads >= d / 4) continue;
#pragma unroll
      for (int t = 0; t < TMAX; ++t) {
        if (t < T) {
          uint2 x2 = xv[u][t];
          if (chain)
            x2 = make_uint2(scaled_bf16(x2.x & 0xFFFFu, scale[t]) | (scaled_bf16(x2.x >> 16, scale[t]) << 16),
                            scaled_bf16(x2.y & 0xFFFFu, scale[t]) | (scaled_bf16(x2.y >> 16, scale[t]) << 16));
          acc[t] += wv[u].x * bf16_lo(x2.x);
          acc[t] += wv[u].y * bf16_hi(x2.x);
          acc[t] += wv[u].z * bf16_lo(x2.y);
          acc[t] += wv[u].w * bf16_hi(x2.y);
        }
      }
    }
  }
#pragma unroll
  for (int t = 0; t < TMAX; ++t) {
    const float v = wave_sum(acc[t]);
    if (lane == 0) red[wave][t] = v;
  }
  __syncthreads();
  if (tid < T) a.logits[(size_t)tid * (E + 1) + row] = (red[0][tid] + red[1][tid]) + (red[2][tid] + red[3][tid]);
}

// ------------------------------------------------------ MFMA router (T > 8)
// fp32 router rows split into three bf16 parts (hi, mid, lo: hi + mid + lo
// carries the fp32 significand); x is exactly bf16, so every product on the
// matrix cores is exact in fp32.  Each 32-wide K step starts fresh
// accumulators (<= 32 additions) that are folded into a running fp32 sum
// (d/(32 S) additions), so the summation depth stays near a plain tiled GEMM:
// 32 + 2 + d/(32 S) per split, plus S-1 for the fixed-order sum of the S
// split-K partials in the top-k kernel, plus one for the bias.
//
// Block: 128 tokens x 64 router rows, 8 waves of 32 x 32; k advances 64 at a
// time (two of the 32-wide steps) through one LDS stage.  The x and fp32 W
// pieces of the stages after it are loaded into registers, two stages ahead,
// while the matrix cores work on the current one, and split and stored once
// every wave has read it: the router weights are split as they are staged
// (no separate pass over W).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Two weights a, b as bf16 parts hi + mid + lo, each the bf16 rounding (to
// nearest even, the hardware's packed conversion) of what is left; the pairs
// are packed with a in the low half.
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2(float p, float q) {
  const bf16x2_t v = {(__bf16)p, (__bf16)q};
  return __builtin_bit_cast(uint32_t, v);
}
__device__ __forceinline__ void split3x2(float a, float b, uint32_t& hi, uint32_t& mid, uint32_t& lo) {
  hi = bf16x2(a, b);
  const float a1 = a - bf16_lo(hi), b1 = b - bf16_hi(hi);
  mid = bf16x2(a1, b1);
  const float a2 = a1 - bf16_lo(mid), b2 = b1 - bf16_hi(mid);
  lo = bf16x2(a2, b2);
}

constexpr int kRtM = 128, kRtN = 64, kRtK = 64, kRtLds = 72;   // block tile, k per stage, LDS row (bf16)

__global__ __launch_bounds__(512) void router_mfma_kernel(const uint16_t* __restrict__ x, int T, int d,
                                                          const float* __restrict__ W, int R,
                                                          int S, float* __restrict__ part) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[kRtM * kRtLds];
  __shared__ __attribute__((aligned(16))) uint16_t ws[3][kRtN * kRtLds];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // Workgroups go to the 8 XCDs in turn; each XCD takes a contiguous range of
  // tiles, ordered (split, token tile, row tile), so the row tiles of one
  // token tile share its x rows in one L2 and one split's W columns stay there
  const int nt = (R + kRtN - 1) / kRtN, mt = (T + kRtM - 1) / kRtM;
  const int G = gridDim.x, tile = (blockIdx.x & 7) * (G >> 3) + (blockIdx.x >> 3);
  if (tile >= nt * mt * S) return;               // grid padded to a multiple of 8
  const int m0 = (tile / nt) % mt * kRtM, n0 = tile % nt * kRtN, sp = tile / (nt * mt);
  const int kspan = d / S, kbeg = sp * kspan, kend = kbeg + kspan;
  const int wm = 32 * (wave & 3), wn = 32 * (wave >> 2);
  // this thread's pieces of a stage, two of each: x row xr (8 bf16 at column
  // 8 xq), W row wr (4 fp32 at column 4 wq), read through buffer resources
  // over the block's own rows (fixed offsets, the k position a scalar).  Rows
  // past T or R read as zeros; they would feed only outputs that are never
  // stored (an MFMA output row depends on its A row alone, a column on its B
  // row).
  const rsrc_t rX = make_rsrc(x + (size_t)m0 * d, (uint32_t)(min(kRtM, T - m0) * d * 2));
  const rsrc_t rW = make_rsrc(W + (size_t)n0 * d, (uint32_t)(min(kRtN, R - n0) * d * 4));
  uint32_t xv[2], wv[2];
  int xo[2], wo[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const int id = tid + 512 * u;
    const int xr = id >> 3, xq = id & 7, wr = id >> 4, wq = id & 15;
    xv[u] = (uint32_t)(xr * d + 8 * xq) * 2;
    wv[u] = (uint32_t)(wr * d + 4 * wq) * 4;
    xo[u] = xr * kRtLds + 8 * xq;
    wo[u] = wr * kRtLds + 4 * wq;
  }
  struct Piece {
    u32x4 x[2];
    u32x4 w[2];
  };
  auto load = [&](Piece& pc, int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      pc.x[u] = __builtin_amdgcn_raw_buffer_load_b128(rX, xv[u], (uint32_t)k0 * 2, 0);
      pc.w[u] = __builtin_amdgcn_raw_buffer_load_b128(rW, wv[u], (uint32_t)k0 * 4, 0);
    }
  };
  auto store = [&](const Piece& pc) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      *reinterpret_cast<u32x4*>(&xs[xo[u]]) = pc.x[u];
      const float4 f = make_float4(__uint_as_float(pc.w[u].x), __uint_as_float(pc.w[u].y),
                                   __uint_as_float(pc.w[u].z), __uint_as_float(pc.w[u].w));
      uint32_t p[3][2];
      split3x2(f.x, f.y, p[0][0], p[1][0], p[2][0]);
      split3x2(f.z, f.w, p[0][1], p[1][1], p[2][1]);
#pragma unroll
      for (int j = 0; j < 3; ++j) *reinterpret_cast<uint2*>(&ws[j][wo[u]]) = make_uint2(p[j][0], p[j][1]);
    }
  };
  float run[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) run[i] = 0.f;
  // one stage of MFMAs from LDS: two 32-wide steps, fresh accumulators each
  auto mma = [&]() {
#pragma unroll
    for (int h2 = 0; h2 < 2; ++h2) {
      f32x16_t acc[3];
#pragma unroll
      for (int j = 0; j < 3; ++j)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[j][i] = 0.f;
#pragma unroll
      for (int kh = 0; kh < 2; ++kh) {
        const int col = 32 * h2 + 16 * kh + 8 * (lane >> 5);
        const bf16x8_t av = *reinterpret_cast<const bf16x8_t*>(&xs[(wm + (lane & 31)) * kRtLds + col]);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          const bf16x8_t bv = *reinterpret_cast<const bf16x8_t*>(&ws[j][(wn + (lane & 31)) * kRtLds + col]);
          acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc[j], 0, 0, 0);
        }
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) run[i] += (acc[0][i] + acc[1][i]) + acc[2][i];
    }
  };
  // stages two ahead in registers (pa, pb in turn): the loads of stage t + 2
  // are issued before stage t's MFMAs, stage t + 1 is stored after them
  Piece pa, pb;
  load(pa, kbeg);
  if (kbeg + kRtK < kend) load(pb, kbeg + kRtK);
  store(pa);
  __syncthreads();
  for (int k0 = kbeg; k0 < kend; k0 += 2 * kRtK) {
    if (k0 + 2 * kRtK < kend) load(pa, k0 + 2 * kRtK);
    mma();
    __syncthreads();                             // every wave is done with the stage
    if (k0 + kRtK >= kend) break;
    store(pb);
    __syncthreads();
    if (k0 + 3 * kRtK < kend) load(pb, k0 + 3 * kRtK);
    mma();
    __syncthreads();
    if (k0 + 2 * kRtK >= kend) break;
    store(pa);
    __syncthreads();
  }
  float* out = part + (size_t)sp * T * R;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const int m = m0 + wm + (i >> 2) * 8 + (lane >> 5) * 4 + (i & 3);
    const int n = n0 + wn + (lane & 31);
    if (m < T && n < R) out[(size_t)m * R + n] = run[i];
  }
}

// split-K count for T > 8: the smallest power of two (<= 8) that gives the
// launch about 1024 blocks of 128 tokens x 64 rows (at E = 512: 8 below 128
// tokens, 4 at 4096 tokens); every split spans a multiple of 64 columns (d is
// a multiple of 64), whole stages of the MFMA kernel
int router_splits(int T, int d, int E) {
  const long tiles = (long)((E + 1 + kRtN - 1) / kRtN) * ((T + kRtM - 1) / kRtM);
  int S = 1;
  while (S < 8 && tiles * S < 1024) S *= 2;
  while (S > 1 && (d / kRtK) % S != 0) S /= 2;
  return S;
}

// One wave per token.  With S > 1 the logits arrive as S split-K partials
// [S][T][E+1], summed here in split order before the selection.
// logits_out (optional, [T][E+1]): the logits the selection reads (the
// split-K sum where S > 1, before the bias), copied out unchanged.
template <int NK>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, int S,
                                                   const float* __restrict__ bias,
                                                   int T, int E, int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ w, float* __restrict__ sgate,
                                                   uint32_t* __restrict__ usage,
                                                   float* __restrict__ logits_out) {
  extern __shared__ uint32_t dyn_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int k4 = (k + 3) & ~3;
  const int stride = 2 * k4 + topk_scratch_words(E) + ((E + 1 + 3) & ~3);
  uint32_t* base = dyn_lds + wave * stride;
  float* sel_l = reinterpret_cast<float*>(base);
  int32_t* sel_e = reinterpret_cast<int32_t*>(base + k4);
  uint32_t* scr = base + 2 * k4;
  float* lsum = reinterpret_cast<float*>(scr + topk_scratch_words(E));
  const size_t TR = (size_t)T * (E + 1);
  const float* row = logits + (size_t)t * (E + 1);
  if (S > 1) {
    // every partial of this lane's logits in flight at once (S <= 8), then
    // summed in split order
    constexpr int kMaxS = 8;
    float pv[NK + 1][kMaxS];
#pragma unroll
    for (int j = 0; j <= NK; ++j) {
      const int ec = min(lane + 64 * j, E);
#pragma unroll
      for (int q = 0; q < kMaxS; ++q) pv[j][q] = row[ec + (size_t)min(q, S - 1) * TR];
    }
#pragma unroll
    for (int j = 0; j <= NK; ++j) {
      float v = pv[j][0];
#pragma unroll
      for (int q = 1; q < kMaxS; ++q)
        if (q < S) v += pv[j][q];
      if (lane + 64 * j <= E) lsum[lane + 64 * j] = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    row = lsum;
  }
  if (logits_out) {
    for (int e = lane; e <= E; e += 64) logits_out[(size_t)t * (E + 1) + e] = row[e];
  }
  // one partial: the selection reads the logits where they are (its loads
  // are all issued before any use)
  topk_select<NK>(row, bias, E, k, sel_l, sel_e, scr);
  topk_finish(sel_l, sel_e, k, idx + (size_t)t * k, w + (size_t)t * k, usage);
  if (lane == 0 && sgate) sgate[t] = sigmoidf_(row[E]);
}

}  // namespace

int xprep_launch(const uint16_t* x, int T, int d, uint32_t* xq, float* xs, hipStream_t s) {
  const int G = d / 64;
  if (T * G == 0) return MOE_OK;
  xprep_kernel<<<(T * G + 255) / 256, 256, 0, s>>>(x, T, d, xq, xs);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

size_t router_ws_bytes(int T, int d, int E) {
  Carver c(nullptr, (size_t)-1);
  RouterWs ws;
  router_ws_carve(c, T, d, E, &ws);
  return c.off + 256;
}

bool router_ws_carve(Carver& c, int T, int d, int E, RouterWs* ws) {
  ws->logits = c.take<float>((size_t)(T <= 8 ? 1 : router_splits(T, d, E)) * T * (E + 1));
  ws->xq = c.take<uint32_t>((size_t)T * d / 2);
  ws->xs = c.take<float>((size_t)T * d / 64);
  return c.ok();
}

int router_logits_launch(const uint16_t* x, int T, int d, const float* W, int E, const RouterWs& ws,
                         hipStream_t s, bool prep_x, const float* ssp, float eps) {
  if (T == 0) return MOE_OK;
  if (ssp && T > 8) return MOE_ERR_INVALID_ARG;
  if (T <= 8) {
    DecodeArgs a{x, T, d, W, E, ws.logits, ws.xq, ws.xs, ssp, eps};
    void* fn = T == 1 ? (void*)router_decode_kernel<1> : T == 2 ? (void*)router_decode_kernel<2>
             : T <= 4 ? (void*)router_decode_kernel<4> : (void*)router_decode_kernel<8>;
    void* args[] = {&a};
    MOE_HIP(hipLaunchKernel(fn, dim3(E + 1), dim3(kRouterThreads), args, 0, s));
    return MOE_OK;
  }
  if (prep_x) MOE_TRY(xprep_launch(x, T, d, ws.xq, ws.xs, s));
  const int R = E + 1, S = router_splits(T, d, E);
  const int tiles = ((R + kRtN - 1) / kRtN) * ((T + kRtM - 1) / kRtM) * S;
  router_mfma_kernel<<<(unsigned)((tiles + 7) & ~7), 512, 0, s>>>(x, T, d, W, R, S, ws.logits);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

int topk_launch(const float* logits, const float* bias, int T, int d, int E, int k, int32_t* idx, float* w,
                float* sgate, uint32_t* usage, hipStream_t s, float* logits_out) {
  if (T == 0) return MOE_OK;
  const int S = T <= 8 ? 1 : router_splits(T, d, E);
  const size_t lds = (size_t)4 * (2 * ((k + 3) & ~3) + topk_scratch_words(E) + ((E + 1 + 3) & ~3)) * 4;
  const dim3 tg((T + 3) / 4);
  switch (nk_for(E)) {
    case 1: topk_kernel<1><<<tg, 256, lds, s>>>(logits, S, bias, T, E, k, idx, w, sgate, usage, logits_out); break;
    case 2: topk_kernel<2><<<tg, 256, lds, s>>>(logits, S, bias, T, E, k, idx, w, sgate, usage, logits_out); break;
    case 4: topk_kernel<4><<<tg, 256, lds, s>>>(logits, S, bias, T, E, k, idx, w, sgate, usage, logits_out); break;
    case 8: topk_kernel<8><<<tg, 256, lds, s>>>(logits, S, bias, T, E, k, idx, w, sgate, usage, logits_out); break;
    default: topk_kernel<16><<<tg, 256, lds, s>>>(logits, S, bias, T, E, k, idx, w, sgate, usage, logits_out); break;
  }
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

int router_launch(const uint16_t* x, int T, int d, const float* W, const float* bias, int E,
                  int k, int32_t* idx, float* w, float* sgate, uint32_t* usage,
                  const RouterWs& ws, hipStream_t s, bool prep_x, float* logits_out) {
  MOE_TRY(router_logits_launch(x, T, d, W, E, ws, s, prep_x));
  return topk_launch(ws.logits, bias, T, d, E, k, idx, w, sgate, usage, s, logits_out);
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_router_workspace_bytes(int32_t T, int32_t d, int32_t E) {
  if (T < 0 || d <= 0 || E <= 0) return 0;
  return router_ws_bytes(T, d, E);
}

extern "C" int32_t moe_router_sum_depth(int32_t T, int32_t d, int32_t E) {
  if (d <= 0 || T < 0 || E < 1) return -1;
  if (T <= 8) return d / 256 + 9;
  const int S = router_splits(T, d, E);
  return 32 + 2 + d / (32 * S) + (S - 1) + 1;
}

extern "C" int moe_router_topk_logits(const uint16_t* x, int32_t T, int32_t d, const float* W,
                                      const float* bias, int32_t E, int32_t k, int32_t* idx, float* w,
                                      float* sgate, uint32_t* usage, float* logits_out, void* ws,
                                      size_t ws_bytes, hipStream_t s) {
  MOE_CHECK(T >= 0 && d > 0 && d % 64 == 0 && d <= 8192);
  MOE_CHECK(E >= 1 && E <= 1024 && k >= 1 && k <= E);
  if (T == 0) return MOE_OK;
  MOE_CHECK(x && W && idx && w && ws);
  MOE_CHECK(aligned(x, 16) && aligned(W, 16) && aligned(ws, 256));
  Carver c(ws, ws_bytes);
  RouterWs rw;
  if (!router_ws_carve(c, T, d, E, &rw)) return MOE_ERR_INVALID_ARG;
  return router_launch(x, T, d, W, bias, E, k, idx, w, sgate, usage, rw, s, false, logits_out);
}

extern "C" int moe_router_topk(const uint16_t* x, int32_t T, int32_t d, const float* W,
                               const float* bias, int32_t E, int32_t k, int32_t* idx, float* w,
                               float* sgate, uint32_t* usage, void* ws, size_t ws_bytes,
                               hipStream_t s) {
  return moe_router_topk_logits(x, T, d, W, bias, E, k, idx, w, sgate, usage, nullptr, ws, ws_bytes, s);
}
