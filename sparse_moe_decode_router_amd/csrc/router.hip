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
// int4 GEMVs consume, and the fp32 sum of the group (column order).
__device__ void xprep_group(const uint16_t* __restrict__ x, int d, int t, int g,
                            uint32_t* __restrict__ xq, float* __restrict__ xs) {
  const uint4* src = reinterpret_cast<const uint4*>(x + (size_t)t * d + 64 * g);
  uint4* dst = reinterpret_cast<uint4*>(xq + (size_t)t * (d / 2) + 32 * g);
  float s = 0.0f;
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    uint4 v = src[q];
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
// prepare xq/xs.  No block waits for another.
struct DecodeArgs {
  const uint16_t* x; int T, d;
  const float* W; int E;
  float* logits; uint32_t* xq; float* xs;
};

template <int TMAX>
__global__ __launch_bounds__(kRouterThreads) void router_decode_kernel(DecodeArgs a) {
  __shared__ float red[4][TMAX];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = blockIdx.x;
  const int d = a.d, T = a.T, E = a.E;
  {
    const int G = d / 64;
    const int id = blockIdx.x * kRouterThreads + tid;
    if (id < T * G) xprep_group(a.x, d, id / G, id % G, a.xq, a.xs);
  }
  float acc[TMAX];
#pragma unroll
  for (int t = 0; t < TMAX; ++t) acc[t] = 0.0f;
  const float4* Wr = reinterpret_cast<const float4*>(a.W + (size_t)row * d);
  for (int c = tid; c < d / 4; c += kRouterThreads) {
    const float4 wv = Wr[c];
#pragma unroll
    for (int t = 0; t < TMAX; ++t) {
      if (t < T) {
        const uint2 xv = *reinterpret_cast<const uint2*>(a.x + (size_t)t * d + 4 * c);
        acc[t] += wv.x * bf16_lo(xv.x);
        acc[t] += wv.y * bf16_hi(xv.x);
        acc[t] += wv.z * bf16_lo(xv.y);
        acc[t] += wv.w * bf16_hi(xv.y);
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

// ---------------------------------------------------------- batched router
// logits[t][e] for T > 8: 64x64 output tiles, K tiles of 32 staged in LDS.
// Each K tile is summed on its own (depth 32) before joining the running
// total (depth d/32): depth 32 + d/32, plus one for the bias.
__global__ __launch_bounds__(256) void router_gemm_kernel(const uint16_t* __restrict__ x, int T, int d,
                                                          const float* __restrict__ W, int R,
                                                          float* __restrict__ logits) {
  __shared__ float As[32][64 + 4];
  __shared__ float Bs[32][64 + 4];
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < d; k0 += 32) {
    {  // x tile: 64 tokens x 32 cols, 8 bf16 per thread
      const int m = tid >> 2, c8 = (tid & 3) * 8;
      uint4 v = make_uint4(0, 0, 0, 0);
      if (m0 + m < T) v = *reinterpret_cast<const uint4*>(x + (size_t)(m0 + m) * d + k0 + c8);
      As[c8 + 0][m] = bf16_lo(v.x); As[c8 + 1][m] = bf16_hi(v.x);
      As[c8 + 2][m] = bf16_lo(v.y); As[c8 + 3][m] = bf16_hi(v.y);
      As[c8 + 4][m] = bf16_lo(v.z); As[c8 + 5][m] = bf16_hi(v.z);
      As[c8 + 6][m] = bf16_lo(v.w); As[c8 + 7][m] = bf16_hi(v.w);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {  // W tile: 64 rows x 32 cols
      const int idx = tid + 256 * h;
      const int n = idx >> 3, c4 = (idx & 7) * 4;
      float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
      if (n0 + n < R) v = *reinterpret_cast<const float4*>(W + (size_t)(n0 + n) * d + k0 + c4);
      Bs[c4 + 0][n] = v.x; Bs[c4 + 1][n] = v.y; Bs[c4 + 2][n] = v.z; Bs[c4 + 3][n] = v.w;
    }
    __syncthreads();
    float part[4][4] = {};
#pragma unroll 8
    for (int kk = 0; kk < 32; ++kk) {
      float av[4], bv[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = As[kk][ty * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i) bv[i] = Bs[kk][tx * 4 + i];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) part[i][jj] += av[i] * bv[jj];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int jj = 0; jj < 4; ++jj) acc[i][jj] += part[i][jj];
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int m = m0 + ty * 4 + i;
    if (m >= T) continue;
#pragma unroll
    for (int jj = 0; jj < 4; ++jj) {
      const int n = n0 + tx * 4 + jj;
      if (n < R) logits[(size_t)m * R + n] = acc[i][jj];
    }
  }
}

template <int NK>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ logits, const float* __restrict__ bias,
                                                   int T, int E, int k, int32_t* __restrict__ idx,
                                                   float* __restrict__ w, float* __restrict__ sgate,
                                                   uint32_t* __restrict__ usage) {
  extern __shared__ uint32_t dyn_lds[];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + wave;
  if (t >= T) return;
  const int k4 = (k + 3) & ~3;
  uint32_t* base = dyn_lds + wave * (2 * k4 + topk_scratch_words(E));
  float* sel_l = reinterpret_cast<float*>(base);
  int32_t* sel_e = reinterpret_cast<int32_t*>(base + k4);
  const float* lrow = logits + (size_t)t * (E + 1);
  topk_select<NK>(lrow, bias, E, k, sel_l, sel_e, base + 2 * k4);
  topk_finish(sel_l, sel_e, k, idx + (size_t)t * k, w + (size_t)t * k, usage);
  if (lane == 0 && sgate) sgate[t] = sigmoidf_(lrow[E]);
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
  ws->ticket = c.take<uint32_t>(64);
  ws->logits = c.take<float>((size_t)T * (E + 1));
  ws->xq = c.take<uint32_t>((size_t)T * d / 2);
  ws->xs = c.take<float>((size_t)T * d / 64);
  return c.ok();
}

int router_logits_launch(const uint16_t* x, int T, int d, const float* W, int E, const RouterWs& ws,
                         hipStream_t s) {
  if (T == 0) return MOE_OK;
  if (T <= 8) {
    DecodeArgs a{x, T, d, W, E, ws.logits, ws.xq, ws.xs};
    void* fn = T == 1 ? (void*)router_decode_kernel<1> : T == 2 ? (void*)router_decode_kernel<2>
             : T <= 4 ? (void*)router_decode_kernel<4> : (void*)router_decode_kernel<8>;
    void* args[] = {&a};
    MOE_HIP(hipLaunchKernel(fn, dim3(E + 1), dim3(kRouterThreads), args, 0, s));
    return MOE_OK;
  }
  MOE_TRY(xprep_launch(x, T, d, ws.xq, ws.xs, s));
  router_gemm_kernel<<<dim3((E + 1 + 63) / 64, (T + 63) / 64), 256, 0, s>>>(x, T, d, W, E + 1, ws.logits);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

int topk_launch(const float* logits, const float* bias, int T, int E, int k, int32_t* idx, float* w,
                float* sgate, uint32_t* usage, hipStream_t s) {
  if (T == 0) return MOE_OK;
  const size_t lds = (size_t)4 * (2 * ((k + 3) & ~3) + topk_scratch_words(E)) * 4;
  const dim3 tg((T + 3) / 4);
  switch (nk_for(E)) {
    case 1: topk_kernel<1><<<tg, 256, lds, s>>>(logits, bias, T, E, k, idx, w, sgate, usage); break;
    case 2: topk_kernel<2><<<tg, 256, lds, s>>>(logits, bias, T, E, k, idx, w, sgate, usage); break;
    case 4: topk_kernel<4><<<tg, 256, lds, s>>>(logits, bias, T, E, k, idx, w, sgate, usage); break;
    case 8: topk_kernel<8><<<tg, 256, lds, s>>>(logits, bias, T, E, k, idx, w, sgate, usage); break;
    default: topk_kernel<16><<<tg, 256, lds, s>>>(logits, bias, T, E, k, idx, w, sgate, usage); break;
  }
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

int router_launch(const uint16_t* x, int T, int d, const float* W, const float* bias, int E,
                  int k, int32_t* idx, float* w, float* sgate, uint32_t* usage,
                  const RouterWs& ws, hipStream_t s) {
  MOE_TRY(router_logits_launch(x, T, d, W, E, ws, s));
  return topk_launch(ws.logits, bias, T, E, k, idx, w, sgate, usage, s);
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_router_workspace_bytes(int32_t T, int32_t d, int32_t E) {
  if (T < 0 || d <= 0 || E <= 0) return 0;
  return router_ws_bytes(T, d, E);
}

extern "C" int32_t moe_router_sum_depth(int32_t T, int32_t d) {
  if (d <= 0) return -1;
  return T <= 8 ? d / 256 + 9 : 32 + d / 32 + 1;
}

extern "C" int moe_router_topk(const uint16_t* x, int32_t T, int32_t d, const float* W,
                               const float* bias, int32_t E, int32_t k, int32_t* idx, float* w,
                               float* sgate, uint32_t* usage, void* ws, size_t ws_bytes,
                               hipStream_t s) {
  MOE_CHECK(T >= 0 && d > 0 && d % 64 == 0 && d <= 8192);
  MOE_CHECK(E >= 1 && E <= 1024 && k >= 1 && k <= E);
  if (T == 0) return MOE_OK;
  MOE_CHECK(x && W && idx && w && ws);
  MOE_CHECK(aligned(x, 16) && aligned(W, 16) && aligned(ws, 256));
  Carver c(ws, ws_bytes);
  RouterWs rw;
  if (!router_ws_carve(c, T, d, E, &rw)) return MOE_ERR_INVALID_ARG;
  return router_launch(x, T, d, W, bias, E, k, idx, w, sgate, usage, rw, s);
}
