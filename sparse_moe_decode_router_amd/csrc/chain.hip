// A chain of MoE layers per token: several routed-expert layers applied one
// after the other (the pages' models stack dozens of them per token; their
// decode loop is bound by dispatch, not IO).  Each layer is a pre-norm
// residual block read without the attention half and without a learned norm
// weight:
//   u_l = bf16(x_l / sqrt(mean(x_l^2) + eps)),  x_{l+1} = bf16(x_l + MoE_l(u_l)),
// the residual add in fp32.  Decode layers of quantised experts hand the
// residual stream on inside their own launches (the down kernel adds the
// layer output and sums squares, the next router normalises); other layers
// take one glue launch each.  The whole chain goes on one stream, so a
// caller can capture it in a single HIP graph.
#include "internal.h"
#include "device.h"

namespace moe {
namespace {

constexpr int kGlueThreads = 256;

// One block per token.  y == nullptr: x_out = x (the first layer).  u_out ==
// nullptr: no normalisation (after the last layer).
constexpr int kGlueGroups = 8192 / 8 / kGlueThreads;   // groups of 8 elements per thread (d <= 8192)

// The sum of squares of a row in chain order: the row cut into groups of 8
// consecutive elements, each group summed as sq_tree8; thread tid adds the
// groups tid, tid + 256, ... in that order; then a wave butterfly and the
// four waves as (w0 + w1) + (w2 + w3).  The decode down kernel produces the
// same group sums (its 8 lanes per 8 output rows, sum8_dpp) and the decode
// router adds them up the same way, so a chain gives the same bits with or
// without this kernel between its layers.
__global__ __launch_bounds__(kGlueThreads) void chain_glue_kernel(const uint16_t* __restrict__ x,
                                                                  const float* __restrict__ y, int d, float eps,
                                                                  uint16_t* __restrict__ x_out,
                                                                  uint16_t* __restrict__ u_out) {
  __shared__ float red[kGlueThreads / 64];
  const int t = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const size_t base = (size_t)t * d;
  const int ng = d / 8;
  // all loads first; x_l kept in registers for the second pass
  float v[kGlueGroups][8];
#pragma unroll
  for (int j = 0; j < kGlueGroups; ++j) {
    const int g = tid + kGlueThreads * j;
#pragma unroll
    for (int i = 0; i < 8; ++i) v[j][i] = 0.f;
    if (g < ng) {
      const uint4 xv = reinterpret_cast<const uint4*>(x + base)[g];
      const uint32_t xw[4] = {xv.x, xv.y, xv.z, xv.w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        v[j][2 * i] = bf16_lo(xw[i]);
        v[j][2 * i + 1] = bf16_hi(xw[i]);
      }
      if (y) {
        const float4 y0 = reinterpret_cast<const float4*>(y + base)[2 * g];
        const float4 y1 = reinterpret_cast<const float4*>(y + base)[2 * g + 1];
        v[j][0] += y0.x; v[j][1] += y0.y; v[j][2] += y0.z; v[j][3] += y0.w;
        v[j][4] += y1.x; v[j][5] += y1.y; v[j][6] += y1.z; v[j][7] += y1.w;
      }
    }
  }
  float ss = 0.f;
#pragma unroll
  for (int j = 0; j < kGlueGroups; ++j) {
    const int g = tid + kGlueThreads * j;
    if (g < ng) {
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        b[i] = f32_to_bf16(v[j][i]);
        v[j][i] = __uint_as_float(b[i] << 16);
      }
      reinterpret_cast<uint4*>(x_out + base)[g] =
          make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
      ss += sq_tree8(v[j]);
    }
  }
  if (!u_out) return;
  ss = wave_sum(ss);
  if (lane == 0) red[wave] = ss;
  __syncthreads();
  const float tot = (red[0] + red[1]) + (red[2] + red[3]);
  const float scale = 1.0f / sqrtf(tot / (float)d + eps);
#pragma unroll
  for (int j = 0; j < kGlueGroups; ++j) {
    const int g = tid + kGlueThreads * j;
    if (g < ng) {
      uint32_t b[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) b[i] = f32_to_bf16(v[j][i] * scale);
      reinterpret_cast<uint4*>(u_out + base)[g] =
          make_uint4(b[0] | (b[1] << 16), b[2] | (b[3] << 16), b[4] | (b[5] << 16), b[6] | (b[7] << 16));
    }
  }
}

int glue_launch(const uint16_t* x, const float* y, int T, int d, float eps, uint16_t* x_out, uint16_t* u_out,
                hipStream_t s) {
  chain_glue_kernel<<<T, kGlueThreads, 0, s>>>(x, y, d, eps, x_out, u_out);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

struct ChainWs {
  uint16_t* resid[2]; // [T][d] residual stream, layers alternate (when not traced)
  uint16_t* u;        // [T][d] normalised layer input (when not traced)
  float* y;           // [T][d] layer output
  float* ssp[2];      // [T][d/8] sums of squares handed from layer to layer
  float* w;           // [T][k]
  float* sgate;       // [T]
  int32_t* idx;       // [T][k] (when not returned)
  void* layer_ws;
  size_t layer_bytes;
};

bool carve_chain(Carver& c, const moe_layer_desc* layers, int L, int T, int path, ChainWs* w) {
  const int d = layers[0].sh.d, k = layers[0].k;
  w->resid[0] = c.take<uint16_t>((size_t)T * d);
  w->resid[1] = c.take<uint16_t>((size_t)T * d);
  w->u = c.take<uint16_t>((size_t)T * d);
  w->y = c.take<float>((size_t)T * d);
  w->ssp[0] = c.take<float>((size_t)T * d / 8);
  w->ssp[1] = c.take<float>((size_t)T * d / 8);
  w->w = c.take<float>((size_t)T * k);
  w->sgate = c.take<float>((size_t)T);
  w->idx = c.take<int32_t>((size_t)T * k);
  size_t lb = 0;
  for (int l = 0; l < L; ++l) {
    const size_t b = moe_layer_workspace_bytes(&layers[l], T, path);
    lb = b > lb ? b : lb;
  }
  w->layer_bytes = lb;
  w->layer_ws = c.take<uint8_t>(lb);
  return c.ok();
}

int check_chain(const moe_layer_desc* layers, int L, int T) {
  if (!layers || L < 1 || T < 0) return MOE_ERR_INVALID_ARG;
  for (int l = 0; l < L; ++l) {
    if (moe_layer_workspace_bytes(&layers[l], 0, MOE_PATH_DECODE) == 0) return MOE_ERR_INVALID_ARG;
    if (layers[l].sh.d != layers[0].sh.d || layers[l].k != layers[0].k) return MOE_ERR_INVALID_ARG;
  }
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" size_t moe_chain_workspace_bytes(const moe_layer_desc* layers, int32_t L, int32_t T, int32_t path) {
  if (check_chain(layers, L, T) != MOE_OK) return 0;
  Carver c(nullptr, (size_t)-1);
  ChainWs w;
  carve_chain(c, layers, L, T, path, &w);
  return c.off + 256;
}

extern "C" int moe_chain_forward(const moe_layer_desc* layers, int32_t L, float eps, const uint16_t* x, int32_t T,
                                 uint16_t* x_out, uint16_t* trace_x, uint16_t* trace_u, int32_t* topk_idx,
                                 int32_t path, void* ws, size_t ws_bytes, hipStream_t s) {
  MOE_TRY(check_chain(layers, L, T));
  MOE_CHECK(eps >= 0.0f);
  if (T == 0) return MOE_OK;
  MOE_CHECK(x && x_out && ws && aligned(x, 16) && aligned(x_out, 16) && aligned(ws, 256));
  MOE_CHECK(!trace_x || aligned(trace_x, 16));
  MOE_CHECK(!trace_u || aligned(trace_u, 16));
  Carver c(ws, ws_bytes);
  ChainWs w;
  if (!carve_chain(c, layers, L, T, path, &w)) return MOE_ERR_INVALID_ARG;
  const int d = layers[0].sh.d, k = layers[0].k;
  const size_t td = (size_t)T * d;
  // x_l and x_{l-1} alternate between two buffers (or the trace)
  auto resid = [&](int l) { return trace_x ? trace_x + (size_t)l * td : w.resid[l & 1]; };
  auto uin = [&](int l) { return trace_u ? trace_u + (size_t)l * td : w.u; };
  // Decode layers of 4- and 8-bit experts hand the residual stream on
  // themselves (ChainIO): the down kernel writes x_{l+1} and its sums of
  // squares, the next router normalises; no glue launch between them, and
  // the same bits as with it.  Otherwise (other paths, f32 experts, or the
  // normalised inputs wanted as a trace) a glue launch per layer.
  bool handover = !trace_u;
  for (int l = 0; l < L && handover; ++l) {
    const moe_layer_desc* D = &layers[l];
    handover = shape_bits(&D->sh) != 32 && shape_bits(&D->shared_sh) != 32 &&
               resolve_path(path, T, d, D->k, D->E, shape_bits(&D->sh),
                            D->sh.I > D->shared_sh.I ? D->sh.I : D->shared_sh.I) == MOE_PATH_DECODE;
  }
  if (handover) {
    MOE_TRY(glue_launch(x, nullptr, T, d, eps, resid(0), w.u, s));        // x_0 and u_0
    for (int l = 0; l < L; ++l) {
      int32_t* idx = topk_idx ? topk_idx + (size_t)l * T * k : w.idx;
      ChainIO io{l == 0 ? nullptr : w.ssp[l & 1], eps, resid(l), l + 1 == L ? x_out : resid(l + 1),
                 w.ssp[(l + 1) & 1]};
      MOE_TRY(layer_forward(&layers[l], l == 0 ? w.u : resid(l), T, w.y, idx, w.w, w.sgate, path, w.layer_ws,
                            w.layer_bytes, s, &io));
    }
    if (trace_x) MOE_HIP(hipMemcpyAsync(trace_x + (size_t)L * td, x_out, td * 2, hipMemcpyDeviceToDevice, s));
    return MOE_OK;
  }
  for (int l = 0; l < L; ++l) {
    int32_t* idx = topk_idx ? topk_idx + (size_t)l * T * k : w.idx;
    // x_l = bf16(x_{l-1} + y_{l-1}) (x_0 copied) and u_l
    MOE_TRY(glue_launch(l == 0 ? x : resid(l - 1), l == 0 ? nullptr : w.y, T, d, eps, resid(l), uin(l), s));
    MOE_TRY(moe_layer_forward(&layers[l], uin(l), T, w.y, idx, w.w, w.sgate, path, w.layer_ws, w.layer_bytes, s));
  }
  // x_L = bf16(x_{L-1} + y_{L-1})
  MOE_TRY(glue_launch(resid(L - 1), w.y, T, d, eps, x_out, nullptr, s));
  if (trace_x) MOE_HIP(hipMemcpyAsync(trace_x + (size_t)L * td, x_out, td * 2, hipMemcpyDeviceToDevice, s));
  return MOE_OK;
}
