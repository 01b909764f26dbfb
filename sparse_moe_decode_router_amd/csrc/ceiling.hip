// Measured ceilings of the chip, for reporting the layer's kernels against
// what the MI355X actually sustains beside its published peaks: a plain
// streaming read of HBM in one launch, and a loop of dense fp16 MFMAs.
#include "internal.h"
#include "device.h"
#include "moe355_probe.h"

namespace moe {
namespace {

constexpr int kReadThreads = 256;
constexpr int kReadUnroll = 8;

// Every 16-byte piece of [buf, buf + n16 * 16) read once (all of a thread's
// kReadUnroll loads issued before their use), folded by XOR into one word per
// block so the loads stay live.
__global__ __launch_bounds__(kReadThreads) void stream_read_kernel(const uint4* __restrict__ buf, size_t n16,
                                                                   uint32_t* __restrict__ sink) {
  const size_t stride = (size_t)gridDim.x * kReadThreads;
  uint32_t acc = 0;
  for (size_t base = (size_t)blockIdx.x * kReadThreads + threadIdx.x; base < n16; base += stride * kReadUnroll) {
    uint4 v[kReadUnroll];
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) {
      const size_t i = base + u * stride;
      v[u] = buf[i < n16 ? i : base];             // clamped: in bounds, loads unconditional
    }
#pragma unroll
    for (int u = 0; u < kReadUnroll; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[kReadThreads / 64];
  for (int s = 32; s >= 1; s >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, s, 64);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = acc;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float16_t __attribute__((ext_vector_type(16)));

// Four independent accumulation chains of v_mfma_f32_32x32x16_f16 per wave,
// operands in registers: iters x 4 x 32 x 32 x 16 x 2 flop per wave.
__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & 63;
  half8_t a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (_Float16)(0.001f * (float)((lane + i) & 7));
    b[i] = (_Float16)(0.001f * (float)((lane * 3 + i) & 7));
  }
  float16_t c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int it = 0; it < iters; ++it) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c3, 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) s += c0[i] + c1[i] + c2[i] + c3[i];
  sink[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_probe_stream_read(const void* buf, size_t bytes, uint32_t* sink, int32_t blocks,
                                     hipStream_t s) {
  MOE_CHECK(buf && sink && blocks >= 1 && blocks <= 65536 && bytes >= 16 && bytes % 16 == 0);
  MOE_CHECK(aligned(buf, 16) && aligned(sink, 4));
  stream_read_kernel<<<blocks, kReadThreads, 0, s>>>(static_cast<const uint4*>(buf), bytes / 16, sink);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

extern "C" int moe_probe_mfma_f16(int32_t iters, float* sink, int32_t blocks, hipStream_t s) {
  MOE_CHECK(sink && blocks >= 1 && blocks <= 65536 && iters >= 1);
  mfma_loop_kernel<<<blocks, 256, 0, s>>>(iters, sink);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

extern "C" double moe_probe_mfma_f16_flops(int32_t iters, int32_t blocks) {
  return (double)blocks * 4.0 * (double)iters * 4.0 * 32.0 * 32.0 * 16.0 * 2.0;
}
