// moe_layer_forward without a caller workspace: the layer's scratch (router
// logits, activation pairs, intermediates, bucket lists, partial outputs)
// lives in one file-scope device array per GPU, so the call allocates nothing
// (for code under HIP graph capture, tight serving loops and harnesses that
// forbid hipMalloc).
//
// The array's host-side name is only a stand-in for the symbol: its device
// address comes from hipGetSymbolAddress, taken once per device with that
// device current and kept; kernels get that address, never the name.
#include <mutex>

#include "internal.h"

namespace moe {
namespace {

constexpr size_t kScratchBytes = (size_t)MOE_NOALLOC_SCRATCH_BYTES;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Clears the scratch once per device (a kernel rather than a memset, so the
// first call may itself be captured into a graph).
__global__ __launch_bounds__(256) void scratch_fill_kernel(uint4* __restrict__ p, size_t n16) {
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += (size_t)gridDim.x * blockDim.x)
    p[i] = make_uint4(0, 0, 0, 0);
}

std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};

// Device address of this device's scratch, set up on the first call (the
// clearing kernel goes on `s`, ahead of the call's own work).
int scratch_for_current_device(hipStream_t s, void** out) {
  int dev = -1;
  MOE_HIP(hipGetDevice(&dev));
  if (dev < 0 || dev >= kMaxDevices) return MOE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    MOE_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)));
    if (!p) return MOE_ERR_HIP;
    scratch_fill_kernel<<<1024, 256, 0, s>>>(static_cast<uint4*>(p), kScratchBytes / 16);
    MOE_HIP(hipGetLastError());
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return MOE_OK;
}

}  // namespace
}  // namespace moe

using namespace moe;

extern "C" int moe_layer_forward_noalloc(const moe_layer_desc* L, const uint16_t* x, int32_t T, float* y,
                                         int32_t* idx, float* w, float* sgate, int32_t path, hipStream_t s) {
  MOE_CHECK(L && T >= 0);
  if (T == 0) return MOE_OK;
  const size_t need = moe_layer_workspace_bytes(L, T, path);
  if (need == 0) return MOE_ERR_INVALID_ARG;
  if (need > kScratchBytes) return MOE_ERR_UNSUPPORTED;
  void* ws = nullptr;
  MOE_TRY(scratch_for_current_device(s, &ws));
  return layer_forward(L, x, T, y, idx, w, sgate, path, ws, kScratchBytes, s, nullptr);
}
