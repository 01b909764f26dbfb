// Weighted combine of routed expert outputs and the gated shared expert:
// y[t] = sum_{r<k} w[t,r] * partial[t*k+r] + s_t * shared_out[t], in that
// order (Swiftlet pages, "How it works": routed experts plus a resident shared
// expert; correctness section: placement never changes the answer, which a
// fixed summation order with no float atomics guarantees bit for bit).
#include "internal.h"
#include "device.h"

namespace moe {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(const float* __restrict__ partial,
                                                      const float* __restrict__ shared_out,
                                                      const float* __restrict__ w,
                                                      const float* __restrict__ sgate, int T, int k,
                                                      int d, float* __restrict__ y) {
  const int d4 = d / 4;
  const long id = (long)blockIdx.x * blockDim.x + threadIdx.x;
  if (id >= (long)T * d4) return;
  const int t = (int)(id / d4), c = (int)(id % d4);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  // up to kMaxK ranks: every load in flight before the (rank-order) sum
  constexpr int kMaxK = 16;
  float4 pv[kMaxK];
  float wv[kMaxK];
#pragma unroll
  for (int r = 0; r < kMaxK; ++r) {
    if (r < k) {
      wv[r] = w[(size_t)t * k + r];
      pv[r] = reinterpret_cast<const float4*>(partial + ((size_t)t * k + r) * d)[c];
    }
  }
#pragma unroll
  for (int r = 0; r < kMaxK; ++r) {
    if (r < k) {
      acc.x += wv[r] * pv[r].x; acc.y += wv[r] * pv[r].y; acc.z += wv[r] * pv[r].z; acc.w += wv[r] * pv[r].w;
    }
  }
  for (int r = kMaxK; r < k; ++r) {
    const float wr = w[(size_t)t * k + r];
    const float4 p = reinterpret_cast<const float4*>(partial + ((size_t)t * k + r) * d)[c];
    acc.x += wr * p.x; acc.y += wr * p.y; acc.z += wr * p.z; acc.w += wr * p.w;
  }
  if (shared_out) {
    const float s = sgate[t];
    const float4 p = reinterpret_cast<const float4*>(shared_out + (size_t)t * d)[c];
    acc.x += s * p.x; acc.y += s * p.y; acc.z += s * p.z; acc.w += s * p.w;
  }
  reinterpret_cast<float4*>(y + (size_t)t * d)[c] = acc;
}

// Slot-table edits carried by value in the launch, so no host buffer has to
// outlive the call.
struct TableEdit {
  int32_t n;
  int32_t expert[30];
  int32_t slot[30];
};

__global__ void table_edit_kernel(int32_t* __restrict__ table, TableEdit ed) {
  // edits apply in order: later entries win
  if (threadIdx.x == 0)
    for (int q = 0; q < ed.n; ++q) table[ed.expert[q]] = ed.slot[q];
}

// Blob copies host -> slot carried by value as well: blob q of the launch is
// read from src + expert[q] * src_stride (pinned host memory, read over PCIe
// by the CUs) and written to dst + slot[q] * dst_stride.
struct BlobPull {
  const uint4* src;
  uint4* dst;
  long src_stride16, dst_stride16, n16;     // in 16-byte pieces (n16 per blob, from off16)
  long off16;
  int32_t n;
  int32_t expert[30];
  int32_t slot[30];
};

__global__ __launch_bounds__(256) void blob_pull_kernel(BlobPull j) {
  const long total = j.n16 * j.n;
  const long step = (long)gridDim.x * blockDim.x;
  // four pieces per thread in flight (clamped loads, guarded stores)
  for (long q0 = (long)blockIdx.x * blockDim.x + threadIdx.x; q0 < total; q0 += 4 * step) {
    uint4 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long q = q0 + u * step < total ? q0 + u * step : 0;
      const int b = (int)(q / j.n16);
      v[u] = j.src[j.expert[b] * j.src_stride16 + j.off16 + q % j.n16];
    }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const long q = q0 + u * step;
      if (q < total) {
        const int b = (int)(q / j.n16);
        j.dst[j.slot[b] * j.dst_stride16 + j.off16 + q % j.n16] = v[u];
      }
    }
  }
}

}  // namespace

int blob_pull_launch(const void* src_dev, size_t src_stride, void* dst, size_t dst_stride, size_t off,
                     size_t bytes, const int32_t* experts, const int32_t* slots, int n, hipStream_t s) {
  if ((uintptr_t)src_dev % 16 || (uintptr_t)dst % 16 || src_stride % 16 || dst_stride % 16 || bytes % 16 ||
      off % 16)
    return MOE_ERR_INVALID_ARG;
  for (int base = 0; base < n; base += 30) {
    BlobPull j;
    j.src = static_cast<const uint4*>(src_dev);
    j.dst = static_cast<uint4*>(dst);
    j.src_stride16 = (long)(src_stride / 16);
    j.dst_stride16 = (long)(dst_stride / 16);
    j.n16 = (long)(bytes / 16);
    j.off16 = (long)(off / 16);
    j.n = (n - base) < 30 ? (n - base) : 30;
    for (int q = 0; q < j.n; ++q) {
      j.expert[q] = experts[base + q];
      j.slot[q] = slots[base + q];
    }
    // 64 blocks already keep the PCIe link full; more would only take CUs
    blob_pull_kernel<<<64, 256, 0, s>>>(j);
    MOE_HIP(hipGetLastError());
  }
  return MOE_OK;
}

int combine_launch(const float* partial, const float* shared_out, const float* w, const float* sgate,
                   int T, int k, int d, float* y, hipStream_t s) {
  const long n = (long)T * (d / 4);
  if (n == 0) return MOE_OK;
  combine_kernel<<<(unsigned)((n + 255) / 256), 256, 0, s>>>(partial, shared_out, w, sgate, T, k, d, y);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

int table_edit_launch(int32_t* table, const int32_t* experts, const int32_t* slots, int n,
                      hipStream_t s) {
  for (int base = 0; base < n; base += 30) {
    TableEdit ed;
    ed.n = (n - base) < 30 ? (n - base) : 30;
    for (int q = 0; q < ed.n; ++q) {
      ed.expert[q] = experts[base + q];
      ed.slot[q] = slots[base + q];
    }
    table_edit_kernel<<<1, 64, 0, s>>>(table, ed);
    MOE_HIP(hipGetLastError());
  }
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" int moe_combine(const float* partial, const float* shared_out, const float* w,
                           const float* sgate, int32_t T, int32_t k, int32_t d, float* y,
                           hipStream_t s) {
  MOE_CHECK(T >= 0 && k >= 1 && d > 0 && d % 4 == 0);
  if (T == 0) return MOE_OK;
  MOE_CHECK(partial && w && y);
  MOE_CHECK((shared_out == nullptr) == (sgate == nullptr));
  MOE_CHECK(aligned(partial, 16) && aligned(y, 16) && (!shared_out || aligned(shared_out, 16)));
  return combine_launch(partial, shared_out, w, sgate, T, k, d, y, s);
}
