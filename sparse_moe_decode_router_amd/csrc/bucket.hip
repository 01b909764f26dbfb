// Token -> expert bucketing: a stable counting sort of the (token, rank)
// pairs i = t*k + r by expert (histogram, exclusive scan, stable scatter).
// The pages do not describe batching; this is the grouping the batched and
// prefill expert passes need so each expert's weights are read once per step.
//
// Pairs are cut into blocks of 1024 (one per thread).  Within a block a
// pair's stable rank among equal keys is: rank among equal keys in its wave
// (ballot match on the key bits) + equal keys in earlier waves (LDS table of
// per-wave counts).  Across blocks the scan runs in (expert, block) order.
// Everything is integer work: bit-exact and deterministic.
#include "internal.h"
#include "device.h"

namespace moe {
namespace {

constexpr int kB = 1024;     // pairs per block
constexpr int kW = kB / 64;  // waves per block

__device__ __forceinline__ int key_bits(int E) { return 32 - __clz(E > 1 ? E - 1 : 1); }

// Stable within-block position of this thread's pair; base(e) gives where the
// block's first pair of expert e lands.  wc: LDS [kW][E] (zeroed here).
template <class BaseFn>
__device__ void scatter_block(int key, bool valid, int i, int E, uint8_t* wc, BaseFn base,
                              int32_t* __restrict__ pair_ids) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  for (int q = tid; q < kW * E; q += kB) wc[q] = 0;
  __syncthreads();
  uint64_t peers = __ballot(valid);
  if (!valid) peers = 0;
  const int nb = key_bits(E);
  for (int b = 0; b < nb; ++b) {
    const uint64_t m = __ballot(valid && ((key >> b) & 1));
    if (valid) peers &= ((key >> b) & 1) ? m : ~m;
  }
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  const int rank_w = __popcll(peers & below);
  if (valid && rank_w == 0) wc[wave * E + key] = (uint8_t)__popcll(peers);
  __syncthreads();
  if (valid) {
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wc[w * E + key];
    pair_ids[base(key) + before + rank_w] = i;
  }
}

// Whole sort in one block (T*k <= 1024).
__global__ __launch_bounds__(kB) void bucket_single_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                           int32_t* __restrict__ counts,
                                                           int32_t* __restrict__ offsets,
                                                           int32_t* __restrict__ pair_ids,
                                                           uint32_t* __restrict__ usage) {
  extern __shared__ int lds[];          // cnt[E] | scan[1024] | wc[kW][E] bytes
  int* cnt = lds;
  int* scan = lds + E;
  uint8_t* wc = reinterpret_cast<uint8_t*>(scan + kB);
  const int tid = threadIdx.x;
  for (int e = tid; e < E; e += kB) cnt[e] = 0;
  __syncthreads();
  const bool valid_i = tid < n;
  int key = valid_i ? idx[tid] : -1;
  const bool valid = valid_i && key >= 0 && key < E;
  if (valid) atomicAdd(&cnt[key], 1);
  __syncthreads();
  // exclusive scan over E <= 1024 bins, one per thread
  const int c = tid < E ? cnt[tid] : 0;
  scan[tid] = c;
  __syncthreads();
  for (int off = 1; off < kB; off <<= 1) {
    const int v = tid >= off ? scan[tid - off] : 0;
    __syncthreads();
    scan[tid] += v;
    __syncthreads();
  }
  if (tid < E) {
    counts[tid] = c;
    offsets[tid] = scan[tid] - c;
    cnt[tid] = scan[tid] - c;           // reuse as base
    if (usage && c > 0) atomicAdd(&usage[tid], (uint32_t)c);
  }
  if (tid == 0) offsets[E] = scan[kB - 1];
  __syncthreads();
  scatter_block(key, valid, tid, E, wc, [&](int e) { return cnt[e]; }, pair_ids);
}

// Multi-block: per-block histograms bc[e][nb].
__global__ __launch_bounds__(kB) void bucket_hist_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                         int nb, int32_t* __restrict__ bc) {
  extern __shared__ int cnt[];
  const int tid = threadIdx.x, b = blockIdx.x;
  for (int e = tid; e < E; e += kB) cnt[e] = 0;
  __syncthreads();
  const int i = b * kB + tid;
  if (i < n) {
    const int key = idx[i];
    if (key >= 0 && key < E) atomicAdd(&cnt[key], 1);
  }
  __syncthreads();
  for (int e = tid; e < E; e += kB) bc[(size_t)e * nb + b] = cnt[e];
}

// Exclusive scan of bc in (expert, block) order -> base; counts, offsets.
// Each thread owns a contiguous run of bc, read kU entries at a time with
// all loads of a batch in flight (one memory latency per batch, not per
// entry).  usage (optional): usage[e] += counts[e], one atomic per expert.
constexpr int kU = 16;
__global__ __launch_bounds__(kB) void bucket_scan_kernel(int32_t* __restrict__ bc, int E, int nb,
                                                         int32_t* __restrict__ counts,
                                                         int32_t* __restrict__ offsets,
                                                         uint32_t* __restrict__ usage) {
  __shared__ int part[kB];
  const int tid = threadIdx.x;
  const long N = (long)E * nb;
  const long per = (N + kB - 1) / kB;
  const long lo = tid * per, hi = lo + per < N ? lo + per : N;
  int s = 0;
  for (long q0 = lo; q0 < hi; q0 += kU) {
    int v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = q0 + u < hi ? bc[q0 + u] : 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) s += v[u];
  }
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < kB; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (long q0 = lo; q0 < hi; q0 += kU) {
    int v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) v[u] = q0 + u < hi ? bc[q0 + u] : 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      if (q0 + u < hi) bc[q0 + u] = run;
      run += v[u];
    }
  }
  __syncthreads();
  // counts/offsets per expert
  for (int e = tid; e < E; e += kB) {
    const int first = bc[(size_t)e * nb];
    const int next = (e + 1 < E) ? bc[(size_t)(e + 1) * nb] : part[kB - 1];
    offsets[e] = first;
    counts[e] = next - first;
    if (usage && next > first) atomicAdd(&usage[e], (uint32_t)(next - first));
  }
  if (tid == 0) offsets[E] = part[kB - 1];
}

// The same scan with bc staged in LDS (when E nb entries fit): the loads
// and the write-back are coalesced (kU loads per thread in flight), the
// per-thread runs are scanned in LDS.  Same integers as bucket_scan_kernel.
constexpr int kScanLdsMax = 24576;              // entries (96 KB)
__global__ __launch_bounds__(kB) void bucket_scan_lds_kernel(int32_t* __restrict__ bc, int E, int nb,
                                                             int32_t* __restrict__ counts,
                                                             int32_t* __restrict__ offsets,
                                                             uint32_t* __restrict__ usage) {
  extern __shared__ int sbc[];                  // [E nb]
  __shared__ int part[kB];
  const int tid = threadIdx.x;
  const int N = E * nb;
  for (int q0 = 0; q0 < N; q0 += kU * kB) {
    int v[kU];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int q = q0 + u * kB + tid;
      v[u] = bc[q < N ? q : 0];                 // clamped: loads stay unconditional
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int q = q0 + u * kB + tid;
      if (q < N) sbc[q] = v[u];
    }
  }
  __syncthreads();
  const int per = (N + kB - 1) / kB;
  const int lo = tid * per < N ? tid * per : N, hi = lo + per < N ? lo + per : N;
  int s = 0;
  for (int q = lo; q < hi; ++q) s += sbc[q];
  part[tid] = s;
  __syncthreads();
  for (int off = 1; off < kB; off <<= 1) {
    const int v = tid >= off ? part[tid - off] : 0;
    __syncthreads();
    part[tid] += v;
    __syncthreads();
  }
  int run = part[tid] - s;
  for (int q = lo; q < hi; ++q) {
    const int v = sbc[q];
    sbc[q] = run;
    run += v;
  }
  __syncthreads();
  for (int q = tid; q < N; q += kB) bc[q] = sbc[q];
  for (int e = tid; e < E; e += kB) {
    const int first = sbc[e * nb];
    const int next = (e + 1 < E) ? sbc[(e + 1) * nb] : part[kB - 1];
    offsets[e] = first;
    counts[e] = next - first;
    if (usage && next > first) atomicAdd(&usage[e], (uint32_t)(next - first));
  }
  if (tid == 0) offsets[E] = part[kB - 1];
}

__global__ __launch_bounds__(kB) void bucket_scatter_kernel(const int32_t* __restrict__ idx, int n, int E,
                                                            int nb, const int32_t* __restrict__ base,
                                                            int32_t* __restrict__ pair_ids) {
  extern __shared__ uint8_t wc[];
  const int b = blockIdx.x, i = b * kB + threadIdx.x;
  const bool in = i < n;
  const int key = in ? idx[i] : -1;
  const bool valid = in && key >= 0 && key < E;
  scatter_block(key, valid, i, E, wc, [&](int e) { return base[(size_t)e * nb + b]; }, pair_ids);
}

}  // namespace

size_t bucket_ws_bytes(int T, int k, int E) {
  const long n = (long)T * k;
  const long nb = (n + kB - 1) / kB;
  return (size_t)(E * nb) * 4 + 512;
}

int bucket_launch(const int32_t* idx, int T, int k, int E, int32_t* counts, int32_t* offsets,
                  int32_t* pair_ids, void* ws, size_t ws_bytes, hipStream_t s, uint32_t* usage) {
  const long n = (long)T * k;
  if (n <= kB) {
    const size_t lds = ((size_t)E + kB) * 4 + (size_t)kW * E;
    bucket_single_kernel<<<1, kB, lds, s>>>(idx, (int)n, E, counts, offsets, pair_ids, usage);
    MOE_HIP(hipGetLastError());
    return MOE_OK;
  }
  const int nb = (int)((n + kB - 1) / kB);
  if (!ws || ws_bytes < bucket_ws_bytes(T, k, E)) return MOE_ERR_INVALID_ARG;
  int32_t* bc = (int32_t*)ws;
  bucket_hist_kernel<<<nb, kB, (size_t)E * 4, s>>>(idx, (int)n, E, nb, bc);
  MOE_HIP(hipGetLastError());
  if ((long)E * nb <= kScanLdsMax)
    bucket_scan_lds_kernel<<<1, kB, (size_t)E * nb * 4, s>>>(bc, E, nb, counts, offsets, usage);
  else
    bucket_scan_kernel<<<1, kB, 0, s>>>(bc, E, nb, counts, offsets, usage);
  MOE_HIP(hipGetLastError());
  bucket_scatter_kernel<<<nb, kB, (size_t)kW * E, s>>>(idx, (int)n, E, nb, bc, pair_ids);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" size_t moe_bucket_workspace_bytes(int32_t T, int32_t k, int32_t E) {
  if (T < 0 || k <= 0 || E <= 0) return 0;
  return bucket_ws_bytes(T, k, E);
}

extern "C" int moe_bucket_tokens(const int32_t* idx, int32_t T, int32_t k, int32_t E, int32_t* counts,
                                 int32_t* offsets, int32_t* pair_ids, void* ws, size_t ws_bytes,
                                 hipStream_t s) {
  MOE_CHECK(T >= 0 && k >= 1 && E >= 1 && E <= 1024);
  MOE_CHECK((long)T * k <= (1L << 30));
  MOE_CHECK(counts && offsets);
  if (T > 0) MOE_CHECK(idx && pair_ids);
  if (T == 0) {
    MOE_HIP(hipMemsetAsync(counts, 0, (size_t)E * 4, s));
    MOE_HIP(hipMemsetAsync(offsets, 0, (size_t)(E + 1) * 4, s));
    return MOE_OK;
  }
  return bucket_launch(idx, T, k, E, counts, offsets, pair_ids, ws, ws_bytes, s, nullptr);
}
