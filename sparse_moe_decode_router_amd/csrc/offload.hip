// Refill planned and copied by the GPU (moe_layer_forward_offload): the
// pool's LFU + recency policy ("How it works": hot experts kept in a bounded
// pool, the rest fetched on demand; relationship-to-TurboFieldfare section:
// LFU with recency) run by one wave on a device copy of the policy state,
// then the missing blobs read over PCIe from mapped pinned host memory by a
// copy kernel that takes its work list from the plan.  No host wait sits
// between the router and the experts.
//
// The rules are those of moe_lfu_plan, decision for decision:
//   * the step's distinct experts in first-appearance order; every
//     selection adds one to its expert's count and sets its last-use step;
//   * a needed expert with a slot is a hit; a miss takes the lowest free
//     slot, else evicts the resident expert this step does not need with the
//     smallest (count, last use, id);
//   * stats: steps, hits, misses, loads, evictions, bytes loaded.
#include "internal.h"
#include "device.h"
#include "pull.h"

namespace moe {
namespace {

constexpr int kPlanMax = 1024;         // E and n_slots limits of the device plan

// (count, last, id) key order of the eviction rule, reduced over one wave.
struct VKey {
  uint64_t count;
  int64_t last;
  int32_t id;                          // -1: no candidate
};

__device__ __forceinline__ bool vkey_less(const VKey& a, const VKey& b) {
  if (a.id < 0) return false;
  if (b.id < 0) return true;
  if (a.count != b.count) return a.count < b.count;
  if (a.last != b.last) return a.last < b.last;
  return a.id < b.id;
}

__device__ __forceinline__ VKey vkey_shfl_xor(const VKey& k, int m) {
  VKey o;
  o.count = ((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)(k.count >> 32), m, 64) << 32) |
            (uint32_t)__shfl_xor((int)(uint32_t)k.count, m, 64);
  o.last = (int64_t)(((uint64_t)(uint32_t)__shfl_xor((int)(uint32_t)((uint64_t)k.last >> 32), m, 64) << 32) |
                     (uint32_t)__shfl_xor((int)(uint32_t)(uint64_t)k.last, m, 64));
  o.id = __shfl_xor(k.id, m, 64);
  return o;
}

__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = min(v, __shfl_xor(v, m, 64));
  return v;
}

// The whole policy state sits in LDS for the step: four waves load and
// store it (every load of a thread in flight at once); wave 0 marks the
// needed experts (selections: at most 64, one a lane) and plans.  The loop
// over the needed experts is block-uniform (its branches read LDS that every
// wave sees after the barrier), so all waves meet every barrier.
constexpr int kPlanThreads = 256;
__global__ __launch_bounds__(kPlanThreads) void lfu_plan_kernel(DevLfu v, int E, int n_slots, uint64_t stride,
                                                                int32_t* __restrict__ table,
                                                                int32_t* __restrict__ err,
                                                                const int32_t* __restrict__ sel, int n,
                                                                int32_t* __restrict__ n_loads_out) {
  __shared__ unsigned long long cnt_s[kPlanMax];
  __shared__ int64_t last_s[kPlanMax];
  __shared__ int32_t slot_s[kPlanMax];
  __shared__ int32_t holder_s[kPlanMax];
  __shared__ int32_t need_l[64];
  __shared__ uint8_t need_s[kPlanMax];
  __shared__ int32_t sel_s[64];
  __shared__ int m_s, stop_s;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {
    constexpr int U = kPlanMax / kPlanThreads;
    uint64_t c[U];
    int64_t l[U];
    int32_t so[U], ho[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = tid + kPlanThreads * u;
      c[u] = e < E ? v.count[e] : 0;
      l[u] = e < E ? v.last[e] : 0;
      so[u] = e < E ? v.slot_of[e] : 0;
      ho[u] = e < n_slots ? v.holder[e] : 0;
    }
    const int se = tid < n ? sel[tid] : 0;
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int e = tid + kPlanThreads * u;
      if (e < E) {
        cnt_s[e] = c[u];
        last_s[e] = l[u];
        slot_s[e] = so[u];
        need_s[e] = 0;
      }
      if (e < n_slots) holder_s[e] = ho[u];
    }
    if (tid < n) sel_s[tid] = se;
  }
  __syncthreads();
  const int64_t step = (int64_t)v.meta[0];
  if (wave == 0) {
    // first appearances (in selection order), every selection's count and
    // last use, and the needed list by a ballot
    const int my = lane < n ? sel_s[lane] : -1;
    const bool bad = __any(lane < n && (my < 0 || my >= E));
    bool first = lane < n;
    for (int q = 0; q < n; ++q)
      if (q < lane && sel_s[q] == my) first = false;
    if (!bad) {
      if (lane < n) {
        atomicAdd(&cnt_s[my], 1ull);
        last_s[my] = step;
        need_s[my] = 1;
      }
      const uint64_t fm = __ballot(first);
      if (first) need_l[__popcll(fm & ((1ull << lane) - 1))] = my;
      if (lane == 0) m_s = __popcll(fm);
    } else if (lane == 0) {
      m_s = -1;
    }
    if (lane == 0) stop_s = 0;
  }
  __syncthreads();
  const int m = m_s;
  if (m < 0) {                          // a selection outside [0, E): nothing planned, error word set
    if (tid == 0) {
      v.plan[0] = 0;
      if (n_loads_out) *n_loads_out = 0;
      atomicOr(err, 4);
    }
    return;
  }
  uint64_t hits = 0, misses = 0, evictions = 0;
  int nl = 0;
  bool any_free = true;                 // wave 0's view
  for (int j = 0; j < m; ++j) {
    const int e = need_l[j];
    if (slot_s[e] >= 0) {
      ++hits;
      continue;
    }
    ++misses;
    if (wave == 0) {
      int slot = -1, victim = -1;
      if (any_free) {
        int f = 0x7fffffff;
        for (int sl = lane; sl < n_slots; sl += 64)
          if (holder_s[sl] < 0) f = min(f, sl);
        f = wave_min_int(f);
        if (f == 0x7fffffff) any_free = false;
        else slot = f;
      }
      if (slot < 0) {
        VKey best{0, 0, -1};
        for (int c = lane; c < E; c += 64)
          if (slot_s[c] >= 0 && !need_s[c]) {
            const VKey k{cnt_s[c], last_s[c], c};
            if (vkey_less(k, best)) best = k;
          }
#pragma unroll
        for (int mm = 32; mm >= 1; mm >>= 1) {
          const VKey o = vkey_shfl_xor(best, mm);
          if (vkey_less(o, best)) best = o;
        }
        victim = best.id;               // exists: n <= n_slots is checked by the host
        if (victim >= 0) {
          slot = slot_s[victim];
          ++evictions;
        }
      }
      if (lane == 0) {
        if (slot < 0) {                 // never taken: reported, the step plans nothing more
          atomicOr(err, 4);
          stop_s = 1;
        } else {
          if (victim >= 0) {
            slot_s[victim] = -1;
            table[victim] = -1;
          }
          holder_s[slot] = e;
          slot_s[e] = slot;
          table[e] = slot;
          v.plan[1 + nl] = e;
          v.plan[1 + E + nl] = slot;
          v.plan[1 + 2 * E + nl] = victim;
        }
      }
    }
    __syncthreads();
    if (stop_s) break;
    ++nl;
  }
  for (int e = tid; e < E; e += kPlanThreads) {
    v.count[e] = cnt_s[e];
    v.last[e] = last_s[e];
    v.slot_of[e] = slot_s[e];
  }
  for (int sl = tid; sl < n_slots; sl += kPlanThreads) v.holder[sl] = holder_s[sl];
  if (tid == 0) {
    v.plan[0] = nl;
    if (n_loads_out) *n_loads_out = nl;
    v.meta[0] = (uint64_t)(step + 1);
    v.meta[1] += 1;                     // steps
    v.meta[2] += hits;
    v.meta[3] += misses;
    v.meta[4] += (uint64_t)nl;          // loads
    v.meta[5] += evictions;             // counted by wave 0, whose tid 0 writes
    v.meta[6] += (uint64_t)nl * stride; // bytes loaded
  }
}

// The planned blobs' byte range copied from host memory into their slots,
// the work list read from the plan in device memory.
__global__ __launch_bounds__(256) void plan_pull_kernel(PullJob j) { plan_pull_body(j, blockIdx.x); }

}  // namespace

bool lfu_plan_fits(int E, int n_slots, int n) { return E <= kPlanMax && n_slots <= kPlanMax && n <= 64; }

int lfu_plan_launch(const DevLfu& v, int E, int n_slots, size_t stride, int32_t* table, int32_t* err,
                    const int32_t* sel, int n, int32_t* n_loads_out, hipStream_t s) {
  if (!lfu_plan_fits(E, n_slots, n) || n < 0) return MOE_ERR_UNSUPPORTED;
  lfu_plan_kernel<<<1, kPlanThreads, 0, s>>>(v, E, n_slots, (uint64_t)stride, table, err, sel, n, n_loads_out);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

int plan_pull_launch(const void* src_dev, size_t src_stride, void* dst, size_t dst_stride, size_t off,
                     size_t bytes, const int32_t* plan, int E, hipStream_t s) {
  if ((uintptr_t)src_dev % 16 || (uintptr_t)dst % 16 || src_stride % 16 || dst_stride % 16 || bytes % 16 ||
      off % 16 || !plan)
    return MOE_ERR_INVALID_ARG;
  PullJob j;
  j.src = static_cast<const uint4*>(src_dev);
  j.dst = static_cast<uint4*>(dst);
  j.src_stride16 = (long)(src_stride / 16);
  j.dst_stride16 = (long)(dst_stride / 16);
  j.off16 = (long)(off / 16);
  j.n16 = (long)(bytes / 16);
  j.plan = plan;
  j.E = E;
  j.blocks = 64;                        // 64 blocks keep the PCIe link full (as the host-planned copy)
  plan_pull_kernel<<<j.blocks, 256, 0, s>>>(j);
  MOE_HIP(hipGetLastError());
  return MOE_OK;
}

}  // namespace moe
