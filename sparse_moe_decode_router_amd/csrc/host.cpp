// Host side of libmoe355: status strings, blob packing, the slot pool with
// its LFU + recency policy, and the whole-layer driver.
//
// Swiftlet pages: routed experts are repacked as fixed-stride blobs so one
// fetch is one read, and cached in a bounded slot pool evicted by LFU plus
// recency ("How it works"; relationship-to-TurboFieldfare section); a cached
// expert and a freshly loaded one give the same answer (correctness section).
#include <algorithm>
#include <cstring>
#include <memory>
#include <new>
#include <stdexcept>
#include <string>
#include <vector>

#include "internal.h"

namespace moe {

static thread_local std::string g_last_hip;

int hip_fail(hipError_t e) {
  g_last_hip = std::string(hipGetErrorName(e)) + ": " + hipGetErrorString(e);
  return MOE_ERR_HIP;
}

// Host entry points that grow std::vectors: an allocation failure comes back
// as MOE_ERR_OUT_OF_MEMORY instead of an exception crossing the C ABI.
template <class F>
static int no_throw(F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return MOE_ERR_OUT_OF_MEMORY;
  } catch (...) {
    return MOE_ERR_INVALID_ARG;
  }
}

bool shape_ok(const moe_ffn_shape* sh) {
  return sh && sh->group == 64 && sh->d >= 64 && sh->I >= 64 && sh->d % 64 == 0 && sh->I % 64 == 0 &&
         sh->d <= 16384 && sh->I <= 16384 &&
         (sh->bits == 0 || sh->bits == 4 || sh->bits == 8 || sh->bits == 32);
}

int blob_pull_launch(const void* src_dev, size_t src_stride, void* dst, size_t dst_stride, size_t off,
                     size_t bytes, const int32_t* experts, const int32_t* slots, int n, hipStream_t s);
int table_edit_launch(int32_t* table, const int32_t* experts, const int32_t* slots, int n,
                      hipStream_t s);

}  // namespace moe

using namespace moe;

// ------------------------------------------------------------------ status
extern "C" const char* moe_status_string(int st) {
  switch (st) {
    case MOE_OK: return "ok";
    case MOE_ERR_INVALID_ARG: return "invalid argument";
    case MOE_ERR_UNSUPPORTED: return "unsupported shape";
    case MOE_ERR_NOT_RESIDENT: return "selected expert not resident";
    case MOE_ERR_POOL_TOO_SMALL: return "pool too small for one step's experts";
    case MOE_ERR_HIP: return "HIP runtime error";
    case MOE_ERR_OUT_OF_MEMORY: return "host allocation failed";
    default: return "unknown status";
  }
}

extern "C" const char* moe_last_hip_error(void) { return g_last_hip.c_str(); }
extern "C" const char* moe_version(void) { return "libmoe355 0.1 gfx950"; }

// ------------------------------------------------------------------ blobs
extern "C" size_t moe_blob_bytes(const moe_ffn_shape* sh) {
  return shape_ok(sh) ? blob_layout(sh->d, sh->I, shape_bits(sh)).bytes : 0;
}
extern "C" size_t moe_blob_stride(const moe_ffn_shape* sh) {
  return shape_ok(sh) ? blob_layout(sh->d, sh->I, shape_bits(sh)).stride : 0;
}

// Inside each 8 inputs, 8-bit codes are stored in the byte order
// (0, 1, 4, 5, 2, 3, 6, 7): byte j of the block holds input kPerm8[j] (the
// permutation is its own inverse).
static const int kPerm8[8] = {0, 1, 4, 5, 2, 3, 6, 7};

extern "C" int moe_pack_expert(const moe_ffn_shape* sh, const uint8_t* const codes[3],
                               const uint16_t* const scales[3], const uint16_t* const biases[3],
                               void* out) {
  if (!shape_ok(sh) || !codes || !scales || !biases || !out) return MOE_ERR_INVALID_ARG;
  const int bits = shape_bits(sh);
  if (bits == 32) return MOE_ERR_INVALID_ARG;     // f32 experts: moe_pack_expert_f32
  const BlobLayout L = blob_layout(sh->d, sh->I, bits);
  const int outs[3] = {sh->I, sh->I, sh->d};
  const int ins[3] = {sh->d, sh->d, sh->I};
  uint8_t* blob = static_cast<uint8_t*>(out);
  for (int m = 0; m < 3; ++m) {
    if (!codes[m] || !scales[m] || !biases[m]) return MOE_ERR_INVALID_ARG;
    const size_t n = (size_t)outs[m] * ins[m];
    if (bits == 4)
      for (size_t q = 0; q < n; ++q)
        if (codes[m][q] > 15) return MOE_ERR_INVALID_ARG;
  }
  std::memset(blob, 0, L.stride);
  for (int m = 0; m < 3; ++m) {
    const int O = outs[m], N = ins[m];
    uint8_t* cd = blob + L.m[m].codes;
    if (bits == 4) {
      for (int c = 0; c < N / 32; ++c)
        for (int o = 0; o < O; ++o) {
          const uint8_t* src = codes[m] + (size_t)o * N + 32 * c;
          uint8_t* dst = cd + ((size_t)c * O + o) * 16;
          for (int b = 0; b < 16; ++b) dst[b] = (uint8_t)(src[2 * b] | (src[2 * b + 1] << 4));
        }
    } else {
      for (int c = 0; c < N / 16; ++c)
        for (int o = 0; o < O; ++o) {
          const uint8_t* src = codes[m] + (size_t)o * N + 16 * c;
          uint8_t* dst = cd + ((size_t)c * O + o) * 16;
          for (int b = 0; b < 16; ++b) dst[b] = src[(b & 8) + kPerm8[b & 7]];
        }
    }
    uint16_t* sb = reinterpret_cast<uint16_t*>(blob + L.m[m].sb);
    for (int g = 0; g < N / 64; ++g)
      for (int o = 0; o < O; ++o) {
        sb[((size_t)g * O + o) * 2 + 0] = scales[m][(size_t)o * (N / 64) + g];
        sb[((size_t)g * O + o) * 2 + 1] = biases[m][(size_t)o * (N / 64) + g];
      }
  }
  return MOE_OK;
}

extern "C" int moe_unpack_expert(const moe_ffn_shape* sh, const void* in, uint8_t* const codes[3],
                                 uint16_t* const scales[3], uint16_t* const biases[3]) {
  if (!shape_ok(sh) || !in || !codes || !scales || !biases) return MOE_ERR_INVALID_ARG;
  const int bits = shape_bits(sh);
  if (bits == 32) return MOE_ERR_INVALID_ARG;     // f32 experts: moe_unpack_expert_f32
  const BlobLayout L = blob_layout(sh->d, sh->I, bits);
  const int outs[3] = {sh->I, sh->I, sh->d};
  const int ins[3] = {sh->d, sh->d, sh->I};
  const uint8_t* blob = static_cast<const uint8_t*>(in);
  for (int m = 0; m < 3; ++m) {
    if (!codes[m] || !scales[m] || !biases[m]) return MOE_ERR_INVALID_ARG;
    const int O = outs[m], N = ins[m];
    const uint8_t* cd = blob + L.m[m].codes;
    if (bits == 4) {
      for (int c = 0; c < N / 32; ++c)
        for (int o = 0; o < O; ++o) {
          const uint8_t* src = cd + ((size_t)c * O + o) * 16;
          uint8_t* dst = codes[m] + (size_t)o * N + 32 * c;
          for (int b = 0; b < 16; ++b) {
            dst[2 * b] = src[b] & 0xF;
            dst[2 * b + 1] = src[b] >> 4;
          }
        }
    } else {
      for (int c = 0; c < N / 16; ++c)
        for (int o = 0; o < O; ++o) {
          const uint8_t* src = cd + ((size_t)c * O + o) * 16;
          uint8_t* dst = codes[m] + (size_t)o * N + 16 * c;
          for (int b = 0; b < 16; ++b) dst[(b & 8) + kPerm8[b & 7]] = src[b];
        }
    }
    const uint16_t* sb = reinterpret_cast<const uint16_t*>(blob + L.m[m].sb);
    for (int g = 0; g < N / 64; ++g)
      for (int o = 0; o < O; ++o) {
        scales[m][(size_t)o * (N / 64) + g] = sb[((size_t)g * O + o) * 2 + 0];
        biases[m][(size_t)o * (N / 64) + g] = sb[((size_t)g * O + o) * 2 + 1];
      }
  }
  return MOE_OK;
}

extern "C" int moe_pack_expert_f32(const moe_ffn_shape* sh, const float* const w[3], void* out) {
  if (!shape_ok(sh) || shape_bits(sh) != 32 || !w || !out) return MOE_ERR_INVALID_ARG;
  const BlobLayout L = blob_layout(sh->d, sh->I, 32);
  const size_t n[3] = {(size_t)sh->I * sh->d, (size_t)sh->I * sh->d, (size_t)sh->d * sh->I};
  for (int m = 0; m < 3; ++m)
    if (!w[m]) return MOE_ERR_INVALID_ARG;
  uint8_t* blob = static_cast<uint8_t*>(out);
  std::memset(blob, 0, L.stride);
  for (int m = 0; m < 3; ++m) std::memcpy(blob + L.m[m].codes, w[m], n[m] * sizeof(float));
  return MOE_OK;
}

extern "C" int moe_unpack_expert_f32(const moe_ffn_shape* sh, const void* in, float* const w[3]) {
  if (!shape_ok(sh) || shape_bits(sh) != 32 || !w || !in) return MOE_ERR_INVALID_ARG;
  const BlobLayout L = blob_layout(sh->d, sh->I, 32);
  const size_t n[3] = {(size_t)sh->I * sh->d, (size_t)sh->I * sh->d, (size_t)sh->d * sh->I};
  const uint8_t* blob = static_cast<const uint8_t*>(in);
  for (int m = 0; m < 3; ++m) {
    if (!w[m]) return MOE_ERR_INVALID_ARG;
    std::memcpy(w[m], blob + L.m[m].codes, n[m] * sizeof(float));
  }
  return MOE_OK;
}

extern "C" int moe_pack_expert_int4(const moe_ffn_shape* sh, const uint8_t* const codes[3],
                                    const uint16_t* const scales[3], const uint16_t* const biases[3],
                                    void* out) {
  if (!shape_ok(sh) || shape_bits(sh) != 4) return MOE_ERR_INVALID_ARG;
  return moe_pack_expert(sh, codes, scales, biases, out);
}

extern "C" int moe_unpack_expert_int4(const moe_ffn_shape* sh, const void* in, uint8_t* const codes[3],
                                      uint16_t* const scales[3], uint16_t* const biases[3]) {
  if (!shape_ok(sh) || shape_bits(sh) != 4) return MOE_ERR_INVALID_ARG;
  return moe_unpack_expert(sh, in, codes, scales, biases);
}

// -------------------------------------------------------- LFU + recency
// Host-only policy state: residency map, selection counts, last-use steps.
struct moe_lfu {
  int32_t E = 0, n_slots = 0;
  std::vector<uint64_t> count;
  std::vector<int64_t> last;
  std::vector<int32_t> slot_of;  // expert -> slot or -1
  std::vector<int32_t> holder;   // slot -> expert or -1
  int64_t step = 0;
  moe_pool_stats st{};
};

extern "C" int moe_lfu_create(int32_t E, int32_t n_slots, moe_lfu** out) {
  return no_throw([&]() -> int {
    if (!out || E < 1 || E > 1024 || n_slots < 1) return MOE_ERR_INVALID_ARG;
    std::unique_ptr<moe_lfu> l(new (std::nothrow) moe_lfu());
    if (!l) return MOE_ERR_OUT_OF_MEMORY;
    l->E = E;
    l->n_slots = n_slots;
    l->count.assign(E, 0);
    l->last.assign(E, -1);
    l->slot_of.assign(E, -1);
    l->holder.assign(n_slots, -1);
    *out = l.release();
    return MOE_OK;
  });
}

extern "C" int moe_lfu_destroy(moe_lfu* l) {
  if (!l) return MOE_ERR_INVALID_ARG;
  delete l;
  return MOE_OK;
}

extern "C" int moe_lfu_get_stats(const moe_lfu* l, moe_pool_stats* st) {
  if (!l || !st) return MOE_ERR_INVALID_ARG;
  *st = l->st;
  return MOE_OK;
}

extern "C" int moe_lfu_plan(moe_lfu* p, const int32_t* sel, int32_t n, int32_t* le, int32_t* ls,
                            int32_t* lv, int32_t* n_loads) {
  return no_throw([&]() -> int {
    if (!p || n < 0 || (n > 0 && !sel) || !n_loads) return MOE_ERR_INVALID_ARG;
    if (n > 0 && (!le || !ls || !lv)) return MOE_ERR_INVALID_ARG;
    // distinct needed experts in first-appearance order
    std::vector<int32_t> need;
    std::vector<char> is_need(p->E, 0);
    for (int q = 0; q < n; ++q) {
      const int32_t e = sel[q];
      if (e < 0 || e >= p->E) return MOE_ERR_INVALID_ARG;
      if (!is_need[e]) {
        is_need[e] = 1;
        need.push_back(e);
      }
    }
    if ((int)need.size() > p->n_slots) return MOE_ERR_POOL_TOO_SMALL;
    for (int q = 0; q < n; ++q) {
      p->count[sel[q]] += 1;
      p->last[sel[q]] = p->step;
    }
    int nl = 0;
    for (int32_t e : need) {
      if (p->slot_of[e] >= 0) {
        p->st.hits += 1;
        continue;
      }
      p->st.misses += 1;
      int32_t slot = -1, victim = -1;
      for (int s = 0; s < p->n_slots; ++s)
        if (p->holder[s] < 0) { slot = s; break; }
      if (slot < 0) {
        // least frequent, then least recent, then lowest id, among resident
        // experts this step does not need
        for (int32_t v = 0; v < p->E; ++v) {
          if (p->slot_of[v] < 0 || is_need[v]) continue;
          if (victim < 0 || p->count[v] < p->count[victim] ||
              (p->count[v] == p->count[victim] && p->last[v] < p->last[victim]))
            victim = v;
        }
        slot = p->slot_of[victim];
        p->slot_of[victim] = -1;
        p->st.evictions += 1;
      }
      p->holder[slot] = e;
      p->slot_of[e] = slot;
      le[nl] = e;
      ls[nl] = slot;
      lv[nl] = victim;
      ++nl;
    }
    p->step += 1;
    p->st.steps += 1;
    *n_loads = nl;
    return MOE_OK;
  });
}

// ------------------------------------------------------------------- pool
struct moe_pool {
  int32_t E = 0, n_slots = 0;
  moe_ffn_shape sh{};
  size_t stride = 0;
  uint8_t* slab = nullptr;
  int32_t* table = nullptr;     // device [E]
  uint32_t* usage = nullptr;    // device [E]
  int32_t* err = nullptr;       // device [1]
  moe_lfu lfu;                  // host residency + policy state
  // streamed steps (moe_layer_forward_streamed): pinned staging of a step's
  // selections and two events, made on first use
  int32_t* sel_host = nullptr;  // pinned [8 * 1024]
  hipEvent_t ev_sel = nullptr, ev_gu = nullptr, ev_copy = nullptr;
  // refills planned on the device (moe_layer_forward_offload): a device copy
  // of the policy state, made on first use.  One of the two copies is always
  // current; the other is brought up to date before it is used.
  DevLfu dev{};
  void* dev_mem = nullptr;
  bool dev_valid = false, host_valid = true;
};

// The host copy of the policy state, current (waits for the device's steps).
static int lfu_on_host(moe_pool* p) {
  if (p->host_valid) return MOE_OK;
  MOE_HIP(hipDeviceSynchronize());
  moe_lfu& l = p->lfu;
  uint64_t meta[7];
  MOE_HIP(hipMemcpy(l.count.data(), p->dev.count, sizeof(uint64_t) * p->E, hipMemcpyDeviceToHost));
  MOE_HIP(hipMemcpy(l.last.data(), p->dev.last, sizeof(int64_t) * p->E, hipMemcpyDeviceToHost));
  MOE_HIP(hipMemcpy(l.slot_of.data(), p->dev.slot_of, sizeof(int32_t) * p->E, hipMemcpyDeviceToHost));
  MOE_HIP(hipMemcpy(l.holder.data(), p->dev.holder, sizeof(int32_t) * p->n_slots, hipMemcpyDeviceToHost));
  MOE_HIP(hipMemcpy(meta, p->dev.meta, sizeof(meta), hipMemcpyDeviceToHost));
  l.step = (int64_t)meta[0];
  l.st.steps = meta[1];
  l.st.hits = meta[2];
  l.st.misses = meta[3];
  l.st.loads = meta[4];
  l.st.evictions = meta[5];
  l.st.bytes_loaded = meta[6];
  p->host_valid = true;
  return MOE_OK;
}

// The device copy, current (allocated on first use).
static int lfu_on_device(moe_pool* p) {
  const size_t E = (size_t)p->E, S = (size_t)p->n_slots;
  auto up = [](size_t b) { return (b + 255) & ~(size_t)255; };
  const size_t o_last = up(8 * E), o_slot = o_last + up(8 * E), o_holder = o_slot + up(4 * E),
               o_meta = o_holder + up(4 * S), o_plan = o_meta + up(8 * 8), total = o_plan + up(4 * (1 + 3 * E));
  if (!p->dev_mem) {
    MOE_HIP(hipMalloc(&p->dev_mem, total));
    uint8_t* b = static_cast<uint8_t*>(p->dev_mem);
    p->dev.count = reinterpret_cast<uint64_t*>(b);
    p->dev.last = reinterpret_cast<int64_t*>(b + o_last);
    p->dev.slot_of = reinterpret_cast<int32_t*>(b + o_slot);
    p->dev.holder = reinterpret_cast<int32_t*>(b + o_holder);
    p->dev.meta = reinterpret_cast<uint64_t*>(b + o_meta);
    p->dev.plan = reinterpret_cast<int32_t*>(b + o_plan);
    p->dev_valid = false;
  }
  if (p->dev_valid) return MOE_OK;
  MOE_TRY(lfu_on_host(p));
  const moe_lfu& l = p->lfu;
  const uint64_t meta[7] = {(uint64_t)l.step, l.st.steps, l.st.hits, l.st.misses,
                            l.st.loads, l.st.evictions, l.st.bytes_loaded};
  MOE_HIP(hipDeviceSynchronize());
  MOE_HIP(hipMemcpy(p->dev.count, l.count.data(), sizeof(uint64_t) * E, hipMemcpyHostToDevice));
  MOE_HIP(hipMemcpy(p->dev.last, l.last.data(), sizeof(int64_t) * E, hipMemcpyHostToDevice));
  MOE_HIP(hipMemcpy(p->dev.slot_of, l.slot_of.data(), sizeof(int32_t) * E, hipMemcpyHostToDevice));
  MOE_HIP(hipMemcpy(p->dev.holder, l.holder.data(), sizeof(int32_t) * S, hipMemcpyHostToDevice));
  MOE_HIP(hipMemcpy(p->dev.meta, meta, sizeof(meta), hipMemcpyHostToDevice));
  p->dev_valid = true;
  return MOE_OK;
}

// A host-side policy call: the host copy first, and the device copy stale after.
#define LFU_HOST_EDIT(p)        \
  do {                          \
    MOE_TRY(lfu_on_host(p));    \
    (p)->dev_valid = false;     \
  } while (0)

namespace moe {
bool pool_view(const moe_pool* p, PoolView* v) {
  if (!p) return false;
  v->slab = p->slab;
  v->stride = p->stride;
  v->slot_table = p->table;
  v->err = p->err;
  v->E = p->E;
  return true;
}
}  // namespace moe

extern "C" int moe_pool_create(int32_t E, int32_t n_slots, const moe_ffn_shape* sh, moe_pool** out) {
  return no_throw([&]() -> int {
    if (!out || E < 1 || E > 1024 || n_slots < 1 || !shape_ok(sh)) return MOE_ERR_INVALID_ARG;
    *out = nullptr;
    std::unique_ptr<moe_pool> owner(new (std::nothrow) moe_pool());
    if (!owner) return MOE_ERR_OUT_OF_MEMORY;
    owner->lfu.count.assign(E, 0);               // host state first: may throw, nothing on the device yet
    owner->lfu.last.assign(E, -1);
    owner->lfu.slot_of.assign(E, -1);
    owner->lfu.holder.assign(n_slots, -1);
    moe_pool* p = owner.release();
    p->E = E;
    p->n_slots = n_slots;
    p->sh = *sh;
    p->stride = blob_layout(sh->d, sh->I, shape_bits(sh)).stride;
    p->lfu.E = E;
    p->lfu.n_slots = n_slots;
    hipError_t e = hipMalloc(&p->slab, p->stride * (size_t)n_slots);
    if (e == hipSuccess) e = hipMalloc(&p->table, sizeof(int32_t) * E);
    if (e == hipSuccess) e = hipMalloc(&p->usage, sizeof(uint32_t) * E);
    if (e == hipSuccess) e = hipMalloc(&p->err, 256);
    if (e == hipSuccess) e = hipMemset(p->table, 0xFF, sizeof(int32_t) * E);
    if (e == hipSuccess) e = hipMemset(p->usage, 0, sizeof(uint32_t) * E);
    if (e == hipSuccess) e = hipMemset(p->err, 0, 256);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      moe_pool_destroy(p);
      return hip_fail(e);
    }
    *out = p;
    return MOE_OK;
  });
}

extern "C" int moe_pool_destroy(moe_pool* p) {
  if (!p) return MOE_ERR_INVALID_ARG;
  if (p->slab) (void)hipFree(p->slab);
  if (p->table) (void)hipFree(p->table);
  if (p->usage) (void)hipFree(p->usage);
  if (p->err) (void)hipFree(p->err);
  if (p->sel_host) (void)hipHostFree(p->sel_host);
  if (p->ev_sel) (void)hipEventDestroy(p->ev_sel);
  if (p->ev_gu) (void)hipEventDestroy(p->ev_gu);
  if (p->ev_copy) (void)hipEventDestroy(p->ev_copy);
  if (p->dev_mem) (void)hipFree(p->dev_mem);
  delete p;
  return MOE_OK;
}

extern "C" void* moe_pool_slab(const moe_pool* p) { return p ? p->slab : nullptr; }
extern "C" size_t moe_pool_stride(const moe_pool* p) { return p ? p->stride : 0; }
extern "C" int32_t* moe_pool_slot_table(const moe_pool* p) { return p ? p->table : nullptr; }
extern "C" uint32_t* moe_pool_usage(const moe_pool* p) { return p ? p->usage : nullptr; }
extern "C" int32_t moe_pool_num_experts(const moe_pool* p) { return p ? p->E : 0; }
extern "C" int32_t moe_pool_num_slots(const moe_pool* p) { return p ? p->n_slots : 0; }

static void host_place(moe_lfu* p, int32_t e, int32_t slot, std::vector<int32_t>* te,
                       std::vector<int32_t>* ts) {
  const int32_t prev = p->holder[slot];
  if (prev >= 0 && prev != e) {
    p->slot_of[prev] = -1;
    te->push_back(prev);
    ts->push_back(-1);
  }
  if (p->slot_of[e] >= 0 && p->slot_of[e] != slot) {
    p->holder[p->slot_of[e]] = -1;
  }
  p->holder[slot] = e;
  p->slot_of[e] = slot;
  te->push_back(e);
  ts->push_back(slot);
}

static int load_common(moe_pool* p, int32_t e, int32_t slot, const void* blob, hipMemcpyKind kind,
                       hipStream_t s) {
  if (!p || !blob || e < 0 || e >= p->E || slot < 0 || slot >= p->n_slots) return MOE_ERR_INVALID_ARG;
  LFU_HOST_EDIT(p);
  MOE_HIP(hipMemcpyAsync(p->slab + (size_t)slot * p->stride, blob, p->stride, kind, s));
  std::vector<int32_t> te, ts;
  host_place(&p->lfu, e, slot, &te, &ts);
  p->lfu.st.loads += 1;
  p->lfu.st.bytes_loaded += p->stride;
  return table_edit_launch(p->table, te.data(), ts.data(), (int)te.size(), s);
}

extern "C" int moe_pool_load(moe_pool* p, int32_t e, int32_t slot, const void* blob, hipStream_t s) {
  return no_throw([&]() -> int {
    return load_common(p, e, slot, blob, hipMemcpyHostToDevice, s);
  });
}

extern "C" int moe_pool_load_device(moe_pool* p, int32_t e, int32_t slot, const void* blob,
                                    hipStream_t s) {
  return no_throw([&]() -> int {
    return load_common(p, e, slot, blob, hipMemcpyDeviceToDevice, s);
  });
}

extern "C" int moe_pool_plan(moe_pool* p, const int32_t* sel, int32_t n, int32_t* le, int32_t* ls,
                             int32_t* lv, int32_t* n_loads) {
  if (!p) return MOE_ERR_INVALID_ARG;
  LFU_HOST_EDIT(p);
  return moe_lfu_plan(&p->lfu, sel, n, le, ls, lv, n_loads);
}

// Plan one step's refill and copy the missing blobs on copy_s; the table
// edits (victims out, new residents in) are collected for the caller to
// publish on the stream that must see them.  With split_ev, every blob's
// gate/up sections are copied first and split_ev is recorded on copy_s
// before the down sections follow (gate/up can then start while down is on
// the way).
static int plan_and_copy(moe_pool* p, const int32_t* sel, int32_t n, const void* host_blobs, size_t host_stride,
                         hipStream_t copy_s, std::vector<int32_t>* te, std::vector<int32_t>* ts, int32_t* nl,
                         hipEvent_t split_ev = nullptr) {
  std::vector<int32_t> le(n > 0 ? n : 1), ls(n > 0 ? n : 1), lv(n > 0 ? n : 1);
  *nl = 0;
  MOE_TRY(moe_pool_plan(p, sel, n, le.data(), ls.data(), lv.data(), nl));
  const size_t down_off = split_ev ? blob_layout(p->sh.d, p->sh.I, shape_bits(&p->sh)).m[2].codes : p->stride;
  // The copies: one kernel per byte range reading the pinned host blobs over
  // PCIe (54 GB/s on the MI355X against 44 GB/s for one copy-engine transfer
  // per blob) when the host memory is mapped for the device and 16-byte
  // aligned; otherwise hipMemcpyAsync per blob and range.
  void* src_dev = nullptr;
  bool pulled = false;
  if (*nl > 0) {
    if (hipHostGetDevicePointer(&src_dev, const_cast<void*>(host_blobs), 0) == hipSuccess && src_dev) {
      pulled = blob_pull_launch(src_dev, host_stride, p->slab, p->stride, 0, down_off, le.data(), ls.data(),
                                *nl, copy_s) == MOE_OK;
    } else {
      (void)hipGetLastError();                    // not mapped: clear the error, use the copy engine
    }
    if (!pulled)
      for (int q = 0; q < *nl; ++q)
        MOE_HIP(hipMemcpyAsync(p->slab + (size_t)ls[q] * p->stride,
                               static_cast<const uint8_t*>(host_blobs) + (size_t)le[q] * host_stride, down_off,
                               hipMemcpyHostToDevice, copy_s));
    if (split_ev) {
      MOE_HIP(hipEventRecord(split_ev, copy_s));
      const size_t rest = p->stride - down_off;
      if (!(pulled && blob_pull_launch(src_dev, host_stride, p->slab, p->stride, down_off, rest, le.data(),
                                       ls.data(), *nl, copy_s) == MOE_OK))
        for (int q = 0; q < *nl; ++q)
          MOE_HIP(hipMemcpyAsync(p->slab + (size_t)ls[q] * p->stride + down_off,
                                 static_cast<const uint8_t*>(host_blobs) + (size_t)le[q] * host_stride + down_off,
                                 rest, hipMemcpyHostToDevice, copy_s));
    }
  }
  for (int q = 0; q < *nl; ++q) {
    if (lv[q] >= 0) {
      te->push_back(lv[q]);
      ts->push_back(-1);
    }
    te->push_back(le[q]);
    ts->push_back(ls[q]);
    p->lfu.st.loads += 1;
    p->lfu.st.bytes_loaded += p->stride;
  }
  return MOE_OK;
}

extern "C" int moe_pool_refill(moe_pool* p, const int32_t* sel, int32_t n, const void* host_blobs,
                               size_t host_stride, hipStream_t s) {
  return no_throw([&]() -> int {
    if (!p || !host_blobs || host_stride < p->stride) return MOE_ERR_INVALID_ARG;
    std::vector<int32_t> te, ts;
    int32_t nl = 0;
    MOE_TRY(plan_and_copy(p, sel, n, host_blobs, host_stride, s, &te, &ts, &nl));
    if (!te.empty()) MOE_TRY(table_edit_launch(p->table, te.data(), ts.data(), (int)te.size(), s));
    return MOE_OK;
  });
}

extern "C" int moe_pool_set_slot_table(moe_pool* p, const int32_t* table, hipStream_t s) {
  return no_throw([&]() -> int {
    if (!p || !table) return MOE_ERR_INVALID_ARG;
    LFU_HOST_EDIT(p);
    std::vector<char> used(p->n_slots, 0);
    for (int e = 0; e < p->E; ++e) {
      const int32_t sl = table[e];
      if (sl < -1 || sl >= p->n_slots) return MOE_ERR_INVALID_ARG;
      if (sl >= 0) {
        if (used[sl]) return MOE_ERR_INVALID_ARG;
        used[sl] = 1;
      }
    }
    std::fill(p->lfu.holder.begin(), p->lfu.holder.end(), -1);
    for (int e = 0; e < p->E; ++e) {
      p->lfu.slot_of[e] = table[e];
      if (table[e] >= 0) p->lfu.holder[table[e]] = e;
    }
    MOE_HIP(hipMemcpyAsync(p->table, table, sizeof(int32_t) * p->E, hipMemcpyHostToDevice, s));
    MOE_HIP(hipStreamSynchronize(s));
    return MOE_OK;
  });
}

extern "C" int moe_pool_get_stats(const moe_pool* p, moe_pool_stats* st) {
  if (!p || !st) return MOE_ERR_INVALID_ARG;
  MOE_TRY(lfu_on_host(const_cast<moe_pool*>(p)));
  *st = p->lfu.st;
  return MOE_OK;
}

extern "C" int moe_pool_check_error(moe_pool* p, hipStream_t s, int32_t* err) {
  if (!p || !err) return MOE_ERR_INVALID_ARG;
  int32_t v = 0;
  MOE_HIP(hipStreamSynchronize(s));
  MOE_HIP(hipMemcpy(&v, p->err, sizeof(v), hipMemcpyDeviceToHost));
  MOE_HIP(hipMemset(p->err, 0, sizeof(v)));
  // bit 0: a selected expert had no slot; bit 1: a prefill activation or
  // intermediate fell outside the fp16 range
  *err = (v & 1) ? MOE_ERR_NOT_RESIDENT : (v & 2) ? MOE_ERR_UNSUPPORTED : MOE_OK;
  return MOE_OK;
}

extern "C" int moe_pool_read_state(const moe_pool* p, int32_t* table, uint32_t* usage, hipStream_t s) {
  if (!p) return MOE_ERR_INVALID_ARG;
  MOE_HIP(hipStreamSynchronize(s));
  if (table) MOE_HIP(hipMemcpy(table, p->table, sizeof(int32_t) * p->E, hipMemcpyDeviceToHost));
  if (usage) MOE_HIP(hipMemcpy(usage, p->usage, sizeof(uint32_t) * p->E, hipMemcpyDeviceToHost));
  return MOE_OK;
}

extern "C" int moe_pool_reset_usage(moe_pool* p, hipStream_t s) {
  if (!p) return MOE_ERR_INVALID_ARG;
  MOE_HIP(hipMemsetAsync(p->usage, 0, sizeof(uint32_t) * p->E, s));
  return MOE_OK;
}

// -------------------------------------------------------------- expert FFN
extern "C" size_t moe_ffn_workspace_bytes(const moe_ffn_shape* sh, const moe_ffn_shape* ssh, int32_t T,
                                          int32_t k, int32_t E, int32_t path) {
  if (!shape_ok(sh) || !shape_ok(ssh) || sh->d != ssh->d || T < 0 || k < 1 || E < 1) return 0;
  path = resolve_path(path, T, sh->d, k, E, shape_bits(sh), sh->I > ssh->I ? sh->I : ssh->I);
  return ffn_ws_bytes(sh->d, sh->I, ssh->I, T, k, E, path);
}

static int check_ffn(const moe_pool* pool, const moe_ffn_shape* sh, const moe_ffn_shape* ssh,
                     const void* shared_blob, int T, int k) {
  if (!pool || !shape_ok(sh) || !shape_ok(ssh) || sh->d != ssh->d) return MOE_ERR_INVALID_ARG;
  if (pool->sh.d != sh->d || pool->sh.I != sh->I || shape_bits(&pool->sh) != shape_bits(sh))
    return MOE_ERR_INVALID_ARG;
  if (T < 0 || k < 1 || k > pool->E || !shared_blob || !aligned(shared_blob, 16)) return MOE_ERR_INVALID_ARG;
  if (sh->d > 8192) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

extern "C" int moe_expert_ffn(const moe_pool* pool, const moe_ffn_shape* sh, const void* shared_blob,
                              const moe_ffn_shape* ssh, const uint16_t* x, int32_t T, int32_t k,
                              const int32_t* idx, const float* w, const float* sgate,
                              const int32_t* offsets, const int32_t* pair_ids, float* out,
                              float* partial, float* shared_out, int32_t path, void* ws,
                              size_t ws_bytes, hipStream_t s) {
  MOE_TRY(check_ffn(pool, sh, ssh, shared_blob, T, k));
  if (T == 0) return MOE_OK;
  path = resolve_path(path, T, sh->d, k, pool->E, shape_bits(sh), sh->I > ssh->I ? sh->I : ssh->I);
  MOE_CHECK(x && idx && ws && aligned(x, 16) && aligned(ws, 256));
  FfnArgs a{};
  pool_view(pool, &a.pool);
  a.d = sh->d; a.I = sh->I; a.Ish = ssh->I;
  a.bits = shape_bits(sh); a.bits_sh = shape_bits(ssh);
  a.shared_blob = static_cast<const uint8_t*>(shared_blob);
  a.x = x; a.xq = nullptr; a.xs = nullptr;
  a.T = T; a.k = k; a.idx = const_cast<int32_t*>(idx); a.w = const_cast<float*>(w);
  a.sgate = const_cast<float*>(sgate);
  a.offsets = offsets; a.pair_ids = pair_ids;
  a.y = out; a.partial = partial; a.shared_out = shared_out;
  if (path == MOE_PATH_DECODE) {
    MOE_CHECK(T <= 8 && w && sgate && out && (long)T * (k + 1) <= 2048);
  } else if (path == MOE_PATH_BATCHED || is_mfma_path(path)) {
    MOE_CHECK(offsets && pair_ids && partial && shared_out);
    MOE_CHECK(aligned(partial, 16) && aligned(shared_out, 16));
  } else {
    return MOE_ERR_INVALID_ARG;
  }
  return ffn_launch(a, path, ws, ws_bytes, s);
}

extern "C" int moe_expert_ffn_int4(const moe_pool* pool, const moe_ffn_shape* sh, const void* shared_blob,
                                   const moe_ffn_shape* ssh, const uint16_t* x, int32_t T, int32_t k,
                                   const int32_t* idx, const float* w, const float* sgate,
                                   const int32_t* offsets, const int32_t* pair_ids, float* out,
                                   float* partial, float* shared_out, int32_t path, void* ws,
                                   size_t ws_bytes, hipStream_t s) {
  if (!shape_ok(sh) || !shape_ok(ssh) || shape_bits(sh) != 4 || shape_bits(ssh) != 4)
    return MOE_ERR_INVALID_ARG;
  return moe_expert_ffn(pool, sh, shared_blob, ssh, x, T, k, idx, w, sgate, offsets, pair_ids, out,
                        partial, shared_out, path, ws, ws_bytes, s);
}

// ------------------------------------------------------------- whole layer
struct LayerWs {
  RouterWs r;
  int32_t* counts; int32_t* offsets; int32_t* pair_ids;
  float* partial; float* shared_out;
  void* bucket_ws; size_t bucket_bytes;
  void* ffn_ws; size_t ffn_bytes;
};

static bool carve_layer(Carver& c, const moe_layer_desc* L, int T, int path, LayerWs* w) {
  const int d = L->sh.d, E = L->E, k = L->k;
  router_ws_carve(c, T, d, E, &w->r);
  w->counts = w->offsets = w->pair_ids = nullptr;
  w->partial = w->shared_out = nullptr;
  w->bucket_ws = nullptr;
  w->bucket_bytes = 0;
  if (path != MOE_PATH_DECODE) {
    w->counts = c.take<int32_t>(E);
    w->offsets = c.take<int32_t>(E + 1);
    w->pair_ids = c.take<int32_t>((size_t)T * k);
    w->partial = c.take<float>((size_t)T * k * d);
    w->shared_out = c.take<float>((size_t)T * d);
    w->bucket_bytes = bucket_ws_bytes(T, k, E);
    w->bucket_ws = c.take<uint8_t>(w->bucket_bytes);
  }
  w->ffn_bytes = ffn_ws_bytes(d, L->sh.I, L->shared_sh.I, T, k, E, path);
  w->ffn_ws = c.take<uint8_t>(w->ffn_bytes);
  return c.ok();
}

static int layer_imax(const moe_layer_desc* L) { return L->sh.I > L->shared_sh.I ? L->sh.I : L->shared_sh.I; }

static int check_layer(const moe_layer_desc* L) {
  if (!L || !L->pool || !L->w_router_dev || !L->shared_blob_dev) return MOE_ERR_INVALID_ARG;
  if (!shape_ok(&L->sh) || !shape_ok(&L->shared_sh) || L->sh.d != L->shared_sh.d) return MOE_ERR_INVALID_ARG;
  if (L->E != L->pool->E || L->k < 1 || L->k > L->E) return MOE_ERR_INVALID_ARG;
  if (L->pool->sh.d != L->sh.d || L->pool->sh.I != L->sh.I || shape_bits(&L->pool->sh) != shape_bits(&L->sh))
    return MOE_ERR_INVALID_ARG;
  if (L->sh.d > 8192) return MOE_ERR_UNSUPPORTED;
  return MOE_OK;
}

extern "C" size_t moe_layer_workspace_bytes(const moe_layer_desc* L, int32_t T, int32_t path) {
  if (check_layer(L) != MOE_OK || T < 0) return 0;
  path = resolve_path(path, T, L->sh.d, L->k, L->E, shape_bits(&L->sh), layer_imax(L));
  Carver c(nullptr, (size_t)-1);
  LayerWs w;
  carve_layer(c, L, T, path, &w);
  return c.off + 256;
}

namespace moe {
int layer_forward(const moe_layer_desc* L, const uint16_t* x, int T, float* y, int32_t* idx, float* w,
                  float* sgate, int path, void* ws, size_t ws_bytes, hipStream_t s, const ChainIO* io) {
  MOE_TRY(check_layer(L));
  MOE_CHECK(T >= 0);
  if (T == 0) return MOE_OK;
  MOE_CHECK(x && y && idx && w && sgate && ws);
  MOE_CHECK(aligned(x, 16) && aligned(y, 16) && aligned(ws, 256) && aligned(L->w_router_dev, 16));
  path = resolve_path(path, T, L->sh.d, L->k, L->E, shape_bits(&L->sh), layer_imax(L));
  if (path == MOE_PATH_DECODE) MOE_CHECK(T <= 8 && (long)T * (L->k + 1) <= 2048);
  // the chain hand-over exists on the decode path of 4- and 8-bit experts
  if (io) MOE_CHECK(path == MOE_PATH_DECODE && shape_bits(&L->sh) != 32 && shape_bits(&L->shared_sh) != 32);
  Carver c(ws, ws_bytes);
  LayerWs lw;
  if (!carve_layer(c, L, T, path, &lw)) return MOE_ERR_INVALID_ARG;
  const int d = L->sh.d;
  const bool f32 = shape_bits(&L->sh) == 32;
  // one token: the decode FFN selects the experts in-kernel (its blocks all
  // run at once, so the selection costs one pass); more tokens take several
  // rounds of gate/up blocks, each of which would repeat it: one top-k
  // kernel, then the FFN with the routing given
  const bool sel_in_ffn = path == MOE_PATH_DECODE && !f32 && T == 1;
  if (path == MOE_PATH_DECODE && !f32) {
    MOE_TRY(router_logits_launch(x, T, d, L->w_router_dev, L->E, lw.r, s, true, io ? io->ssp_in : nullptr,
                                 io ? io->eps : 0.f));
    if (!sel_in_ffn)
      MOE_TRY(topk_launch(lw.r.logits, L->logit_bias_dev, T, d, L->E, L->k, idx, w, sgate, L->usage_dev, s));
  } else if (path == MOE_PATH_DECODE) {
    // f32 experts: top-k here, then the FFN with the routing given
    MOE_TRY(router_launch(x, T, d, L->w_router_dev, L->logit_bias_dev, L->E, L->k, idx, w, sgate,
                          L->usage_dev, lw.r, s, false));
  } else {
    // usage is counted from the buckets below (one atomic per expert); the
    // bf16 activation pairs are prepared only for the bucketed GEMVs
    MOE_TRY(router_launch(x, T, d, L->w_router_dev, L->logit_bias_dev, L->E, L->k, idx, w, sgate,
                          nullptr, lw.r, s, path == MOE_PATH_BATCHED));
  }
  FfnArgs a{};
  pool_view(L->pool, &a.pool);
  a.d = d; a.I = L->sh.I; a.Ish = L->shared_sh.I;
  a.bits = shape_bits(&L->sh); a.bits_sh = shape_bits(&L->shared_sh);
  a.shared_blob = static_cast<const uint8_t*>(L->shared_blob_dev);
  a.x = x; a.xq = lw.r.xq; a.xs = lw.r.xs;
  a.T = T; a.k = L->k; a.idx = idx; a.w = w; a.sgate = sgate;
  if (path == MOE_PATH_DECODE) {
    a.y = y;
    if (sel_in_ffn) {
      a.logits = lw.r.logits;
      a.bias = L->logit_bias_dev;
      a.usage = L->usage_dev;
    } else if (!f32 && !io) {
      a.xq = nullptr;                           // the gate/up blocks form the pairs from x (same bits)
      a.xs = nullptr;
    }
    if (io) {
      a.res_in = io->res_in;
      a.res_out = io->res_out;
      a.ssp_out = io->ssp_out;
    }
    return ffn_launch(a, path, lw.ffn_ws, lw.ffn_bytes, s);
  }
  MOE_TRY(bucket_launch(idx, T, L->k, L->E, lw.counts, lw.offsets, lw.pair_ids, lw.bucket_ws,
                        lw.bucket_bytes, s, L->usage_dev));
  a.offsets = lw.offsets; a.pair_ids = lw.pair_ids;
  a.partial = lw.partial; a.shared_out = lw.shared_out;
  MOE_TRY(ffn_launch(a, path, lw.ffn_ws, lw.ffn_bytes, s));
  return combine_launch(lw.partial, lw.shared_out, w, sgate, T, L->k, d, y, s);
}
}  // namespace moe

extern "C" int moe_layer_forward(const moe_layer_desc* L, const uint16_t* x, int32_t T, float* y,
                                 int32_t* idx, float* w, float* sgate, int32_t path, void* ws,
                                 size_t ws_bytes, hipStream_t s) {
  return layer_forward(L, x, T, y, idx, w, sgate, path, ws, ws_bytes, s, nullptr);
}

extern "C" int moe_layer_forward_streamed(const moe_layer_desc* L, const void* host_blobs, size_t host_stride,
                                          const uint16_t* x, int32_t T, float* y, int32_t* idx, float* w,
                                          float* sgate, void* ws, size_t ws_bytes, hipStream_t s,
                                          hipStream_t copy_s, int32_t* n_loads) {
  return no_throw([&]() -> int {
    MOE_TRY(check_layer(L));
    moe_pool* p = const_cast<moe_pool*>(L->pool);
    MOE_CHECK(T >= 1 && T <= 8 && (long)T * (L->k + 1) <= 2048);
    MOE_CHECK(shape_bits(&L->sh) != 32 && shape_bits(&L->shared_sh) != 32);
    MOE_CHECK(x && y && idx && w && sgate && ws && host_blobs && host_stride >= p->stride);
    MOE_CHECK(aligned(x, 16) && aligned(y, 16) && aligned(ws, 256) && aligned(L->w_router_dev, 16));
    Carver c(ws, ws_bytes);
    LayerWs lw;
    if (!carve_layer(c, L, T, MOE_PATH_DECODE, &lw)) return MOE_ERR_INVALID_ARG;
    if (!p->sel_host) {
      MOE_HIP(hipHostMalloc((void**)&p->sel_host, sizeof(int32_t) * 8 * 1024, hipHostMallocDefault));
      MOE_HIP(hipEventCreateWithFlags(&p->ev_sel, hipEventDisableTiming));
      MOE_HIP(hipEventCreateWithFlags(&p->ev_gu, hipEventDisableTiming));
      MOE_HIP(hipEventCreateWithFlags(&p->ev_copy, hipEventDisableTiming));
    }
    const int d = L->sh.d, k = L->k, n = T * k;
    // 1. routing: selections, weights, shared gate, usage, and the activation
    //    pairs for the GEMVs; the selections go to the host at once
    MOE_TRY(router_launch(x, T, d, L->w_router_dev, L->logit_bias_dev, L->E, k, idx, w, sgate, L->usage_dev,
                          lw.r, s, true));
    MOE_HIP(hipMemcpyAsync(p->sel_host, idx, sizeof(int32_t) * n, hipMemcpyDeviceToHost, s));
    MOE_HIP(hipEventRecord(p->ev_sel, s));
    // 2. phase 1: the resident selections and the shared expert, queued now so
    //    they run while the host plans and the missing blobs copy in
    FfnArgs a{};
    pool_view(p, &a.pool);
    a.d = d; a.I = L->sh.I; a.Ish = L->shared_sh.I;
    a.bits = shape_bits(&L->sh); a.bits_sh = shape_bits(&L->shared_sh);
    a.shared_blob = static_cast<const uint8_t*>(L->shared_blob_dev);
    a.x = x; a.xq = lw.r.xq; a.xs = lw.r.xs;
    a.T = T; a.k = k; a.idx = idx; a.w = w; a.sgate = sgate; a.y = y;
    a.phase = 1;
    MOE_TRY(ffn_launch(a, MOE_PATH_DECODE, lw.ffn_ws, lw.ffn_bytes, s));
    // 3. plan on the host, copy on copy_s (every blob's gate/up sections
    //    first, then the down sections); the compute stream waits for the
    //    gate/up sections before it publishes the new slots and runs the
    //    phase-2 gate/up pass, and for the rest before the down pass
    MOE_HIP(hipEventSynchronize(p->ev_sel));
    std::vector<int32_t> te, ts;
    int32_t nl = 0;
    MOE_TRY(plan_and_copy(p, p->sel_host, n, host_blobs, host_stride, copy_s, &te, &ts, &nl, p->ev_gu));
    if (nl > 0) {
      MOE_HIP(hipEventRecord(p->ev_copy, copy_s));
      MOE_HIP(hipStreamWaitEvent(s, p->ev_gu, 0));
      MOE_TRY(table_edit_launch(p->table, te.data(), ts.data(), (int)te.size(), s));
      a.down_wait = p->ev_copy;
    }
    // 4. phase 2: the deferred selections, then the rank-order combine
    a.phase = 2;
    a.pending = nl;
    MOE_TRY(ffn_launch(a, MOE_PATH_DECODE, lw.ffn_ws, lw.ffn_bytes, s));
    if (n_loads) *n_loads = nl;
    return MOE_OK;
  });
}

extern "C" int moe_layer_forward_offload(const moe_layer_desc* L, const void* host_blobs, size_t host_stride,
                                         const uint16_t* x, int32_t T, float* y, int32_t* idx, float* w,
                                         float* sgate, void* ws, size_t ws_bytes, int32_t* n_loads_dev,
                                         hipStream_t s) {
  return no_throw([&]() -> int {
    MOE_TRY(check_layer(L));
    moe_pool* p = const_cast<moe_pool*>(L->pool);
    MOE_CHECK(T >= 1 && T <= 8 && (long)T * (L->k + 1) <= 2048);
    MOE_CHECK(shape_bits(&L->sh) != 32 && shape_bits(&L->shared_sh) != 32);
    MOE_CHECK(x && y && idx && w && sgate && ws && host_blobs && host_stride >= p->stride);
    MOE_CHECK(aligned(x, 16) && aligned(y, 16) && aligned(ws, 256) && aligned(L->w_router_dev, 16));
    const int n = T * L->k;
    // a step never needs more experts than the pool holds, and the plan's
    // state fits one wave's LDS
    if (n > p->n_slots || !lfu_plan_fits(p->E, p->n_slots, n)) return MOE_ERR_UNSUPPORTED;
    void* src_dev = nullptr;
    if (hipHostGetDevicePointer(&src_dev, const_cast<void*>(host_blobs), 0) != hipSuccess || !src_dev) {
      (void)hipGetLastError();
      return MOE_ERR_INVALID_ARG;                 // not pinned host memory mapped for the device
    }
    MOE_CHECK(aligned(src_dev, 16) && host_stride % 16 == 0);
    Carver c(ws, ws_bytes);
    LayerWs lw;
    if (!carve_layer(c, L, T, MOE_PATH_DECODE, &lw)) return MOE_ERR_INVALID_ARG;
    MOE_TRY(lfu_on_device(p));
    const int d = L->sh.d, k = L->k;
    // 1. routing; 2. the plan (slot table edited on the device); 3. the
    // missing blobs over PCIe; 4. the experts and the combine
    MOE_TRY(router_launch(x, T, d, L->w_router_dev, L->logit_bias_dev, L->E, k, idx, w, sgate, L->usage_dev,
                          lw.r, s, true));
    MOE_TRY(lfu_plan_launch(p->dev, p->E, p->n_slots, p->stride, p->table, p->err, idx, n, n_loads_dev, s));
    p->host_valid = false;
    MOE_TRY(plan_pull_launch(src_dev, host_stride, p->slab, p->stride, 0, p->stride, p->dev.plan, p->E, s));
    FfnArgs a{};
    pool_view(p, &a.pool);
    a.d = d; a.I = L->sh.I; a.Ish = L->shared_sh.I;
    a.bits = shape_bits(&L->sh); a.bits_sh = shape_bits(&L->shared_sh);
    a.shared_blob = static_cast<const uint8_t*>(L->shared_blob_dev);
    a.x = x; a.xq = lw.r.xq; a.xs = lw.r.xs;
    a.T = T; a.k = k; a.idx = idx; a.w = w; a.sgate = sgate; a.y = y;
    return ffn_launch(a, MOE_PATH_DECODE, lw.ffn_ws, lw.ffn_bytes, s);
  });
}
