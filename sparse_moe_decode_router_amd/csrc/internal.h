// Internal declarations shared by the libmoe355 translation units.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stddef.h>

#include "moe355.h"

namespace moe {

// ---------------------------------------------------------------- errors
int hip_fail(hipError_t e);            // records the HIP error, returns MOE_ERR_HIP
#define MOE_HIP(call)                                    \
  do {                                                   \
    hipError_t moe_e_ = (call);                          \
    if (moe_e_ != hipSuccess) return ::moe::hip_fail(moe_e_); \
  } while (0)
#define MOE_CHECK(cond) \
  do { if (!(cond)) return MOE_ERR_INVALID_ARG; } while (0)
#define MOE_TRY(call) \
  do { int moe_s_ = (call); if (moe_s_ != MOE_OK) return moe_s_; } while (0)

inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }

// -------------------------------------------------------------- layout
// Byte offsets of the six sections of an expert blob (see moe355.h).
struct MatLayout {
  uint64_t codes;   // [in/32][out][16] (4-bit), [in/16][out][16] (8-bit) or fp32 [out][in]
  uint64_t sb;      // [in/64][out][2] fp16 (scale, bias)
};
struct BlobLayout {
  MatLayout m[3];   // gate, up, down
  uint64_t bytes, stride;
};

__host__ __device__ inline BlobLayout blob_layout(int d, int I, int bits) {
  BlobLayout L;
  uint64_t off = 0;
  const int outs[3] = {I, I, d};
  const int ins[3] = {d, d, I};
  for (int m = 0; m < 3; ++m) {
    L.m[m].codes = off;
    off += (uint64_t)outs[m] * (uint64_t)ins[m] * (uint64_t)bits / 8;
    L.m[m].sb = off;
    if (bits != 32) off += (uint64_t)(ins[m] / 64) * (uint64_t)outs[m] * 4;   // f32: no scale/bias
  }
  L.bytes = off;
  L.stride = (off + 4095) & ~(uint64_t)4095;
  return L;
}

bool shape_ok(const moe_ffn_shape* sh);
// Code width of a valid shape (bits 0 reads as 4; 32 = unquantised fp32).
inline int shape_bits(const moe_ffn_shape* sh) { return sh->bits == 8 || sh->bits == 32 ? sh->bits : 4; }

// Device view of a pool, passed to kernels by value.
struct PoolView {
  const uint8_t* slab;
  uint64_t stride;
  const int32_t* slot_table;
  int32_t* err;
  int32_t E;
};
bool pool_view(const moe_pool* p, PoolView* v);

// ------------------------------------------------------------ workspace
// Carves a caller workspace into 256-byte aligned pieces.
struct Carver {
  uint8_t* base;
  size_t size, off;
  explicit Carver(void* b, size_t s) : base((uint8_t*)b), size(s), off(0) {}
  template <class T> T* take(size_t n) {
    size_t at = (off + 255) & ~(size_t)255;
    off = at + n * sizeof(T);
    return (base && off <= size) ? (T*)(base + at) : nullptr;
  }
  bool ok() const { return off <= size; }
};

// -------------------------------------------------------- internal entry
// Router pieces used by the layer driver (router.hip).
struct RouterWs {
  float* logits;      // [S][T][E+1] (S split-K partials, S = 1 for T <= 8)
  uint32_t* xq;       // [T][d/2]  bf16 pairs (x[8m+i], x[8m+i+4])
  float* xs;          // [T][d/64] group sums of x
};
// A chain of layers (chain.hip) hands its residual stream from layer to
// layer without a separate launch: the decode down kernel writes
// x_{l+1} = bf16(x_l + y_l) and, per 8 output rows, the sum of their squares
// (sq_tree8 order); the next decode router forms
//   u = bf16(x * 1 / sqrt(sum / d + eps))
// from x and those partial sums (summed in chain_sum_sq order).
struct ChainIO {
  const float* ssp_in;      // router: [T][d/8] partial sums of squares of its input (or null)
  float eps;
  const uint16_t* res_in;   // down: x_l [T][d]
  uint16_t* res_out;        // down: x_{l+1} [T][d]
  float* ssp_out;           // down: [T][d/8]
};
size_t router_ws_bytes(int T, int d, int E);
bool router_ws_carve(Carver& c, int T, int d, int E, RouterWs* ws);
// prep_x: also fill ws.xq / ws.xs for T > 8 (T <= 8 always does, in-kernel)
// Device copy of a pool's LFU + recency state, for refills planned on the GPU
// (moe_layer_forward_offload); the same fields as the host-side policy.
struct DevLfu {
  uint64_t* count;      // [E] selections so far
  int64_t* last;        // [E] step of the last selection, -1 = never
  int32_t* slot_of;     // [E] slot or -1
  int32_t* holder;      // [n_slots] expert or -1
  uint64_t* meta;       // [0] step, [1..6] steps, hits, misses, loads, evictions, bytes loaded
  int32_t* plan;        // the last step's loads: [0] count, then experts [E], slots [E], victims [E]
};
bool lfu_plan_fits(int E, int n_slots, int n);
// One step's plan on the device: selections sel[0..n) (device), the pool's
// slot table edited in place, n_loads_out (device, may be null) = loads.
int lfu_plan_launch(const DevLfu& v, int E, int n_slots, size_t stride, int32_t* table, int32_t* err,
                    const int32_t* sel, int n, int32_t* n_loads_out, hipStream_t s);
// The planned loads' byte range [off, off + bytes) of every blob, host -> slots.
int plan_pull_launch(const void* src_dev, size_t src_stride, void* dst, size_t dst_stride, size_t off,
                     size_t bytes, const int32_t* plan, int E, hipStream_t s);

int router_launch(const uint16_t* x, int T, int d, const float* W, const float* bias,
                  int E, int k, int32_t* idx, float* w, float* sgate, uint32_t* usage,
                  const RouterWs& ws, hipStream_t s, bool prep_x, float* logits_out = nullptr);
// moe_layer_forward with a chain's hand-over (decode path of 4- and 8-bit
// experts only) or none (io == nullptr).
int layer_forward(const moe_layer_desc* L, const uint16_t* x, int T, float* y, int32_t* idx, float* w,
                  float* sgate, int path, void* ws, size_t ws_bytes, hipStream_t s, const ChainIO* io);
// logits [T][E+1] (+ xq/xs) only; the decode FFN selects in-kernel.
// ssp/eps (T <= 8): x is a chain's residual stream, normalised here.
int router_logits_launch(const uint16_t* x, int T, int d, const float* W, int E,
                         const RouterWs& ws, hipStream_t s, bool prep_x,
                         const float* ssp = nullptr, float eps = 0.f);
int topk_launch(const float* logits, const float* bias, int T, int d, int E, int k, int32_t* idx,
                float* w, float* sgate, uint32_t* usage, hipStream_t s, float* logits_out = nullptr);

// usage (optional): usage[e] += the pairs bucketed to e (one atomic per expert)
int bucket_launch(const int32_t* idx, int T, int k, int E, int32_t* counts,
                  int32_t* offsets, int32_t* pair_ids, void* ws, size_t ws_bytes,
                  hipStream_t s, uint32_t* usage);
size_t bucket_ws_bytes(int T, int k, int E);

int combine_launch(const float* partial, const float* shared_out, const float* w,
                   const float* sgate, int T, int k, int d, float* y, hipStream_t s);

// Expert FFN with x already prepared (xq/xs from the router workspace).
struct FfnArgs {
  PoolView pool;
  int d, I, Ish;
  int bits, bits_sh;        // code width of the routed / shared experts (4 or 8)
  const uint8_t* shared_blob;
  const uint16_t* x;        // bf16 [T][d]
  const uint32_t* xq;       // [T][d/2]
  const float* xs;          // [T][d/64]
  int T, k;
  int32_t* idx;             // [T][k] (written when logits is set)
  float* w;                 // [T][k] (written when logits is set)
  float* sgate;             // [T]    (written when logits is set)
  const float* logits;      // decode: [T][E+1] router logits -> select in-kernel
  const float* bias;        // [E] or null (with logits)
  uint32_t* usage;          // [E] or null (with logits)
  const int32_t* offsets;   // [E+1]
  const int32_t* pair_ids;  // [T*k]
  float* y;                 // decode: [T][d]
  float* partial;           // batched: [T*k][d]
  float* shared_out;        // batched: [T][d]
  const uint16_t* res_in;   // decode, chains: residual hand-over (see ChainIO)
  uint16_t* res_out;
  float* ssp_out;
  // decode with routing given, in two phases around a pool refill (the same
  // workspace for both): 1 = resident selections only (missing ones are
  // deferred, not errors), 2 = the deferred ones, then the combine; pending =
  // number of deferred selections (phase 2 skips the gate/up pass at 0)
  int phase;
  int pending;
  hipEvent_t down_wait;     // phase 2: the stream waits for it between the gate/up and down passes
};
size_t ffn_ws_bytes(int d, int I, int Ish, int T, int k, int E, int path);
size_t prefill_ws_bytes(int d, int I, int Ish, int T, int k, int E);
int prefill_launch(const FfnArgs& a, int path, void* ws, size_t ws_bytes, hipStream_t s);
int ffn_launch(const FfnArgs& a, int path, void* ws, size_t ws_bytes, hipStream_t s);
int resolve_path(int path, int T, int d, int k, int E, int bits, int Imax);
// The matrix-core path addresses its activation and intermediate buffers
// through 32-bit buffer descriptors: T d and (T k + T) Imax fp16 values must
// stay below 4 GiB.
bool prefill_fits(int T, int d, int k, int Imax);
// The matrix-core paths: PREFILL (the library picks tiled or streaming
// GEMMs), or one of them forced.
inline bool is_mfma_path(int p) {
  return p == MOE_PATH_PREFILL || p == MOE_PATH_PREFILL_TILED || p == MOE_PATH_PREFILL_STREAM;
}

}  // namespace moe
