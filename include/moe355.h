/*
 * libmoe355 — routed-expert Mixture-of-Experts layer for MI355X (gfx950).
 *
 * The layer (Swiftlet pages, "How it works"): every token is routed to k of E
 * experts (10 of 512 for the 80B model, 8 of 256 for the 35B model); the
 * router and a shared expert stay resident; routed experts are 4-bit MLX
 * affine group-quantised weights, each repacked as one fixed-stride blob so a
 * fetch is one read, cached in a bounded slot pool evicted by LFU + recency
 * (relationship-to-TurboFieldfare section).  Placement never changes the
 * answer (correctness section).
 *
 * Readings where the pages are silent (all calls follow them):
 *   router   l[t,e] = x_t . W_r[e] + b[e]; top-k largest logits, ties to the
 *            lower index, emitted in rank order (logit desc, index asc);
 *            w = softmax over the k chosen logits; shared gate
 *            s_t = sigmoid(x_t . W_r[E]).
 *   expert   SwiGLU: h = silu(W_gate x) * (W_up x), o = W_down h,
 *            W = scale * q + bias per group of 64 inputs, q in 0..15
 *            (4-bit) or 0..255 (8-bit; the pages' kernels cover MLX affine
 *            int4 and int8, relationship-to-TurboFieldfare section).
 *   layer    y_t = sum_{r<k} w[t,r] o_{e_r}(x_t) + s_t o_shared(x_t), summed in
 *            that order, in fp32.
 *
 * Conventions
 *   - Every pointer named *_dev / documented "device" is device memory; every
 *     other pointer is host memory.  The caller owns all buffers except a
 *     pool's slab, slot table, usage counters and error word, which the pool
 *     owns.  No call allocates device memory except moe_pool_create.
 *   - Device work is enqueued asynchronously on the given stream; results are
 *     valid once the stream reaches that point.  Calls that also take host
 *     data (moe_pool_plan, moe_pool_refill) say so.
 *   - Every call returns a status: MOE_OK or a negative MOE_ERR_*.  No call
 *     aborts or throws; kernels report an expert that is selected but not
 *     resident through the pool's device error word (moe_pool_check_error).
 *   - Workspaces: device buffers of the size the *_workspace_bytes call
 *     returns, 256-byte aligned, zero-filled by the caller before their first
 *     use; every call leaves them reusable without another fill.  One
 *     workspace must not be used by two calls in flight at once.
 *   - x is bf16 (uint16 bit patterns) row-major [T][d]; router weights fp32
 *     row-major [E+1][d]; outputs fp32.
 *   - Not thread-safe per pool or per workspace.
 */
#ifndef MOE355_H
#define MOE355_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

enum {
  MOE_OK = 0,
  MOE_ERR_INVALID_ARG = -1,    /* null pointer, bad size, misaligned buffer   */
  MOE_ERR_UNSUPPORTED = -2,    /* shape outside the kernels' envelope         */
  MOE_ERR_NOT_RESIDENT = -3,   /* a selected expert had no slot               */
  MOE_ERR_POOL_TOO_SMALL = -4, /* one step needs more distinct experts than slots */
  MOE_ERR_HIP = -5,            /* HIP runtime error; see moe_last_hip_error   */
  MOE_ERR_OUT_OF_MEMORY = -6   /* a host allocation of the library failed     */
};

/* Flags for moe_expert_ffn / moe_layer_forward. */
enum {
  MOE_PATH_AUTO = 0,       /* choose by token count (see moe_expert_ffn)      */
  MOE_PATH_DECODE = 1,     /* per-(token, rank) GEMV, fused combine (T <= 8)  */
  MOE_PATH_BATCHED = 2,    /* bucketed GEMV, partials + combine               */
  MOE_PATH_PREFILL = 3,    /* bucketed fp16 MFMA grouped GEMM + combine       */
  MOE_PATH_PREFILL_TILED = 4,  /* PREFILL with the tiled GEMMs forced         */
  MOE_PATH_PREFILL_STREAM = 5  /* PREFILL with the weight-streaming GEMMs forced */
};

/* Expert FFN shape.  group must be 64; d and I multiples of 64. */
typedef struct moe_ffn_shape {
  int32_t d;      /* hidden size (input of gate/up, output of down)          */
  int32_t I;      /* intermediate size                                       */
  int32_t group;  /* quantisation group along the input dimension (64)       */
  int32_t bits;   /* code width: 4 or 8 (0 is read as 4); 32 = unquantised  */
                  /* fp32 weights                                           */
} moe_ffn_shape;

/* ---------------------------------------------------------------- errors */
const char* moe_status_string(int status);
/* Text of the last HIP error seen by any call of this thread ("" if none). */
const char* moe_last_hip_error(void);
/* Library version string. */
const char* moe_version(void);

/* ----------------------------------------------------------- blob layout
 * One expert = one fixed-stride blob ("How it works": one fetch is one read).
 * For m in gate [I x d], up [I x d], down [d x I] (out x in):
 *   codes_m [in/32][out][16 B]: q[o][32c+2b] in the low nibble and
 *           q[o][32c+2b+1] in the high nibble of byte b of (c, o)
 *   sb_m    [in/64][out][2] fp16: (scale, bias) of group g of row o
 * in the order gate codes, gate sb, up codes, up sb, down codes, down sb.
 * bytes = 27/16 * d * I; stride = bytes rounded up to 4096, zero padded.
 * 8-bit blobs: the same sections, codes_m [in/16][out][16 B] with one code
 * per byte; inside each 8 inputs the bytes hold inputs (0,1,4,5,2,3,6,7) of
 * the block; bytes = 51/16 * d * I.
 * f32 blobs (bits == 32, unquantised; the pages validate every layer in f32
 * as well as int4 form, correctness section): gate, up, down as row-major
 * fp32 [out][in], one after the other, no scale/bias sections;
 * bytes = 12 * d * I.
 * Offsets are 64-bit (multi-GB pools; MLX affine kernels with 64-bit offsets
 * in the relationship-to-TurboFieldfare section). */
size_t moe_blob_bytes(const moe_ffn_shape* sh);   /* 0 if sh is invalid */
size_t moe_blob_stride(const moe_ffn_shape* sh);  /* 0 if sh is invalid */

/* Pack one expert (host) in the layout of sh->bits.  codes[m]: [out][in]
 * bytes, one code each (0..15 for 4 bits, 0..255 for 8), MLX orientation;
 * scales[m], biases[m]: [out][in/64] fp16 bit patterns; m = 0 gate, 1 up,
 * 2 down.  blob_out: moe_blob_stride bytes, written whole (padding zeroed).
 * 4-bit codes above 15: MOE_ERR_INVALID_ARG. */
int moe_pack_expert(const moe_ffn_shape* sh, const uint8_t* const codes[3],
                    const uint16_t* const scales[3],
                    const uint16_t* const biases[3], void* blob_out);
/* Inverse of moe_pack_expert (host). */
int moe_unpack_expert(const moe_ffn_shape* sh, const void* blob,
                      uint8_t* const codes[3], uint16_t* const scales[3],
                      uint16_t* const biases[3]);
/* f32 experts (sh->bits == 32): w[m] = fp32 [out][in] row-major, m = 0
 * gate, 1 up, 2 down; blob_out: moe_blob_stride bytes, written whole.
 * moe_pack_expert / moe_unpack_expert refuse bits == 32 (and these refuse
 * any other width) with MOE_ERR_INVALID_ARG. */
int moe_pack_expert_f32(const moe_ffn_shape* sh, const float* const w[3],
                        void* blob_out);
int moe_unpack_expert_f32(const moe_ffn_shape* sh, const void* blob,
                          float* const w[3]);
/* The same for 4-bit shapes only (MOE_ERR_INVALID_ARG for sh->bits == 8). */
int moe_pack_expert_int4(const moe_ffn_shape* sh,
                         const uint8_t* const codes[3],
                         const uint16_t* const scales[3],
                         const uint16_t* const biases[3],
                         void* blob_out);
int moe_unpack_expert_int4(const moe_ffn_shape* sh, const void* blob,
                           uint8_t* const codes[3], uint16_t* const scales[3],
                           uint16_t* const biases[3]);

/* ------------------------------------------------------------ slot pool
 * Bounded pool of n_slots blobs in HBM ("How it works": hot experts cached in
 * a bounded pool), a device slot table slot_table[e] (-1 = not resident),
 * device usage counters usage[e] (selections, cumulative) and a device error
 * word.  Host-side LFU + recency state decides refills (moe_pool_plan). */
typedef struct moe_pool moe_pool;

typedef struct moe_pool_stats {
  uint64_t steps, hits, misses, loads, evictions, bytes_loaded;
} moe_pool_stats;

/* LFU + recency policy on its own (host only; a pool embeds one).
 * moe_lfu_plan follows the rules of moe_pool_plan below. */
typedef struct moe_lfu moe_lfu;
int moe_lfu_create(int32_t E, int32_t n_slots, moe_lfu** out);
int moe_lfu_destroy(moe_lfu* lfu);
int moe_lfu_plan(moe_lfu* lfu, const int32_t* selected, int32_t n,
                 int32_t* load_expert, int32_t* load_slot, int32_t* load_victim,
                 int32_t* n_loads);
int moe_lfu_get_stats(const moe_lfu* lfu, moe_pool_stats* st);

/* Allocates slab (n_slots * stride bytes), slot table (all -1), usage (0) and
 * error word (0) on the current device. */
int moe_pool_create(int32_t E, int32_t n_slots, const moe_ffn_shape* sh,
                    moe_pool** out);
int moe_pool_destroy(moe_pool* pool);
void* moe_pool_slab(const moe_pool* pool);              /* device */
size_t moe_pool_stride(const moe_pool* pool);
int32_t* moe_pool_slot_table(const moe_pool* pool);     /* device, [E] */
uint32_t* moe_pool_usage(const moe_pool* pool);         /* device, [E] */
int32_t moe_pool_num_experts(const moe_pool* pool);
int32_t moe_pool_num_slots(const moe_pool* pool);

/* Copy one blob into a slot and make `expert` resident there (evicting any
 * previous holder of the slot).  blob is host memory (pinned for a truly
 * asynchronous copy; it must stay valid until the stream passes the copy)
 * for moe_pool_load, device memory for moe_pool_load_device. */
int moe_pool_load(moe_pool* pool, int32_t expert, int32_t slot,
                  const void* blob, hipStream_t stream);
int moe_pool_load_device(moe_pool* pool, int32_t expert, int32_t slot,
                         const void* blob_dev, hipStream_t stream);

/* LFU + recency plan for one step (host only, no device work).  selected: the
 * step's rank-ordered selections (host, n entries, duplicates allowed).  Each
 * selection adds 1 to the expert's count and stamps it with the step number.
 * Distinct experts are taken in first-appearance order; a resident one is a
 * hit; a missing one goes to the lowest free slot, else replaces the resident
 * expert not needed this step with the smallest (count, last step, id).
 * Writes loads (expert, slot, evicted expert or -1) to the three arrays
 * (capacity n each) and their number to *n_loads, and updates the pool's host
 * residency map.  MOE_ERR_POOL_TOO_SMALL if the distinct experts exceed
 * n_slots (nothing is changed then). */
int moe_pool_plan(moe_pool* pool, const int32_t* selected, int32_t n,
                  int32_t* load_expert, int32_t* load_slot,
                  int32_t* load_victim, int32_t* n_loads);

/* Plan (as above) and carry it out: copy each missing blob from
 * host_blobs + expert * host_stride (pinned host memory holding all E blobs)
 * into its slot and publish the new slot-table entries, all on `stream`. */
int moe_pool_refill(moe_pool* pool, const int32_t* selected, int32_t n,
                    const void* host_blobs, size_t host_stride,
                    hipStream_t stream);

/* Set the whole slot table (host array [E], -1 = absent) and the host map;
 * blobs must already sit in those slots (placement tests, replicas). */
int moe_pool_set_slot_table(moe_pool* pool, const int32_t* table,
                            hipStream_t stream);
int moe_pool_get_stats(const moe_pool* pool, moe_pool_stats* st);
/* Synchronises the stream, reads and clears the device error word:
 * *err = MOE_OK, MOE_ERR_NOT_RESIDENT (a selected expert had no slot) or
 * MOE_ERR_UNSUPPORTED (the prefill path met an activation or intermediate
 * beyond the fp16 range, |v| > 65504). */
int moe_pool_check_error(moe_pool* pool, hipStream_t stream, int32_t* err);
/* Synchronises the stream and copies the device slot table ([E] int32) and
 * usage counters ([E] uint32) to host arrays (either may be NULL). */
int moe_pool_read_state(const moe_pool* pool, int32_t* table, uint32_t* usage,
                        hipStream_t stream);
/* Zero the device usage counters (async). */
int moe_pool_reset_usage(moe_pool* pool, hipStream_t stream);

/* --------------------------------------------------------------- router
 * Router logits, top-k, renormalised weights, shared gate, usage counters.
 * x_dev [T][d] bf16; w_router_dev [E+1][d] fp32 (row E = shared-expert gate);
 * logit_bias_dev [E] fp32 or NULL; outputs topk_idx_dev [T][k] int32 and
 * topk_w_dev [T][k] fp32 in rank order, shared_gate_dev [T] fp32 (may be
 * NULL); usage_dev [E] uint32 or NULL (+1 per selection, atomically).
 * 1 <= k <= E <= 1024, d a multiple of 64 and <= 8192.
 * Each logit is an fp32 sum of the d products (plus the bias) in a fixed
 * tree, so the result is deterministic; moe_router_sum_depth gives the
 * largest number of additions on any path of that tree for (T, d, E) (the
 * tree's split of the d products depends on all three), which bounds the
 * rounding error (gamma_n * sum|x_j W_ej|); -1 for invalid sizes. */
int32_t moe_router_sum_depth(int32_t T, int32_t d, int32_t E);
size_t moe_router_workspace_bytes(int32_t T, int32_t d, int32_t E);
int moe_router_topk(const uint16_t* x_dev, int32_t T, int32_t d,
                    const float* w_router_dev, const float* logit_bias_dev,
                    int32_t E, int32_t k, int32_t* topk_idx_dev,
                    float* topk_w_dev, float* shared_gate_dev,
                    uint32_t* usage_dev, void* workspace_dev,
                    size_t workspace_bytes, hipStream_t stream);
/* moe_router_topk that also copies out the logits its selection reads:
 * logits_dev [T][E+1] fp32 (device; NULL = not wanted), row E the shared-gate
 * logit, before the bias (the selection compares fp32(logit + bias)).  Same
 * kernels, same bits; the export is one extra store per logit.  Lets a
 * caller check each logit against the rounding bound of
 * moe_router_sum_depth and the selection against its own logits. */
int moe_router_topk_logits(const uint16_t* x_dev, int32_t T, int32_t d,
                           const float* w_router_dev,
                           const float* logit_bias_dev, int32_t E, int32_t k,
                           int32_t* topk_idx_dev, float* topk_w_dev,
                           float* shared_gate_dev, uint32_t* usage_dev,
                           float* logits_dev, void* workspace_dev,
                           size_t workspace_bytes, hipStream_t stream);

/* ------------------------------------------------------------ bucketing
 * Stable counting sort of the T*k (token, rank) pairs by expert:
 * counts_dev[E], offsets_dev[E+1] (exclusive prefix, offsets[E] = T*k),
 * pair_ids_dev[T*k] (pair i = t*k + r, ascending within each bucket).
 * Indices outside [0, E) make the call fail on the host side only if it can
 * see them; on the device they are counted into no bucket. */
size_t moe_bucket_workspace_bytes(int32_t T, int32_t k, int32_t E);
int moe_bucket_tokens(const int32_t* topk_idx_dev, int32_t T, int32_t k,
                      int32_t E, int32_t* counts_dev, int32_t* offsets_dev,
                      int32_t* pair_ids_dev, void* workspace_dev,
                      size_t workspace_bytes, hipStream_t stream);

/* ----------------------------------------------------------- expert FFN
 * Apply the selected experts (read from `pool` through its slot table; sh
 * must match the pool's shape, code width included) and the shared expert
 * (shared_blob_dev, shape shared_sh with the same d; its code width may
 * differ from the routed experts').
 *   MOE_PATH_DECODE : out_dev = y [T][d], combine fused (needs topk_w and
 *                     shared_gate).  offsets/pair_ids ignored.  T <= 8.
 *   MOE_PATH_BATCHED/PREFILL : needs offsets_dev/pair_ids_dev from
 *                     moe_bucket_tokens; writes the unweighted expert outputs
 *                     partial_dev [T*k][d] (pair order) and shared_out_dev
 *                     [T][d]; combine with moe_combine (out_dev unused).
 *   MOE_PATH_PREFILL: as BATCHED, on the matrix cores: weights dequantised
 *                     to fp16 (one rounding of s*q + b), activations and the
 *                     SwiGLU intermediate in fp16 (|v| <= 65504, else the
 *                     pool error word reports MOE_ERR_UNSUPPORTED), fp32
 *                     accumulate.  Two sets of kernels, same arithmetic in
 *                     the same order (so the same bits): tiled (buckets in
 *                     chunks of up to 128 tokens, activations and weights
 *                     staged through LDS step by step) for many tokens per
 *                     expert, and weight-streaming (chunks of up to 8
 *                     tokens whose activations stay in LDS while the weights
 *                     stream from HBM) for a few; PREFILL picks streaming
 *                     when T*k <= 4*E and d <= 4096, and
 *                     MOE_PATH_PREFILL_TILED / _STREAM force one (STREAM
 *                     needs d <= 4096, else MOE_ERR_UNSUPPORTED).
 *   MOE_PATH_AUTO   : DECODE for T <= 8 (and T*(k+1) <= 2048), else PREFILL,
 *                     or BATCHED if d is not a multiple of 128 or the
 *                     experts are f32 (the caller must then supply every
 *                     buffer).  PREFILL's fp16 range applies to AUTO calls
 *                     above 8 tokens.
 * f32 experts (bits == 32): DECODE and BATCHED only (PREFILL:
 * MOE_ERR_UNSUPPORTED); products and sums in fp32.
 * A selected expert with slot_table[e] < 0 sets the pool's error word and
 * contributes zero. */
size_t moe_ffn_workspace_bytes(const moe_ffn_shape* sh,
                               const moe_ffn_shape* shared_sh, int32_t T,
                               int32_t k, int32_t E, int32_t path);
int moe_expert_ffn(const moe_pool* pool, const moe_ffn_shape* sh,
                   const void* shared_blob_dev, const moe_ffn_shape* shared_sh,
                   const uint16_t* x_dev, int32_t T, int32_t k,
                   const int32_t* topk_idx_dev, const float* topk_w_dev,
                   const float* shared_gate_dev, const int32_t* offsets_dev,
                   const int32_t* pair_ids_dev, float* out_dev,
                   float* partial_dev, float* shared_out_dev, int32_t path,
                   void* workspace_dev, size_t workspace_bytes,
                   hipStream_t stream);
/* moe_expert_ffn for 4-bit routed and shared experts only
 * (MOE_ERR_INVALID_ARG if either shape has bits == 8). */
int moe_expert_ffn_int4(const moe_pool* pool, const moe_ffn_shape* sh,
                        const void* shared_blob_dev,
                        const moe_ffn_shape* shared_sh,
                        const uint16_t* x_dev, int32_t T, int32_t k,
                        const int32_t* topk_idx_dev, const float* topk_w_dev,
                        const float* shared_gate_dev,
                        const int32_t* offsets_dev, const int32_t* pair_ids_dev,
                        float* out_dev, float* partial_dev,
                        float* shared_out_dev, int32_t path,
                        void* workspace_dev, size_t workspace_bytes,
                        hipStream_t stream);

/* -------------------------------------------------------------- combine
 * y[t] = sum_{r<k} w[t,r] * partial[t*k+r] + s_t * shared_out[t], in that
 * order, fp32.  shared_out_dev / shared_gate_dev may both be NULL. */
int moe_combine(const float* partial_dev, const float* shared_out_dev,
                const float* topk_w_dev, const float* shared_gate_dev,
                int32_t T, int32_t k, int32_t d, float* y_dev,
                hipStream_t stream);

/* ---------------------------------------------------------- whole layer
 * Router -> (bucketing) -> experts -> combine, one call, all on `stream`. */
typedef struct moe_layer_desc {
  moe_ffn_shape sh;            /* routed expert shape                       */
  moe_ffn_shape shared_sh;     /* shared expert shape (same d)              */
  int32_t E, k;
  const float* w_router_dev;   /* [E+1][d]                                  */
  const float* logit_bias_dev; /* [E] or NULL                               */
  const moe_pool* pool;        /* routed experts                            */
  const void* shared_blob_dev; /* one blob of shape shared_sh               */
  uint32_t* usage_dev;         /* [E] or NULL                               */
} moe_layer_desc;

size_t moe_layer_workspace_bytes(const moe_layer_desc* L, int32_t T,
                                 int32_t path);
/* Outputs: y_dev [T][d]; topk_idx_dev [T][k], topk_w_dev [T][k],
 * shared_gate_dev [T] (all required: later stages read them). */
int moe_layer_forward(const moe_layer_desc* L, const uint16_t* x_dev,
                      int32_t T, float* y_dev, int32_t* topk_idx_dev,
                      float* topk_w_dev, float* shared_gate_dev, int32_t path,
                      void* workspace_dev, size_t workspace_bytes,
                      hipStream_t stream);

/* ------------------------------------------- whole layer, no allocation
 * For callers that cannot allocate device memory: code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc.  The same
 * call as moe_layer_forward (same kernels, same bits), with the workspace
 * taken from a scratch array of MOE_NOALLOC_SCRATCH_BYTES that the library
 * holds in device memory, one per GPU, for the life of the process (set up,
 * and cleared once, by the first call on that GPU: a fill kernel on `stream`
 * ahead of the call's own work).  Nothing is allocated, by this call or by
 * the library routines it uses.  Calls whose workspace
 * (moe_layer_workspace_bytes(L, T, path)) exceeds the scratch return
 * MOE_ERR_UNSUPPORTED and do nothing: 32 MiB covers the decode path
 * (T <= 8) at every supported shape and the 80B-shaped batched layer well
 * past 64 tokens, not a 4096-token prefill.  Every call on one GPU shares
 * that GPU's scratch, which keeps the last call's contents: calls that
 * overlap on one GPU (two streams, two threads) race and must be ordered
 * by the caller. */
#define MOE_NOALLOC_SCRATCH_BYTES (32u << 20)
int moe_layer_forward_noalloc(const moe_layer_desc* L, const uint16_t* x_dev,
                              int32_t T, float* y_dev, int32_t* topk_idx_dev,
                              float* topk_w_dev, float* shared_gate_dev,
                              int32_t path, hipStream_t stream);

/* ------------------------------------------------- streamed decode step
 * One decode step (T <= 8, T*(k+1) <= 2048, 4- or 8-bit experts) on a pool
 * that holds only some experts, with the misses copied in while the resident
 * experts compute (the pages keep routed experts in a bounded pool refilled
 * from storage by LFU + recency, "How it works" and the cache discussion;
 * here the storage tier is pinned host memory).  In order:
 *   1. router and top-k on `stream`; the selections are copied to pinned
 *      host memory owned by the pool;
 *   2. phase 1 on `stream`: gate/up and down of the resident selections and
 *      the shared expert (missing selections are deferred, not errors);
 *   3. the calling thread waits for the selections only, plans the refill
 *      (moe_pool_plan: same policy, stats and residency map), and queues the
 *      host_blobs + expert * host_stride -> slot copies on `copy_stream`;
 *   4. `stream` waits for those copies, publishes the slot-table edits and
 *      runs phase 2: the deferred selections, then the rank-order combine.
 * Outputs as moe_layer_forward (decode path) and bit-identical to it on an
 * all-resident pool: every expert's outputs are computed by the same code
 * and combined in the same order.  host_blobs: pinned host memory holding all
 * E blobs (host_stride >= the pool stride), valid until the copies pass.
 * workspace: moe_layer_workspace_bytes(L, T, MOE_PATH_DECODE) bytes.
 * *n_loads (may be NULL): blobs copied this step.  copy_stream may equal
 * stream (no overlap then).  The pool's selection staging is per pool:
 * streamed steps on one pool must not overlap.  Errors as moe_pool_plan
 * (MOE_ERR_POOL_TOO_SMALL: nothing copied, y not written) and the decode
 * path; a selection still missing in phase 2 sets the pool error word. */
int moe_layer_forward_streamed(const moe_layer_desc* L,
                               const void* host_blobs, size_t host_stride,
                               const uint16_t* x_dev, int32_t T, float* y_dev,
                               int32_t* topk_idx_dev, float* topk_w_dev,
                               float* shared_gate_dev, void* workspace_dev,
                               size_t workspace_bytes, hipStream_t stream,
                               hipStream_t copy_stream, int32_t* n_loads);

/* The same decode step with the refill decided and copied by the GPU, so
 * that no host wait sits between the router and the experts ("How it works":
 * experts outside the bounded pool fetched on demand; the pages' streaming
 * of experts from storage).  On `stream`, in order: router and top-k; the
 * pool's LFU + recency plan (the rules and decisions of moe_pool_plan, on a
 * device copy of the pool's policy state, by one wave); the missing blobs
 * read over PCIe from host_blobs by a copy kernel that takes its work list
 * from the plan; the experts and the combine.  The calling thread does not
 * wait, and the outputs are bit-identical to the all-resident decode.
 *   host_blobs: pinned host memory mapped for the device (hipHostMalloc or
 *     torch's pin_memory), 16-byte aligned, blob e at host_blobs + e *
 *     host_stride (host_stride >= the pool's stride, a multiple of 16);
 *     MOE_ERR_INVALID_ARG if it is not mapped.
 *   n_loads_dev: device int32 (may be NULL): blobs copied by this step.
 * T <= 8, 4- or 8-bit experts.  MOE_ERR_UNSUPPORTED when T * k exceeds the
 * pool's slots (a step could then need more experts than it holds; use
 * moe_layer_forward_streamed, which reports MOE_ERR_POOL_TOO_SMALL) or when
 * E or n_slots exceeds 1024.  The pool's policy state then lives on the
 * device as well: the first call allocates its device copy (and copies the
 * host state there), later host-side pool calls (moe_pool_plan, refill,
 * load, set_slot_table, get_stats) first synchronise the device and bring
 * the host copy up to date.  Offload steps on one pool must be issued in
 * order on one stream. */
int moe_layer_forward_offload(const moe_layer_desc* L,
                              const void* host_blobs, size_t host_stride,
                              const uint16_t* x_dev, int32_t T, float* y_dev,
                              int32_t* topk_idx_dev, float* topk_w_dev,
                              float* shared_gate_dev, void* workspace_dev,
                              size_t workspace_bytes, int32_t* n_loads_dev,
                              hipStream_t stream);

/* ------------------------------------------------------------ layer chain
 * L layers applied one after the other to the same T tokens (the pages'
 * models stack dozens of MoE layers per token).  Each is a pre-norm residual
 * block read without the attention half and without a learned norm weight:
 *   u_l = bf16(x_l / sqrt(mean(x_l^2) + eps)),
 *   x_{l+1} = bf16(x_l + moe_layer_forward(layers[l], u_l)),
 * the residual add in fp32, the sum of squares in fp32 in a fixed order.
 * All layers share d and k.  x_dev [T][d] bf16 in, x_out_dev [T][d] bf16 out
 * (x_L).  Optional (NULL = not wanted): trace_x_dev [L+1][T][d] (x_0..x_L),
 * trace_u_dev [L][T][d] (u_0..u_{L-1}), topk_idx_dev [L][T][k].  path as in
 * moe_layer_forward, for every layer.  Everything goes on `stream`.
 * When every layer takes the decode path with 4- or 8-bit experts and
 * trace_u_dev is NULL, the layers hand the residual stream on themselves
 * (each down GEMV adds its output to x_l and sums the squares of x_{l+1} in
 * groups of 8, the next router normalises): one extra launch for the whole
 * chain.  Otherwise one launch per layer for the residual/norm step.  Both
 * give the same bits (same fp32 operations in the same order). */
size_t moe_chain_workspace_bytes(const moe_layer_desc* layers, int32_t L,
                                 int32_t T, int32_t path);
int moe_chain_forward(const moe_layer_desc* layers, int32_t L, float eps,
                      const uint16_t* x_dev, int32_t T, uint16_t* x_out_dev,
                      uint16_t* trace_x_dev, uint16_t* trace_u_dev,
                      int32_t* topk_idx_dev, int32_t path,
                      void* workspace_dev, size_t workspace_bytes,
                      hipStream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* MOE355_H */
