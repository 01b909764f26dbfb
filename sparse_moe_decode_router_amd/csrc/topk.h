// Top-k selection of router logits for one token, one wave (wave64).
#pragma once

#include "device.h"

namespace moe {

inline int nk_for(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

// Words of LDS scratch one wave needs for topk_select with E experts.
__host__ __device__ inline int topk_scratch_words(int E) { return (64 + 2 * E + 3) & ~3; }

// One wave selects the top k of one token's E logits (E <= 64*NK) into
// sel_l / sel_e (rank order: logit descending, index ascending; k entries).
// scr: this wave's LDS scratch, topk_scratch_words(E) words.
//
// Keys are order-preserving uint32 images of the logits (+ bias); lane l
// holds experts l, l+64, ....  No sequential selection rounds:
//  1. T = high 16 bits of the k-th largest lane maximum, found by a 16-step
//     ballot binary search (k <= 64); at least k keys are >= T, so every
//     top-k key is >= T.  (k > 64: T = 1, i.e. every key.)
//  2. keys >= T are compacted into LDS (ballot prefix of per-lane counts):
//     typically a little over k candidates, reloaded one per lane.
//  3. each candidate's rank = number of candidates ahead of it (larger key,
//     or equal key and lower index), from readlane broadcasts; ranks below k
//     are written out.  Integer work throughout: bit-exact.
template <int NK>
__device__ __forceinline__ void topk_select(const float* lrow, const float* __restrict__ bias, int E, int k,
                                            float* sel_l, int32_t* sel_e, uint32_t* scr) {
  const int lane = threadIdx.x & 63;
  float lv[NK];
#pragma unroll
  for (int j = 0; j < NK; ++j) {           // all loads issued before any use
    const int e = lane + 64 * j;
    lv[j] = lrow[e < E ? e : 0];
  }
  if (bias) {
#pragma unroll
    for (int j = 0; j < NK; ++j) {
      const int e = lane + 64 * j;
      lv[j] += bias[e < E ? e : 0];
    }
  }
  uint32_t kv[NK];
  uint32_t lm = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    kv[j] = (lane + 64 * j < E) ? f32_order(lv[j]) : 0u;   // never 0 for a real value
    lm = kv[j] > lm ? kv[j] : lm;
  }
  // 1. threshold on the high half-word of the lane maxima
  uint32_t T = 1;
  if (k <= 64) {
    const uint32_t hi = lm >> 16;
    uint32_t x = 0;
#pragma unroll
    for (int bit = 15; bit >= 0; --bit) {
      const uint32_t c = x | (1u << bit);
      if (__popcll(__ballot(hi >= c)) >= k) x = c;
    }
    T = x << 16;
    if (T == 0) T = 1;
  }
  // 2. candidates: per-lane count, exclusive prefix by ballots of count bits
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) cnt += (kv[j] >= T);
  const uint64_t below = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
  int off = 0, C = 0;
#pragma unroll
  for (int b = 0; b < 5; ++b) {
    const uint64_t m = __ballot((cnt >> b) & 1);
    off += __popcll(m & below) << b;
    C += __popcll(m) << b;
  }
  uint32_t* cv = scr + 64;
  uint32_t* ce = scr + 64 + E;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    if (kv[j] >= T) {
      cv[off] = kv[j];
      ce[off] = lane + 64 * j;
      ++off;
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // 3. ranks
  if (C <= 64) {
    const bool mine = lane < C;
    const uint32_t v = mine ? cv[lane] : 0u;
    const uint32_t e = mine ? ce[lane] : 0u;
    // one 64-bit key per candidate, key(a) > key(b) iff a ranks before b:
    // larger logit key, or the same and a lower index
    const uint64_t key = ((uint64_t)v << 32) | (uint32_t)~e;
    const uint32_t klo = (uint32_t)key, khi = (uint32_t)(key >> 32);
    int rank = 0;
    for (int q = 0; q < C; ++q) {
      const uint64_t k2 = ((uint64_t)(uint32_t)__builtin_amdgcn_readlane((int)khi, q) << 32) |
                          (uint32_t)__builtin_amdgcn_readlane((int)klo, q);
      rank += k2 > key;
    }
    if (mine && rank < k) {
      sel_e[rank] = (int32_t)e;
      sel_l[rank] = f32_unorder(v);
    }
  } else {
    for (int c = lane; c < C + ((64 - (C & 63)) & 63); c += 64) {
      const bool mine = c < C;
      const uint32_t v = mine ? cv[c] : 0u;
      const uint32_t e = mine ? ce[c] : 0u;
      int rank = 0;
      for (int q = 0; q < C; ++q) {
        const uint32_t v2 = cv[q], e2 = ce[q];
        rank += (v2 > v) | ((v2 == v) & (e2 < e));
      }
      if (mine && rank < k) {
        sel_e[rank] = (int32_t)e;
        sel_l[rank] = f32_unorder(v);
      }
    }
  }
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Renormalised weights of the k selections (softmax over the chosen logits)
// written in rank order with the indices; usage counters bumped.  One wave.
__device__ __forceinline__ void topk_finish(const float* sel_l, const int32_t* sel_e, int k, int32_t* __restrict__ idx_out,
                            float* __restrict__ w_out, uint32_t* __restrict__ usage) {
  const int lane = threadIdx.x & 63;
  const float lmax = sel_l[0];
  float z = 0.0f;
  for (int r = lane; r < k; r += 64) z += expf(sel_l[r] - lmax);
  z = wave_sum(z);
  for (int r = lane; r < k; r += 64) {
    const int e = sel_e[r];
    idx_out[r] = e;
    w_out[r] = expf(sel_l[r] - lmax) / z;
    if (usage) atomicAdd(&usage[e], 1u);
  }
}

}  // namespace moe
