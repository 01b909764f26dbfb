// Top-k selection of router logits for one token, one wave (wave64).
#pragma once

#include "device.h"

namespace moe {

inline int nk_for(int E) { return E <= 64 ? 1 : E <= 128 ? 2 : E <= 256 ? 4 : E <= 512 ? 8 : 16; }

// Words of LDS scratch one wave needs for topk_select with E experts (8-byte
// aligned: 64-bit keys of up to E candidates plus 16 spare and pad entries).
__host__ __device__ inline int topk_scratch_words(int E) { return (64 + 2 * E + 3) & ~3; }

// One wave selects the top k of one token's E logits (E <= 64*NK) into
// sel_l / sel_e (rank order: logit descending, index ascending; k entries).
// scr: this wave's LDS scratch, topk_scratch_words(E) words.
//
// Keys are order-preserving uint32 images of the logits (+ bias); lane l
// holds experts l, l+64, ....  No sequential selection rounds:
//  1. T = high 16 bits of the k-th largest lane maximum, found by a ballot
//     search two bits per step (k <= 64); at least k keys are >= T, so every
//     top-k key is >= T.  (k > 64: T = 1, i.e. every key.)
//  2. keys >= T are packed into LDS as 64-bit (key, ~index) values (per
//     slice of 64 keys: ballot, mbcnt): typically a little over k candidates.
//  3. each candidate's rank = number of candidates whose 64-bit value is
//     larger (larger key, or equal key and lower index), from LDS broadcasts;
//     ranks below k are written out.  Integer work throughout: bit-exact.
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
  // keys: the order-preserving map of f32_order without its branch (adding
  // +0 folds -0 onto +0; then x ^ (sign mask | 0x80000000))
  uint32_t kv[NK];
  uint32_t lm = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const uint32_t u = __float_as_uint(lv[j] + 0.0f);
    const uint32_t key = u ^ ((uint32_t)((int32_t)u >> 31) | 0x80000000u);
    kv[j] = (lane + 64 * j < E) ? key : 0u;   // never 0 for a real value
    lm = kv[j] > lm ? kv[j] : lm;
  }
  // 1. threshold on the high half-word of the lane maxima, two bits per
  //    step (three independent ballots)
  uint32_t T = 1;
  if (k <= 64) {
    const uint32_t hi = lm >> 16;
    uint32_t x = 0;
#pragma unroll
    for (int bit = 14; bit >= 0; bit -= 2) {
      const uint32_t c1 = x | (1u << bit), c2 = x | (2u << bit), c3 = x | (3u << bit);
      const int n1 = __popcll(__ballot(hi >= c1)), n2 = __popcll(__ballot(hi >= c2));
      const int n3 = __popcll(__ballot(hi >= c3));
      x = n3 >= k ? c3 : n2 >= k ? c2 : n1 >= k ? c1 : x;
    }
    T = x << 16;
    if (T == 0) T = 1;
  }
  // 2. candidates (keys >= T) packed into LDS slice by slice as 64-bit keys
  //    (key << 32 | ~index: a larger 64-bit key ranks earlier); a
  //    candidate's place is the slice's base plus the candidates in lower
  //    lanes (mbcnt).  Stores are unconditional (others go to spare words),
  //    and eight zero keys (ranking last) pad the list.
  uint64_t* key64 = reinterpret_cast<uint64_t*>(scr);   // [8 spare][C candidates][8 pad]
  int C = 0;
#pragma unroll
  for (int j = 0; j < NK; ++j) {
    const bool cand = kv[j] >= T;
    const uint64_t m = __ballot(cand);
    const int pos = C + (int)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                                       __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
    C += (int)__popcll(m);
    key64[cand ? 8 + pos : (lane & 7)] = ((uint64_t)kv[j] << 32) | (uint32_t)~(uint32_t)(lane + 64 * j);
  }
  if (lane < 8) key64[8 + C + lane] = 0;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  // 3. ranks: each candidate counts the keys above its own, eight LDS
  //    broadcasts at a time
  for (int c0 = 0; c0 < C; c0 += 64) {
    const int c = c0 + lane;
    const uint64_t key = c < C ? key64[8 + c] : 0;
    int rank = 0;
    for (int q = 0; q < C; q += 8) {
      uint64_t k2[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) k2[u] = key64[8 + q + u];
#pragma unroll
      for (int u = 0; u < 8; ++u) rank += k2[u] > key;
    }
    if (c < C && rank < k) {
      sel_e[rank] = (int32_t)~(uint32_t)key;
      sel_l[rank] = f32_unorder((uint32_t)(key >> 32));
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
