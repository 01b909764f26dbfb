// Device-side helpers for the gfx950 kernels (wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

// acc + a.lo*b.lo + a.hi*b.hi on two packed bf16 pairs, fp32 accumulate
// (v_dot2c_f32_bf16).  Products of two bf16 values are exact in fp32.
__device__ __forceinline__ float dot2_bf16(uint32_t a, uint32_t b, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, a),
                                         __builtin_bit_cast(bf16x2_t, b), acc, false);
}

// fp16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(bits16 & 0xFFFFu));
}

__device__ __forceinline__ float bf16_lo(uint32_t p) { return __uint_as_float(p << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t p) { return __uint_as_float(p & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
  return v;
}

// Order-preserving map of an fp32 value to uint32 (-0 folded onto +0).
__device__ __forceinline__ uint32_t f32_order(float f) {
  if (f == 0.0f) f = 0.0f;
  uint32_t u = __float_as_uint(f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float f32_unorder(uint32_t o) {
  uint32_t u = (o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o;
  return __uint_as_float(u);
}

// Wave-wide max of a uint32 via DPP (pair, quad, row rotations, row
// broadcasts); lane 63 ends with the maximum, which is returned to all lanes.
__device__ __forceinline__ uint32_t dpp_max_step(uint32_t v, uint32_t t) { return v > t ? v : t; }
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
  v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0xB1, 0xF, 0xF, false));
  v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x4E, 0xF, 0xF, false));
  v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x124, 0xF, 0xF, false));
  v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x128, 0xF, 0xF, false));
  v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x142, 0xA, 0xF, false));
  v = dpp_max_step(v, (uint32_t)__builtin_amdgcn_update_dpp((int)v, (int)v, 0x143, 0xC, 0xF, false));
  return (uint32_t)__builtin_amdgcn_readlane((int)v, 63);
}

// Sum over each aligned group of 8 consecutive lanes (every lane of the
// group gets the sum): pair swap, quad swap, half-row mirror, all DPP.
__device__ __forceinline__ float sum8_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0xB1, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x4E, 0xF, 0xF, false));
  v += __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x141, 0xF, 0xF, false));
  return v;
}

__device__ __forceinline__ int wave_min_i32(int v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) {
    const int o = __shfl_xor(v, s, 64);
    v = o < v ? o : v;
  }
  return v;
}

__device__ __forceinline__ float sigmoidf_(float z) { return 1.0f / (1.0f + expf(-z)); }

// Sum of squares of 8 consecutive values in the order sum8_dpp adds them
// across 8 lanes: ((e0+e1)+(e2+e3))+((e4+e5)+(e6+e7)), e = v*v rounded.
__device__ __forceinline__ float sq_tree8(const float* v) {
  float e[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) e[i] = __fmul_rn(v[i], v[i]);
  return ((e[0] + e[1]) + (e[2] + e[3])) + ((e[4] + e[5]) + (e[6] + e[7]));
}

// Buffer resource over [base, base + bytes): loads past the end return
// zeros (no fault).  LDS DMA (buffer_load ... lds) takes its LDS address
// block-uniform and opaque to the compiler's alias tracking.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ lds_void* lds_opaque(const void* p) {
  const uint32_t a = (uint32_t)(uintptr_t)(const lds_void*)p;
  return (lds_void*)(uintptr_t)__builtin_amdgcn_readfirstlane(a);
}

}  // namespace moe
