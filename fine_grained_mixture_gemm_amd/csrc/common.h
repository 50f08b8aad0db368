// Shared device helpers for the DeepSeekMoE layer kernels (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "../../include/moe.h"

namespace moe {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr float kE4M3Max = 448.0f;

// ------------------------------------------------------------------ number formats
__device__ __forceinline__ float bf16_to_f32(uint16_t h) { return __uint_as_float(uint32_t(h) << 16); }

// Round to nearest even (the gfx950 conversion instruction).
__device__ __forceinline__ uint16_t f32_to_bf16(float x) {
  __bf16 b = (__bf16)x;
  return __builtin_bit_cast(uint16_t, b);
}

// Two fp32 -> two E4M3 (FN) bytes in the low half of the result, nearest-even. Inputs are clamped
// to +-448 first, which turns the conversion into the saturating one for every finite input.
__device__ __forceinline__ uint32_t f32x2_to_e4m3x2(float a, float b) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  return uint32_t(__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false)) & 0xFFFFu;
}

__device__ __forceinline__ uint32_t f32x4_to_e4m3x4(float a, float b, float c, float d) {
  a = fminf(fmaxf(a, -kE4M3Max), kE4M3Max);
  b = fminf(fmaxf(b, -kE4M3Max), kE4M3Max);
  c = fminf(fmaxf(c, -kE4M3Max), kE4M3Max);
  d = fminf(fmaxf(d, -kE4M3Max), kE4M3Max);
  int v = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  v = __builtin_amdgcn_cvt_pk_fp8_f32(c, d, v, true);
  return uint32_t(v);
}

// Scale of a tile whose largest magnitude is amax: s = amax / 448 and its reciprocal 448 / amax,
// both correctly rounded fp32 divisions; an all-zero tile gets s = inv = 1.
__device__ __forceinline__ void e4m3_scales(float amax, float& s, float& inv) {
  if (amax == 0.0f) {
    s = 1.0f;
    inv = 1.0f;
  } else {
    s = __fdiv_rn(amax, kE4M3Max);
    inv = __fdiv_rn(kE4M3Max, amax);
  }
}

// SiLU(g) = g * sigmoid(g) with the hardware reciprocal (1 ulp) in place of an IEEE division; the result
// is requantized (E4M3 or bf16) or compared at 1e-5 (fp32), far above that difference. Large negative g:
// the reciprocal of +inf is 0, as the division would give.
__device__ __forceinline__ float silu(float g) { return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// ------------------------------------------------------------------ wave reductions
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    uint64_t w = __shfl_xor(v, o, 64);
    v = w > v ? w : v;
  }
  return v;
}

// Order-preserving map of an fp32 key to uint32 (larger key -> larger integer).
__device__ __forceinline__ uint32_t f32_order(float x) {
  uint32_t b = __float_as_uint(x);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ uint64_t f64_order(double x) {
  uint64_t b = (uint64_t)__double_as_longlong(x);
  return (b & 0x8000000000000000ull) ? ~b : (b | 0x8000000000000000ull);
}

// ------------------------------------------------------------------ LDS-DMA copies and waits
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Global -> LDS copy of 16 (or 4) bytes per lane; the wave writes 64 consecutive pieces at `lds_base`.
__device__ __forceinline__ void dma16(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (lds_ptr_t)lds_base, 4, 0, 0);
}

// Wait until this wave has no vector-memory operation in flight (its LDS-DMA copies have landed).
__device__ __forceinline__ void wait_vm0() { __builtin_amdgcn_s_waitcnt(0 | (7 << 4) | (15 << 8)); }

// Workgroup barrier for LDS traffic: waits for this wave's LDS operations (lgkmcnt 0); the empty asm
// statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void barrier_lds() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}


__host__ __device__ __forceinline__ int cdiv(int a, int b) { return (a + b - 1) / b; }
__host__ __device__ __forceinline__ size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

}  // namespace moe
