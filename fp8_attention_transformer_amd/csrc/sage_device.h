// Device-side helpers shared by the prepass and attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "sage_internal.h"

namespace sage {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));

// 16-bit input element -> fp32 (exact).
template <int IN>
__device__ __forceinline__ float in_to_f32(uint16_t bits) {
  if constexpr (IN == 1) {  // bf16
    return __uint_as_float((uint32_t)bits << 16);
  } else {                  // fp16
    _Float16 h;
    __builtin_memcpy(&h, &bits, 2);
    return (float)h;
  }
}

// fp32 -> OCP e4m3fn byte with round-to-nearest-even (hardware conversion).
// The matrix cores of gfx950 read this format for FP8 operands.
__device__ __forceinline__ uint32_t fp8x2(float a, float b) {
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false) & 0xFFFFu;
}
// `dead` is any register value the caller no longer needs: the conversions
// write bytes 0-1 and then 2-3 of it, so its prior contents never matter and
// it needs no zero initialisation.
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d, int dead = 0) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, dead, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// FP6 e2m3 bit pattern of an integer c in [-7, 7]: magnitudes 0..7 encode as
// 0, 8, 16, 20, 24, 26, 28, 30 (1.m x 2^(e-1) with e = 1..3), sign in bit 5.
__device__ __forceinline__ uint32_t fp6_of_int(int c) {
  const uint32_t a = (uint32_t)(c < 0 ? -c : c);
  const uint32_t mag = (uint32_t)(0x1E1C1A1814100800ull >> (8 * a)) & 0x3Fu;
  return c < 0 ? (mag | 32u) : mag;
}
// NF (a multiple of 16) FP6 codes -> 3*NF/16 words, field e at bit 6e.
template <int NF>
__device__ __forceinline__ void pack_fp6(const int* c, uint32_t* w) {
  static_assert(NF % 16 == 0, "whole words");
#pragma unroll
  for (int i = 0; i < 3 * NF / 16; i++) w[i] = 0;
#pragma unroll
  for (int e = 0; e < NF; e++) {
    const uint32_t f = fp6_of_int(c[e]);
    const int bit = 6 * e;
    w[bit / 32] |= f << (bit % 32);
    if (bit % 32 > 26) w[bit / 32 + 1] |= f >> (32 - bit % 32);
  }
}

// One output element in the requested dtype (bf16 and fp16 with RNE).
__device__ __forceinline__ void store_out(void* o, size_t idx, float val, int out_dtype) {
  if (out_dtype == kOutF32) {
    ((float*)o)[idx] = val;
  } else if (out_dtype == kOutBF16) {
    const uint32_t u = __float_as_uint(val);
    ((uint16_t*)o)[idx] = (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
  } else {
    const _Float16 hv = (_Float16)val;
    uint16_t bits;
    __builtin_memcpy(&bits, &hv, 2);
    ((uint16_t*)o)[idx] = bits;
  }
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}
// Max across groups of `width` consecutive lanes (width a power of two <= 64).
template <int WIDTH>
__device__ __forceinline__ float group_max(float v) {
#pragma unroll
  for (int o = WIDTH / 2; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
  return v;
}

}  // namespace sage
