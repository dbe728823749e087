// Device-side helpers shared by the prepass and attention kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
__device__ __forceinline__ uint32_t fp8x4(float a, float b, float c, float d) {
  int lo = __builtin_amdgcn_cvt_pk_fp8_f32(a, b, 0, false);
  return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(c, d, lo, true);
}

// Symmetric INT4 code: clamp(round-half-even(x / delta), -7, 7); delta == 0 -> 0.
__device__ __forceinline__ int int4_code(float x, float delta) {
  if (delta == 0.0f) return 0;
  float r = rintf(x / delta);
  r = fminf(fmaxf(r, -7.0f), 7.0f);
  return (int)r;
}

// Packed pair format: one byte holds channels 2b (even) and 2b+1 (odd) as the
// signed value 16*c_odd + c_even + 8.  Decoding: c_even = (v & 15) - 8,
// c_odd = v >> 4 (arithmetic).  The byte read as an int8 matrix-core operand
// is 16*c_odd + (c_even + 8); masked with 0xF0 it is 16*c_odd.
__device__ __forceinline__ uint32_t pack_pair(int c_even, int c_odd) {
  return (uint32_t)(16 * c_odd + c_even + 8) & 0xFFu;
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
