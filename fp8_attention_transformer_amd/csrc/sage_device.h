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

// One output element in the requested dtype (bf16 and fp16 with RNE).
// The 16-bit output pattern of val (kOutBF16: round to nearest even; kOutF16).
__device__ __forceinline__ uint32_t out_bits16(float val, int out_dtype) {
  if (out_dtype == kOutBF16) {
    const uint32_t u = __float_as_uint(val);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
  }
  const _Float16 hv = (_Float16)val;
  uint16_t bits;
  __builtin_memcpy(&bits, &hv, 2);
  return bits;
}

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

// x / d rounded to nearest in fp32, from r = RN(1/d): the product q = RN(x*r)
// corrected once with the exact remainder fma(-q, d, x) (Markstein's
// correction step) is the correctly rounded quotient whenever d is normal,
// not above 2^126 and its significand is not all ones; d = 0 (r = 0) gives 0.
__device__ __forceinline__ float div_rn(float x, float d, float r) {
  const float q = x * r;
  return __builtin_fmaf(__builtin_fmaf(-q, d, x), r, q);
}
// The same with the sign of x kept on a zero quotient (-0 / d = -0; the two
// FMAs above add +0 and -0 to +0), for d != 0.
__device__ __forceinline__ float div_rn_signed(float x, float d, float r) {
  return __builtin_copysignf(div_rn(x, d, r), x);
}
// divisors outside the case above (a true division is used for them)
__device__ __forceinline__ bool div_rn_hard(float d) {
  const uint32_t b = __float_as_uint(d) & 0x7FFFFFFFu;
  return b != 0u && (b < 0x00800000u || b >= 0x7E800000u || (b & 0x7FFFFFu) == 0x7FFFFFu);
}

// LDS destination of the direct memory-to-LDS copies
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Buffer resource over one head's array: raw addressing, `bytes` records (the
// hardware returns zeros beyond them), default gfx9 data format word.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// s_waitcnt with only the vector-memory counter limited to n (gfx9 encoding:
// vmcnt[3:0] in bits 3:0, vmcnt[5:4] in bits 15:14, expcnt and lgkmcnt at
// max).  On gfx9 the counter retires loads and stores in issue order, so
// vmcnt(n) means: all but the last n vector-memory instructions are done.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

}  // namespace sage
