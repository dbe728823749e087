// Internal declarations shared by the HIP translation units of libsage.
// Nothing here is part of the public C ABI (see include/sage.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace sage {

// Contract constants.  They fix the rounding of the method, so changing one
// changes results and bumps kContractVersion.
constexpr int kBQ = 128;      // tokens per Q-smoothing block, per mean chunk, per query tile
constexpr int kBK = 128;      // keys per online-softmax block (also the level-1 P~V block)
constexpr int kKGroup = 16;   // keys per K scale group (two groups per 32-key tile)
constexpr int kContractVersion = 1;

enum InDtype { kF16 = 0, kBF16 = 1 };
enum OutDtype { kOutF16 = 0, kOutBF16 = 1, kOutF32 = 2 };

struct Dims {
  int B, H, N, D;
  int NP;    // N rounded up to a multiple of 128
  int NQB;   // NP / 128
  int QB;    // bits per Q/K code: 4 (INT4, packed pairs) or 8 (INT8)
  __host__ __device__ int BH() const { return B * H; }
};

// Device buffers written by the prepass and read by the attention kernel.
struct Bufs {
  uint8_t* q_codes;   // [B,H,NP,D*QB/8]: packed INT4 pairs or INT8 codes
  uint8_t* k_codes;   // [B,H,NP,D*QB/8]
  float* q_scale;     // [B,H,NP]
  float* k_scale;     // [B,H,NP/16]
  float* q_mean;      // [B,H,NQB,D]
  float* k_mean;      // [B,H,D]
  uint8_t* v_codes;   // [B,H,NQB,D,128] e4m3fn, keys permuted inside each 128-key block
  float* v_scale;     // [B,H,D]
  float* delta_s;     // [B,H,NQB,NP]   compensation term times ds_scale
  float* k_part;      // [B,H,NQB,D]    per-chunk K channel sums; then bf16 q_mean pieces 1-2
  float* v_part;      // [B,H,NQB,D]    per-chunk V channel absmax; then bf16 q_mean piece 3
};

hipError_t launch_prepass(const void* q, const void* k, const void* v, int in_dtype, const Dims& d,
                          const Bufs& b, float ds_scale, hipStream_t s);
hipError_t launch_attn(const Bufs& b, const Dims& d, int causal, float ks, void* o, int out_dtype,
                       hipStream_t s);
hipError_t launch_qk_debug(const Bufs& b, const Dims& d, int bh, int q0, int k0, int nq, int nk,
                           int32_t* out, hipStream_t s);
hipError_t launch_fp8_encode(const float* in, uint8_t* out, size_t n, hipStream_t s);

}  // namespace sage
