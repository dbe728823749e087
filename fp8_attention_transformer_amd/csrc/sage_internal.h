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
constexpr int kContractVersion = 2;

enum InDtype { kF16 = 0, kBF16 = 1 };
enum OutDtype { kOutF16 = 0, kOutBF16 = 1, kOutF32 = 2 };

// Q/K code layout for 4-bit codes.  Every integer in [-7, 7] is exact in OCP
// FP6 e2m3 (sign, 2 exponent bits with bias 1, 3 mantissa bits), so the codes
// are stored as FP6 values and multiplied on the FP6 matrix core, which forms
// the integer dot products exactly in fp32 (|sum| <= 49*128 < 2^24).
// Rows (tokens) are grouped in tiles of 32.  A tile holds 64 lane chunks of
// fp6_lane_bytes(D) bytes: the chunk of row r and half h is chunk 32h + r%32,
// the data one lane of the 32x32x64 matrix-core instruction reads.  It holds,
// for m < D/64, a 24-byte group with channels 64m + 32h + i (i < 32) as 6-bit
// fields at bit 6i (little endian).  D = 64: a chunk is 24 data bytes and 8
// zero bytes, and its two 16-byte halves are stored swapped when bit 3 of the
// chunk index is set (so 16 neighbouring lanes reading their first halves hit
// distinct LDS banks).  Bytes per row on average: 2 * fp6_lane_bytes(D).
__host__ __device__ constexpr int fp6_lane_bytes(int D) { return D == 128 ? 48 : 32; }
__host__ __device__ inline size_t fp6_chunk_offset(int D, size_t row, int h) {
  return (row >> 5) * 64 * (size_t)fp6_lane_bytes(D) + (size_t)(32 * h + (int)(row & 31)) * fp6_lane_bytes(D);
}
// Byte offset inside a D = 64 chunk of its 16-byte half `half` (0: dwords 0-3).
__host__ __device__ inline int fp6_half_offset(int chunk_index, int half) {
  return 16 * (half ^ ((chunk_index >> 3) & 1));
}

struct Dims {
  int B, H, N, D;   // queries: B batches x H heads x N tokens
  int NP;    // N rounded up to a multiple of 128
  int NQB;   // NP / 128: query blocks per head
  // Keys and values: Hk heads (H is a multiple of Hk; query head h reads K/V
  // head h / (H / Hk)) and Nk tokens.  Self-attention: Hk == H, Nk == N.
  int Hk, Nk;
  int NPk;   // Nk rounded up to a multiple of 128
  int NQBk;  // NPk / 128: key blocks per head
  int QB;    // bits per Q/K code: 4 (INT4, stored as FP6) or 8 (INT8 layout)
  int SV;    // 1: smooth V (subtract the per-channel V mean before FP8)
  // 1: adaptive width (QB == 8 layout): the prepass picks INT4 (codes in
  // [-7, 7], stored as int8) or INT8 per K/V head from its statistics and
  // the softmax scale sm.
  int AD;
  float sm;
  // Packed variable-length batches (self-attention only): when cu is not
  // null, head b*H + h is sequence b, tokens cu[b] .. cu[b+1]-1 of a
  // token-major [T, H, D] tensor, and N is the maximum length (it sets the
  // workspace geometry).
  const int* cu;
  int T;
  __host__ __device__ int BH() const { return B * H; }
  __host__ __device__ int BHk() const { return B * Hk; }
  __host__ __device__ bool self_attention() const { return Hk == H && Nk == N; }
  __host__ __device__ int kv_head(int bh) const { return (bh / H) * Hk + (bh % H) / (H / Hk); }
};

// Where the tokens of head bh live in q, k, v and o: token i starts at element
// base + i*stride; n tokens are valid.  For packed batches the sequence length
// is clamped to [0, N] and to the tensor (offsets outside [0, T] give an
// empty sequence), so malformed offsets never lead outside the buffers.
struct HeadIO {
  int n;
  size_t base, stride;
};
// Query head bh (q and o).
__device__ inline HeadIO head_io(const Dims& d, int bh) {
  HeadIO io;
  if (!d.cu) {
    io.n = d.N;
    io.base = (size_t)bh * d.N * d.D;
    io.stride = (size_t)d.D;
    return io;
  }
  const int b = bh / d.H, h = bh % d.H;
  const int s = d.cu[b], e = d.cu[b + 1];
  int n = (s < 0 || s > d.T) ? 0 : min(e - s, min(d.N, d.T - s));
  n = n < 0 ? 0 : n;
  io.n = n;
  io.base = (((size_t)(n > 0 ? s : 0)) * d.H + h) * d.D;
  io.stride = (size_t)d.H * d.D;
  return io;
}
// Key/value head bhk (k and v); packed batches have Hk == H and Nk == N.
__device__ inline HeadIO head_io_kv(const Dims& d, int bhk) {
  if (d.cu) return head_io(d, bhk);
  HeadIO io;
  io.n = d.Nk;
  io.base = (size_t)bhk * d.Nk * d.D;
  io.stride = (size_t)d.D;
  return io;
}

// Device buffers written by the prepass and read by the attention kernel.
// Query-side arrays use (H, NP, NQB), key/value-side arrays (Hk, NPk, NQBk).
struct Bufs {
  uint8_t* q_codes;   // QB 4: FP6 tiles (above), QB 8: int8 [B,H,NP,D]
  uint8_t* k_codes;   // same layout, [B,Hk,NPk,...]
  float* q_scale;     // [B,H,NP]
  float* k_scale;     // [B,Hk,NPk/16]
  float* q_mean;      // [B,H,NQB,D]
  float* k_mean;      // [B,Hk,D]
  uint8_t* v_codes;   // [B,Hk,NQBk,D,128] e4m3fn, keys permuted inside each 128-key block
  float* v_scale;     // [B,Hk,D]
  float* delta_s;     // [B,H,NQB,NPk]  compensation term
  float* k_part;      // [B,Hk,NQBk,2,D] per-chunk K and V channel sums; then bf16 q_mean
                      //                 pieces 1-2 as [B,H,NQB,2,D] (sized for the larger)
  float* v_part;      // [B,Hk,NQBk,2,D] per-chunk V channel max and min; then bf16 q_mean
                      //                 piece 3 as [B,H,NQB,D]
  float* v_mean;      // [B,Hk,D]        V channel means (zeros without V smoothing)
  // adaptive width only
  float* m2_part;     // [B,Hk,NQBk,2,D] per-chunk K and V channel sums of squares
  float* stat_head;   // [B,Hk,8]        A_Q, E_Q, A_K, E_K, EV, V2 of each K/V head (and its query heads)
  float* stat_qblk;   // [B,H,NQB,2]     per query block: sum of amax^2, sum of centred squares
  float* stat_kblk;   // [B,Hk,NQBk]     per key block: sum of the keys' group amax^2
  int32_t* head_bits; // [B,Hk]          chosen width (4 or 8)
};

// Decoding step (one query token per head): per-range partial outputs.
struct DecodeBufs {
  float* part_o;    // [B*H, S, D] unnormalised outputs of each key range
  float* part_ml;   // [B*H, S, 2] running maximum (log2 domain) and row sum of each range
  int split_keys;   // keys per range (a multiple of 128); S = ceil(Nk / split_keys)
};

hipError_t launch_prepass(const void* q, const void* k, const void* v, int in_dtype, const Dims& d,
                          const Bufs& b, hipStream_t s);
// V statistics only: k_part, v_part (scratch) -> v_scale, v_mean (k_mean 0).
hipError_t launch_v_stats(const void* v, int in_dtype, const Dims& d, const Bufs& b, hipStream_t s);
// Decoding step: V statistics, split-key attention (scores in fp32 from the
// 16-bit keys, FP8 V on the fly), merge of the ranges into o [B*H, D].
hipError_t launch_decode(const void* q, const void* k, const void* v, int in_dtype, const Dims& d, const Bufs& b,
                         const DecodeBufs& db, float ks, void* o, int out_dtype, hipStream_t s);
// Query heads per decoding workgroup for a group of g query heads per K/V head.
int decode_heads_per_group(int g);
hipError_t launch_attn(const Bufs& b, const Dims& d, int causal, float ks, void* o, int out_dtype,
                       hipStream_t s);
// Split key ranges for the fused kernel (dense geometry): per-range states and
// their merge into o.
struct SplitParts {
  float* part_o;     // [B*H*N, S, D] unnormalised O of each range (before vscale)
  float* part_ml;    // [B*H*N, S, 2] running maximum (log2 domain) and row sum
  int split_blocks;  // 128-key blocks per range
  int S;             // ranges: ceil(NQBk / split_blocks)
};
hipError_t launch_attn_split(const Bufs& b, const Dims& d, int causal, float ks, void* o, int out_dtype,
                             const SplitParts& sp, hipStream_t s);
hipError_t launch_qk_debug(const Bufs& b, const Dims& d, int bh, int q0, int k0, int nq, int nk,
                           int32_t* out, hipStream_t s);
hipError_t launch_fp8_encode(const float* in, uint8_t* out, size_t n, hipStream_t s);
hipError_t launch_fp8_mfma_debug(const uint8_t* a, const uint8_t* b, const float* c, float* d, hipStream_t s);

}  // namespace sage
