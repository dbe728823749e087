// SageAttention2 fused attention forward on gfx950.
//
// Method (SageAttention2 abstract, arXiv 2411.10958 page): INT4 QK^T with
// fine-grained scales, online softmax, FP8 P~ and V, and a two-level
// accumulation of P~V (a per-block partial in a fresh FP32 buffer, then added
// into an FP32 running buffer).  The two levels exist because FP8 tensor
// cores elsewhere accumulate in reduced precision.  The gfx950 FP8
// instruction (measured) forms its 64 products exactly, sums them in groups
// of 8 consecutive k truncated 13 bits below the group's largest exponent,
// and combines the group sums with its fp32 accumulator about 25 bits below
// the larger, then rounds to fp32: the in-group truncation does not depend on
// what the accumulator holds, and adding into a large accumulator costs about
// one fp32 rounding.  So here the running buffer is rescaled by alpha and the
// block's products are accumulated into it by the matrix core directly (the
// rounding order differs from the separate partial).
//
// gfx950 mapping.  A workgroup owns one 128-query block of one head (4 waves x
// 32 queries); for dense non-causal calls at D = 128, two adjacent blocks (8
// waves, one workgroup per CU) that share every staged K/V block, over four
// LDS stages.  Scores are built transposed, S^T = K * Q^T, on 32x32 matrix-
// core tiles: every lane then holds one query and 16 keys of each 32-key tile,
// so the dequantization factor is one scalar per lane and tile (per-token Q
// scale times the scale of the lane's 16-key K group) and the row maximum of
// the online softmax stays inside a lane plus one exchange with the partner
// lane 32 away.  P~ stays in registers: converted to e4m3 it is directly the
// B operand of the FP8 matrix core (v_mfma_f32_32x32x64_f8f6f4) computing
// O^T += V^T P~^T, with V stored by the prepass in the matching permuted
// channel-major layout, and the row sum l' of the same e4m3 values (an
// all-ones A operand).
//
// INT4 codes on the FP6 matrix core.  gfx950 has no INT4 matrix instruction,
// but every integer in [-7, 7] is exact in FP6 e2m3, and the f8f6f4
// instruction with FP6 operands (format 2) runs at twice the FP8 rate and sums
// the integer products exactly (its grouped summation keeps every integer
// product and sum: |dot| <= 49*128 < 2^24; the INT4 tiles are pinned
// bit-exact against the oracle).  The prepass
// stores the codes as FP6 in the lane order of the instruction, so a lane's
// operand is one contiguous chunk and the accumulator is the dot product as a
// float, with no unpacking and no conversion.  INT8 codes use the INT8 matrix
// core (v_mfma_i32_32x32x32_i8).
#include "sage_internal.h"
#include "sage_device.h"

#include <type_traits>

namespace sage {
namespace {

constexpr float kLog2_448 = 8.80735492205760410744f;

// The larger of the values of lane l and lane l^32 (the two half-waves hold
// the same query): v_permlane32_swap exchanges the upper half of its first
// operand with the lower half of its second, so with both operands equal to v
// the two results hold, in every lane, v of the lane itself and of its
// partner.
__device__ __forceinline__ float pair_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Code layout and operand shapes.  BITS 4: FP6 tiles of lane chunks (see
// fp6_chunk_offset), D/64 FP6 instructions per 32x32 tile.  BITS 8: int8 rows
// of D bytes; a lane feeds 16-byte chunks 2m + h of its row (matrix step m,
// half-wave h), D/32 INT8 instructions per tile.
template <int D, int BITS>
struct QKCfg;
template <int D>
struct QKCfg<D, 4> {
  static constexpr int LS = fp6_lane_bytes(D);   // bytes per lane chunk
  static constexpr int ROWB = 2 * LS;            // bytes per row (average)
  static constexpr int NM = D / 64;              // FP6 instructions per tile
};
template <int D>
struct QKCfg<D, 8> {
  static constexpr int ROWB = D;
  static constexpr int NCH = D / 32;   // 16-byte chunks per lane per tile
  static constexpr int CPR = D / 16;   // 16-byte chunks per row
};

template <int D, int BITS>
struct QOperand;
template <int D>
struct QOperand<D, 4> {
  v8i x[D / 64];   // six dwords of FP6 fields used per instruction
};
template <int D>
struct QOperand<D, 8> {
  v4i x[D / 32];
};

// The FP6 operands of one lane chunk (`ci` = its chunk index in the tile).
template <int D>
__device__ __forceinline__ void load_fp6_chunk(const uint8_t* chunk, int ci, v8i* a) {
  // Dwords 6-7 of an FP6 operand are not read by the instruction: leaving
  // them undefined lets the 12 loaded dwords serve as both operands in place.
  if constexpr (D == 128) {
    const v4i u0 = *(const v4i*)chunk, u1 = *(const v4i*)(chunk + 16), u2 = *(const v4i*)(chunk + 32);
    const v8i w01 = __builtin_shufflevector(u0, u1, 0, 1, 2, 3, 4, 5, 6, 7);
    a[0] = __builtin_shufflevector(w01, w01, 0, 1, 2, 3, 4, 5, -1, -1);
    a[1] = __builtin_shufflevector(u1, u2, 2, 3, 4, 5, 6, 7, -1, -1);
  } else {
    const v4i lo = *(const v4i*)(chunk + fp6_half_offset(ci, 0));
    const v4i hi = *(const v4i*)(chunk + fp6_half_offset(ci, 1));
    a[0] = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, -1, -1);
  }
}

// Query operands of this lane (query row `qrow` of the head in padded
// coordinates, half h).
template <int D, int BITS>
__device__ __forceinline__ void load_q_operand(const uint8_t* __restrict__ q_codes_head, int qrow, int h,
                                               QOperand<D, BITS>& op) {
  if constexpr (BITS == 4) {
    load_fp6_chunk<D>(q_codes_head + fp6_chunk_offset(D, qrow, h), 32 * h + (qrow & 31), op.x);
  } else {
#pragma unroll
    for (int m = 0; m < D / 32; m++) op.x[m] = *(const v4i*)(q_codes_head + (size_t)qrow * D + m * 32 + h * 16);
  }
}

// One 32-key tile of S^T as floats holding the exact integer dot products.
// FP6: a[m] = this lane's K chunk operands; INT8: a[m] = its 16-byte chunks.
template <int D>
__device__ __forceinline__ v16f qk_tile_fp6(const v8i* a, const QOperand<D, 4>& op) {
  v16f s = {};
#pragma unroll
  for (int m = 0; m < D / 64; m++) s = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a[m], op.x[m], s, 2, 2, 0, 0, 0, 0);
  return s;
}
// INT8: |dot| <= 127^2 * 128 < 2^24, so the int32 -> fp32 conversion is exact.
template <int D>
__device__ __forceinline__ v16f qk_tile_i8(const v4i* a, const QOperand<D, 8>& op) {
  v16i s = {};
#pragma unroll
  for (int m = 0; m < D / 32; m++) s = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[m], op.x[m], s, 0, 0, 0);
  v16f f;
#pragma unroll
  for (int r = 0; r < 16; r++) f[r] = (float)s[r];
  return f;
}

// Map the hardware workgroup id to (head, query block).  Workgroups are
// dealt round-robin to the 8 XCDs; renumbering gives every XCD a contiguous
// range of logical ids, so the query blocks of one head share an L2.
__device__ __forceinline__ int xcd_logical_id(int pid, int nwg) {
  const int xcd = pid & 7, idx = pid >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

// LDS layouts are XOR-swizzled in 16-byte chunks so that the 16 lanes served
// together by one ds_read_b128 hit distinct banks.
//   K tile (INT8): 128 rows (keys) x D bytes; chunk c of row r at c ^ kswz(r).
//   K tile (FP6): copied as stored; lane chunks of 48 bytes (D = 128) or with
//   swapped halves (D = 64) already spread 16 lanes over all banks.
//   V tile: D rows (channels) x 128 bytes; chunk c of row r at c ^ ((r>>1)&7).
template <int CPR>
__device__ __forceinline__ int kswz(int r) {
  static_assert(CPR == 2 || CPR == 4 || CPR == 8, "chunks per row");
  return CPR == 8 ? (r >> 1) & 7 : (CPR == 4 ? (r >> 2) & 3 : (r >> 3) & 1);
}
__device__ __forceinline__ int vswz(int r) { return (r >> 1) & 7; }

// Direct HBM/L2 -> LDS copy of one 128-key block: K codes and FP8 V.  Lane l
// of a wave writes LDS chunk (wave base + l); it fetches the global chunk whose
// swizzled position that is.  Chunk e = 256*i + 64*wave + lane of either array
// comes from byte 4096*i + 1024*wave + off, where the lane part `off` does not
// depend on i (the swizzles repeat every 256 chunks): one 32-bit offset per
// array, computed once, and a wave-uniform base per copy instruction.
template <int D, int BITS>
__device__ __forceinline__ uint32_t k_src_offset(int wave, int lane) {
  constexpr int ROWB = QKCfg<D, BITS>::ROWB;
  const int e = 64 * wave + lane;
  int src = 16 * e;
  if constexpr (BITS == 8) {
    constexpr int CPR = QKCfg<D, 8>::CPR;
    const int r = e / CPR, c = (e % CPR) ^ kswz<CPR>(r);
    src = r * ROWB + 16 * c;
  }
  return (uint32_t)(src - 1024 * wave);
}
__device__ __forceinline__ uint32_t v_src_offset(int wave, int lane) {
  const int e = 64 * wave + lane, r = e / 8, c = (e % 8) ^ vswz(r);
  return (uint32_t)(r * kBK + 16 * c - 1024 * wave);
}

// The copies use buffer loads straight to LDS: the per-lane offset is one VGPR
// and block, round and wave offsets stay scalar.  K codes and V bytes of a
// block are staged at different times (see the key loop), so separately.
template <int D, int BITS>
__device__ __forceinline__ void stage_k_async(uint8_t* sK, __amdgpu_buffer_rsrc_t rk, int t, int wave, uint32_t koff) {
  constexpr int ROWB = QKCfg<D, BITS>::ROWB;
  constexpr int KCH = kBK * ROWB / 16 / 256;
  static_assert(KCH * 16 * 256 == kBK * ROWB, "whole copy rounds");
  const uint32_t kb = (uint32_t)t * (kBK * ROWB) + 1024u * wave;
#pragma unroll
  for (int i = 0; i < KCH; i++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rk, (lds_ptr_t)(sK + 4096 * i + 1024 * wave), 16, koff, kb + 4096 * i, 0,
                                             0);
}
template <int D>
__device__ __forceinline__ void stage_v_async(uint8_t* sV, __amdgpu_buffer_rsrc_t rv, int t, int wave, uint32_t voff) {
  constexpr int VCH = D * kBK / 16 / 256;
  const uint32_t vb = (uint32_t)t * (D * kBK) + 1024u * wave;
#pragma unroll
  for (int i = 0; i < VCH; i++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rv, (lds_ptr_t)(sV + 4096 * i + 1024 * wave), 16, voff, vb + 4096 * i, 0,
                                             0);
}

// NR copy rounds of 4 KB (256 lanes x 16 bytes) from the global chunks at
// base + 4096 i + 1024 wave + off to LDS dst + 4096 i + 1024 wave.
template <int NR>
__device__ __forceinline__ void stage_rounds(uint8_t* dst, __amdgpu_buffer_rsrc_t r, uint32_t base, int wave,
                                             uint32_t off) {
  const uint32_t b = base + 1024u * wave;
#pragma unroll
  for (int i = 0; i < NR; i++)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)(dst + 4096 * i + 1024 * wave), 16, off, b + 4096 * i, 0, 0);
}

template <int D, bool CAUSAL>
struct AttnState {
  static constexpr int NDT = D / 32;
  v16f O[NDT];
  float m, l;
};

// The parts of one 128-key block for this wave.  qk_part: S^T tiles (exact
// integer dot products as floats).  softmax_part: dequantization into the
// log2 domain, masking, online-softmax update, P~ -> e4m3 matrix-core
// operands.  rescale and pv_mfma: O = alpha*O, then O += P~V on the FP8
// matrix core (accumulated into the fp32 running buffer).
template <int D, int BITS>
__device__ __forceinline__ void qk_part(v16f* S, const QOperand<D, BITS>& qop, const uint8_t* cK, int n, int h) {
#pragma unroll
  for (int T = 0; T < 4; T++) {
    if constexpr (BITS == 4) {
      constexpr int LS = QKCfg<D, 4>::LS;
      const int ci = 32 * h + n;
      v8i a[D / 64];
      load_fp6_chunk<D>(cK + (64 * T + ci) * LS, ci, a);
      S[T] = qk_tile_fp6<D>(a, qop);
    } else {
      constexpr int NCH = QKCfg<D, 8>::NCH, CPR = QKCfg<D, 8>::CPR;
      const int row = 32 * T + n;
      v4i a[NCH];
#pragma unroll
      for (int m = 0; m < NCH; m++) a[m] = *(const v4i*)(cK + row * D + 16 * ((2 * m + h) ^ kswz<CPR>(row)));
      S[T] = qk_tile_i8<D>(a, qop);
    }
  }
}

// One FP8 matrix-core product of P~V: O[dt] += V(channels 32dt.., keys of
// half kh) * P~(keys of half kh)^T, V read from the block's LDS slot.
template <int D, bool CAUSAL>
__device__ __forceinline__ void pv_mfma(AttnState<D, CAUSAL>& as, const v8i* P8, const uint8_t* cV, int n, int h,
                                        int dt, int kh) {
  const int row = 32 * dt + n;
  const int c0 = 4 * kh + 2 * h;
  const v4i lo = *(const v4i*)(cV + row * kBK + 16 * (c0 ^ vswz(row)));
  const v4i hi = *(const v4i*)(cV + row * kBK + 16 * ((c0 + 1) ^ vswz(row)));
  const v8i av = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  as.O[dt] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, P8[kh], as.O[dt], 0, 0, 0, 0, 0, 0);
}

// Quarter T of the previous block's P~V products, pinned in the schedule next
// to the vector work of score tile T (the scheduler would otherwise gather
// them).
template <int D, bool CAUSAL>
__device__ __forceinline__ void pv_quarter(AttnState<D, CAUSAL>& as, const v8i* P8p, const uint8_t* cVp, int n, int h,
                                           int T) {
  constexpr int NPV = 2 * (D / 32);   // products per block: (kh, dt) kh-major
#pragma unroll
  for (int j = T * NPV / 4; j < (T + 1) * NPV / 4; j++) pv_mfma<D, CAUSAL>(as, P8p, cVp, n, h, j % (D / 32), j / (D / 32));
  __builtin_amdgcn_sched_barrier(0);
}

// O = alpha * O (the running buffer, once the previous block's products are
// in it).  Skipped when no running maximum of the wave moved (alpha = 1 in
// every lane, and O * 1 = O): on long key ranges the maxima settle and most
// blocks need no rescale.
template <int D, bool CAUSAL>
__device__ __forceinline__ void rescale(AttnState<D, CAUSAL>& as, float alpha) {
  if (!__any(alpha != 1.0f)) return;
#pragma unroll
  for (int dt = 0; dt < D / 32; dt++)
#pragma unroll
    for (int r = 0; r < 16; r++) as.O[dt][r] = as.O[dt][r] * alpha;
}

// Keys past the head's last key are masked by their compensation entry in LDS
// (-inf, so fma(S, c, -inf) = -inf), with no branch and no per-key test in
// the loop.  At D = 64 the loop also keeps a branch that masks them (the same
// -inf): without the branch the scheduler spreads the work and takes the
// kernel past 168 registers, costing it its third wave per SIMD.
template <int D>
constexpr bool kTailBranch = D == 64;

// The softmax of block t.  klim: the last key this lane's query may see
// (causal); need_mask: some key of block t is masked for some query of the
// workgroup (wave-uniform): causally, or at D = 64 past the last key.  PIPE (the
// pipelined key loop): P8p and cVp are the previous block's P~ and V slot,
// and `alpha` holds that block's alpha on entry: O is rescaled by it once
// this block's maximum is known, then the previous block's 2*D/32 P~V
// products (accumulated into O) are spread over this block's exponentials,
// so the matrix core works on them while the vector unit works here; `alpha`
// leaves with this block's alpha.  For the first block of a range P8p is zero
// (the products add exactly zero).
template <int D, bool CAUSAL, bool SPLIT, bool PIPE>
__device__ __forceinline__ void softmax_part(AttnState<D, CAUSAL>& as, const v16f* S, const float* cDS,
                                             const float* cKS, float dq, float ks, int t, int klim, int h, int nk,
                                             bool need_mask, v8i* P8, float& alpha, const v8i* P8p,
                                             const uint8_t* cVp, int n) {
  float s2[4][16];
  float tmax[4];
#pragma unroll
  for (int T = 0; T < 4; T++) {
    const float c = (dq * cKS[2 * T + h]) * ks;
#pragma unroll
    for (int r = 0; r < 16; r++) {
      const int key = 32 * T + 8 * (r >> 2) + 4 * h + (r & 3);
      s2[T][r] = __builtin_fmaf(S[T][r], c, cDS[key]);
    }
    if ((CAUSAL || kTailBranch<D>) && need_mask) {
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int key = t * kBK + 32 * T + 8 * (r >> 2) + 4 * h + (r & 3);
        const bool bad = (kTailBranch<D> && key >= nk) || (CAUSAL && key > klim);
        if (bad) s2[T][r] = -__builtin_inff();
      }
    }
    // two chains of three-input maxima per tile (v_max3: two values per op)
    float c0 = fmaxf(fmaxf(s2[T][0], s2[T][1]), s2[T][2]);
    float c1 = fmaxf(fmaxf(s2[T][8], s2[T][9]), s2[T][10]);
#pragma unroll
    for (int r = 3; r < 7; r += 2) {
      c0 = fmaxf(fmaxf(c0, s2[T][r]), s2[T][r + 1]);
      c1 = fmaxf(fmaxf(c1, s2[T][8 + r]), s2[T][8 + r + 1]);
    }
    tmax[T] = fmaxf(fmaxf(c0, s2[T][7]), fmaxf(c1, s2[T][15]));
  }
  const float bmax = pair_max(fmaxf(fmaxf(fmaxf(tmax[0], tmax[1]), tmax[2]), tmax[3]));
  // Pipelined: O = alpha(t-1) * O before block t-1's products below.  Here, not
  // between the S^T products and the dequantization: its wave-uniform branch
  // would end the basic block there and keep the scheduler from starting the
  // dequantization and maxima of the first tiles under the later products.
  if constexpr (PIPE) rescale<D, CAUSAL>(as, alpha);
  const float mnew = fmaxf(as.m, bmax);
  // Split key ranges: a query may see no key of a range yet (its running max
  // stays -inf); referencing 0 then keeps alpha, p' and the state at 0.
  const float mref = SPLIT ? (mnew == -__builtin_inff() ? 0.0f : mnew) : mnew;
  alpha = __builtin_amdgcn_exp2f(as.m - mref);
  const float mm = mref - kLog2_448;
  // ---- p' = exp2(s2 - mm) in [0, 448]; P~ -> e4m3 B operands (the row sum
  //      of the e4m3 values follows on the matrix core: row_sum)
#pragma unroll
  for (int T = 0; T < 4; T++) {
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; r++) p[r] = __builtin_amdgcn_exp2f(s2[T][r] - mm);
#pragma unroll
    for (int w = 0; w < 4; w++)
      P8[T >> 1][4 * (T & 1) + w] =
          (int)fp8x4(p[4 * w], p[4 * w + 1], p[4 * w + 2], p[4 * w + 3], __float_as_int(s2[T][4 * w]));
    if constexpr (PIPE) pv_quarter<D, CAUSAL>(as, P8p, cVp, n, h, T);
  }
  as.m = mnew;
}

// l' = alpha * l' + (the block's row sum of P~): the sum of the e4m3 values
// that multiply V, on the FP8 matrix core: an all-ones A operand (e4m3 1.0 =
// 0x38) against P~ gives, in every accumulator row of the lane's query, the
// sum over the block's 128 keys (each value exact; as in the P~V products,
// values 2^13 below the largest of their 8-key group drop out of its sum).
__device__ __forceinline__ v16f row_sum_mfma(const v8i* P8) {
  const v8i ones = {0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838, 0x38383838};
  v16f rs = {};
  rs = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, P8[0], rs, 0, 0, 0, 0, 0, 0);
  rs = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(ones, P8[1], rs, 0, 0, 0, 0, 0, 0);
  return rs;
}

// The update itself, placed after the code that follows the products (the
// next block's copies, the compensation row, the barrier): every register of
// the accumulator stays allocated until then, so no vector instruction in
// between writes one of them while the matrix core still does (which would
// cost a wait of the product's full duration).
template <int D, bool CAUSAL>
__device__ __forceinline__ void row_sum_late(AttnState<D, CAUSAL>& as, const v16f& rs, float alpha) {
  as.l = alpha * as.l + rs[0];
  asm volatile("" ::"v"(rs));
}

// Two outputs as one packed pair of 16-bit values, each rounded to nearest
// even (one conversion instruction per pair on gfx950); the same bits as
// store_out's per-element rounding for finite values.
__device__ __forceinline__ uint32_t out_pack2(float a, float b, int out_dtype) {
  typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
  typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
  if (out_dtype == kOutBF16) return __builtin_bit_cast(uint32_t, v2bf_t{(__bf16)a, (__bf16)b});
  return __builtin_bit_cast(uint32_t, v2h_t{(_Float16)a, (_Float16)b});
}

// Workgroup barrier for LDS only: waits for this wave's LDS operations, not
// for its vector-memory loads and stores (as __syncthreads() would).  The
// memory clobber keeps the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// Dense causal calls with at most this many query blocks per head pair the
// blocks in workgroups (measured: +4-7% at 32 and 64 blocks, -1-2% at 128
// and 256, where the finer units balance better).
constexpr int kPairMaxBlocks = 64;
// Key ranges of at most this many 128-key blocks on average run the
// pipelined key loop (D = 128 only).
constexpr int kPipeMaxBlocks = 96;

// SPLIT: workgroup (head, key range, query block) runs the method over one
// range of key blocks from an empty state and writes its unnormalised state
// (O, running max, row sum) for a merge kernel (dense geometry only).
// QPW = 2: 8-wave workgroups over two adjacent query blocks (waves 4-7 the
// second), each K/V block copied once for both (the first block's waves copy
// K, the second's V); the two waves of a SIMD then come from one workgroup.
// Only with the pipelined key loop (four LDS stages).
template <int D, int BITS, bool CAUSAL, bool SPLIT, bool PIPE, int QPW = 1>
__global__ void __launch_bounds__(256 * QPW, 2 / QPW) attn_kernel(Bufs b, Dims d, float ks, void* __restrict__ o,
                                                                int out_dtype, SplitParts sp) {
  static_assert(QPW == 1 || (!CAUSAL && !SPLIT && PIPE), "two query blocks per workgroup: dense non-causal, pipelined");
  constexpr int ROWB = QKCfg<D, BITS>::ROWB;
  constexpr int NDT = D / 32;
  // K/V staging: two LDS stages of one 128-key block each (double buffer),
  // as separate arrays so the compiler can tell the block being read from the
  // block being filled by the asynchronous copies.
  // two query blocks per workgroup: K stages rounded up to whole V copy rounds
  constexpr int KSLOT = QPW == 2 ? (D * kBK > kBK * ROWB ? D * kBK : kBK * ROWB) : kBK * ROWB;
  __shared__ __align__(16) uint8_t sK0[KSLOT], sK1[KSLOT];
  __shared__ __align__(16) uint8_t sV0[D * kBK], sV1[D * kBK];
  __shared__ float sDS0[QPW * kBK], sDS1[QPW * kBK];
  // Two query blocks per workgroup: four stages (block t+2 is copied while
  // block t is computed and block t-1's V is still read); the raw
  // compensation rows (both query blocks) and K scales (64 lanes, the 8
  // scales repeated) of each stage are copied straight into LDS.
  constexpr bool S4 = QPW == 2;
  __shared__ __align__(16) uint8_t sK2[S4 ? KSLOT : 16], sV2[S4 ? D * kBK : 16];
  __shared__ __align__(16) uint8_t sK3[S4 ? KSLOT : 16], sV3[S4 ? D * kBK : 16];
  __shared__ float sDS2[S4 ? QPW * kBK : 4], sDS3[S4 ? QPW * kBK : 4];
  __shared__ __align__(16) float sRD0[S4 ? QPW * kBK : 4], sRD1[S4 ? QPW * kBK : 4], sRD2[S4 ? QPW * kBK : 4],
      sRD3[S4 ? QPW * kBK : 4];
  __shared__ __align__(16) float sRK0[S4 ? 64 : 4], sRK1[S4 ? 64 : 4], sRK2[S4 ? 64 : 4], sRK3[S4 ? 64 : 4];
  __shared__ float sKS0[kBK / kKGroup], sKS1[kBK / kKGroup];
  __shared__ float sVS[D], sVM[D];   // V scales and means of the head, for the epilogue
  auto bK = [&](int i) { return i == 0 ? sK0 : sK1; };
  auto bV = [&](int i) { return i == 0 ? sV0 : sV1; };
  auto bDS = [&](int i) { return i == 0 ? sDS0 : sDS1; };
  auto bKS = [&](int i) { return i == 0 ? sKS0 : sKS1; };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave8 = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int half = QPW == 1 ? 0 : wave8 >> 2;   // which query block of the workgroup
  const int wave = wave8 & 3;                   // wave within its query block
  const int htid = tid & 255;                   // thread within its query block
  const int n = lane & 31, h = lane >> 5;

  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  // One query block (bh, rng, qb) of work; returns early for an empty one.
  auto item = [&](const int bh, const int rng, const int qb) {
  const HeadIO io = head_io(d, bh);              // queries and outputs
  const int nqb = (io.n + kBQ - 1) / kBQ;
  if (qb >= nqb) return;                         // past a shorter packed sequence (whole workgroup)
  const int bhk = d.kv_head(bh);
  const int nk = head_io_kv(d, bhk).n;           // keys of this head
  const int nkb = (nk + kBK - 1) / kBK;
  // causal mask aligned at the last key: query i sees keys j <= i + (nk - n)
  const int off = nk - io.n;
  const int qrow = qb * kBQ + wave * 32 + n;     // padded query index of this lane
  const int klim = qrow + off;
  const size_t hrowp = (size_t)bh * d.NP;

  const float* dsrow = b.delta_s + ((size_t)bh * d.NQB + qb) * d.NPk;
  const uint8_t* kblk = b.k_codes + (size_t)bhk * d.NPk * ROWB;
  const uint8_t* vblk = b.v_codes + (size_t)bhk * d.NQBk * D * kBK;
  const float* kscl = b.k_scale + (size_t)bhk * d.NPk / kKGroup;
  // key blocks: all, or (causal) up to the one holding the last valid query's
  // last key; blocks past the first query's limit need the mask
  const int tend = CAUSAL ? (min(qb * kBQ + kBQ, io.n) - 1 + off) / kBK + 1 : nkb;
  const int tmask = CAUSAL ? (qb * kBQ + off) / kBK : nkb;   // first block with a causally masked key
  const bool ragged = nk != nkb * kBK;
  // key blocks of this workgroup: [tb, te)
  const int tb = SPLIT ? rng * sp.split_blocks : 0;
  const int te = SPLIT ? min(tend, tb + sp.split_blocks) : tend;
  if (tb >= te) return;   // no query of this tile sees a key of the range (whole workgroup)

  // the small loads are unconditional, with in-range indices
  float ds_reg, ks_reg;
  const uint32_t koff = k_src_offset<D, BITS>(wave, lane), voff = v_src_offset(wave, lane);
  const __amdgpu_buffer_rsrc_t rk = head_rsrc(kblk, (uint32_t)d.NPk * ROWB);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc(vblk, (uint32_t)d.NPk * D);
  auto issue_k = [&](int t, int slot) {   // K codes, compensation row and K scales of block t
    if (QPW == 1 || half == 0) stage_k_async<D, BITS>(bK(slot), rk, t, wave, koff);
    ds_reg = dsrow[t * kBK + (htid & (kBK - 1))];
    ks_reg = kscl[t * (kBK / kKGroup) + (htid & (kBK / kKGroup - 1))];
  };
  // compensation row (-inf past the head's last key: those keys are masked)
  // and K scales of block t -> LDS
  auto publish = [&](int slot, int t) {
    if (htid < kBK) bDS(slot)[half * kBK + htid] = t * kBK + htid < nk ? ds_reg * ks : -__builtin_inff();
    if (tid < kBK / kKGroup) bKS(slot)[tid] = ks_reg;
  };
  auto issue_v = [&](int t, int slot) {
    if (QPW == 1 || half == 1) stage_v_async<D>(bV(slot), rv, t, wave, voff);
  };

  // The head's V scales and means (read by the epilogue) load first, so the
  // wait below that covers block tb's copies covers them too.
  float vs_reg = 0.0f, vm_reg = 0.0f;
  if (tid < D) {
    vs_reg = b.v_scale[(size_t)bhk * D + tid];
    vm_reg = b.v_mean[(size_t)bhk * D + tid];
  }
  issue_k(tb, 0);
  issue_v(tb, 0);

  QOperand<D, BITS> qop;
  load_q_operand<D, BITS>(b.q_codes + hrowp * ROWB, qrow, h, qop);
  const float dq = b.q_scale[hrowp + qrow];

  AttnState<D, CAUSAL> as;
#pragma unroll
  for (int dt = 0; dt < NDT; dt++)
#pragma unroll
    for (int r = 0; r < 16; r++) as.O[dt][r] = 0.0f;
  as.m = -__builtin_inff();
  as.l = 0.0f;

  wait_vmcnt<0>();
  publish(0, tb);
  if (tid < D) {
    sVS[tid] = vs_reg;
    sVM[tid] = vm_reg;
  }
  __syncthreads();

  if constexpr (QPW == 2) {
    // Two query blocks, pipelined over four LDS stages.  Step t copies block
    // t+2 (K codes by the first block's waves, V bytes by the second's, the
    // raw compensation rows and K scales by all, straight into LDS), computes
    // block t's S^T tiles, rescales O by block t-1's alpha and runs block t's
    // softmax with block t-1's P~V products spread through it (as in the
    // pipelined loop below); its wait at the end covers block t+1 only.  The
    // loop is unrolled by four so that every stage is a named array in every
    // step: the compiler then tells the stages being read from the ones being
    // filled and adds no wait of its own for the copies in flight (with a
    // stage chosen at run time it waits for every copy before the first
    // read).  K is copied in as many 4 KB rounds as V (the 12 KB FP6 block:
    // the extra round reads the start of the next block, or zeros past the
    // head), so every wave issues the same copies per step and the waits
    // count them exactly; nothing is loaded into registers across a step.
    constexpr int VCH = D * kBK / 16 / 256;   // copy rounds per wave and block
    static_assert(VCH * 4096 <= KSLOT && kBK * ROWB <= VCH * 4096, "copy rounds of K and V");
    auto K_ = [&](auto c) -> uint8_t* { constexpr int x = decltype(c)::value; return x == 0 ? sK0 : x == 1 ? sK1 : x == 2 ? sK2 : sK3; };
    auto V_ = [&](auto c) -> uint8_t* { constexpr int x = decltype(c)::value; return x == 0 ? sV0 : x == 1 ? sV1 : x == 2 ? sV2 : sV3; };
    auto DS_ = [&](auto c) -> float* { constexpr int x = decltype(c)::value; return x == 0 ? sDS0 : x == 1 ? sDS1 : x == 2 ? sDS2 : sDS3; };
    auto RD_ = [&](auto c) -> float* { constexpr int x = decltype(c)::value; return x == 0 ? sRD0 : x == 1 ? sRD1 : x == 2 ? sRD2 : sRD3; };
    auto RK_ = [&](auto c) -> float* { constexpr int x = decltype(c)::value; return x == 0 ? sRK0 : x == 1 ? sRK1 : x == 2 ? sRK2 : sRK3; };
    auto issue_kv = [&](int t, auto c) {
      if (half == 0) stage_rounds<VCH>(K_(c), rk, (uint32_t)t * (kBK * ROWB), wave, koff);
      else stage_rounds<VCH>(V_(c), rv, (uint32_t)t * (D * kBK), wave, voff);
    };
    const __amdgpu_buffer_rsrc_t rd = head_rsrc(dsrow, (uint32_t)d.NPk * 4);
    const __amdgpu_buffer_rsrc_t rks = head_rsrc(kscl, (uint32_t)d.NPk / kKGroup * 4);
    auto issue_sc = [&](int t, auto c) {
      float* rdd = RD_(c) + half * kBK;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_ptr_t)rdd, 4, 4u * lane, (uint32_t)t * kBK * 4, 0, 0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rd, (lds_ptr_t)(rdd + 64), 4, 4u * lane, (uint32_t)t * kBK * 4 + 256, 0,
                                               0);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rks, (lds_ptr_t)RK_(c), 4, 4u * (lane & 7),
                                               (uint32_t)t * (kBK / kKGroup) * 4, 0, 0);
    };
    auto publish = [&](auto c, int t) {
      if (htid < kBK)
        DS_(c)[half * kBK + htid] = t * kBK + htid < nk ? RD_(c)[half * kBK + htid] * ks : -__builtin_inff();
    };
    v8i P8p[2] = {};
    float alpha_p = 1.0f;
    auto step = [&](int t, auto c, auto n1, auto n2, auto pv) {
      issue_kv(min(t + 2, te - 1), n2);
      issue_sc(min(t + 2, te - 1), n2);
      v16f S[4];
      qk_part<D, BITS>(S, qop, K_(c), n, h);
      v8i P8[2];
      // block t-1's V stage (before the first block: stage 3, zeroed, with P8p = 0)
      const uint8_t* cVp = V_(pv);
      softmax_part<D, CAUSAL, SPLIT, true>(as, S, DS_(c) + half * kBK, RK_(c), dq, ks, t, klim, h, nk, false, P8,
                                           alpha_p, P8p, cVp, n);
      const v16f rs = row_sum_mfma(P8);
      P8p[0] = P8[0];
      P8p[1] = P8[1];
      wait_vmcnt<VCH + 3>();
      publish(n1, min(t + 1, te - 1));
      lds_barrier();
      row_sum_late<D, CAUSAL>(as, rs, alpha_p);
    };
    using I0 = std::integral_constant<int, 0>;
    using I1 = std::integral_constant<int, 1>;
    using I2 = std::integral_constant<int, 2>;
    using I3 = std::integral_constant<int, 3>;
    issue_kv(min(tb + 1, te - 1), I1{});
    issue_sc(min(tb + 1, te - 1), I1{});
    if (lane < kBK / kKGroup) sRK0[lane] = sKS0[lane];
    // the first step's "previous block" products read stage 3 with P8p = 0:
    // zero bytes there, so that they add exactly zero
#pragma unroll
    for (int i = 0; i < D * kBK / 16 / 512; i++) *(v4i*)(sV3 + 16 * (tid + 512 * i)) = v4i{0, 0, 0, 0};
    lds_barrier();
    int tl = tb;   // the last block
    for (int t = tb; t < te; t += 4) {
      tl = t;
      step(t, I0{}, I1{}, I2{}, I3{});
      if (t + 1 >= te) break;
      tl = t + 1;
      step(t + 1, I1{}, I2{}, I3{}, I0{});
      if (t + 2 >= te) break;
      tl = t + 2;
      step(t + 2, I2{}, I3{}, I0{}, I1{});
      if (t + 3 >= te) break;
      tl = t + 3;
      step(t + 3, I3{}, I0{}, I1{}, I2{});
    }
    // the last block's P~V (its V stage is (tl - tb) mod 4)
    rescale<D, CAUSAL>(as, alpha_p);
    {
      const int sl = (tl - tb) & 3;
      const uint8_t* cVl = sl == 0 ? sV0 : sl == 1 ? sV1 : sl == 2 ? sV2 : sV3;
#pragma unroll
      for (int j = 0; j < 2 * NDT; j++) pv_mfma<D, CAUSAL>(as, P8p, cVl, n, h, j % NDT, j / NDT);
    }
    wait_vmcnt<0>();   // no copy into LDS outlives the workgroup
  } else if constexpr (!PIPE) {
    // Plain key loop: iteration t stages block t+1 (K codes and V bytes) and
    // runs block t's S^T tiles, softmax and P~V in sequence.
    for (int t = tb; t < te; t++) {
      const int slot = (t - tb) & 1;
      const bool ahead = t + 1 < te;   // block t+1 exists: stage it now
      if (ahead) {
        issue_k(t + 1, slot ^ 1);
        issue_v(t + 1, slot ^ 1);
      }
      const bool need_mask = (CAUSAL && t >= tmask) || (kTailBranch<D> && ragged && t == nkb - 1);
      v16f S[4];
      qk_part<D, BITS>(S, qop, bK(slot), n, h);
      v8i P8[2];
      float alpha;
      softmax_part<D, CAUSAL, SPLIT, false>(as, S, bDS(slot) + half * kBK, bKS(slot), dq, ks, t, klim, h, nk, need_mask,
                                            P8, alpha, nullptr, nullptr, n);
      const v16f rs = row_sum_mfma(P8);
      rescale<D, CAUSAL>(as, alpha);
#pragma unroll
      for (int dt = 0; dt < NDT; dt++) {
        pv_mfma<D, CAUSAL>(as, P8, bV(slot), n, h, dt, 0);
        pv_mfma<D, CAUSAL>(as, P8, bV(slot), n, h, dt, 1);
      }
      if (ahead) {
        wait_vmcnt<0>();   // block t+1 has landed (this wave's copies)
        publish(slot ^ 1, t + 1);
      }
      row_sum_late<D, CAUSAL>(as, rs, alpha);
      __syncthreads();
    }
  } else {
    // Software-pipelined key loop.  Iteration t computes block t's S^T tiles,
    // rescales O by block t-1's alpha, and runs block t's softmax (vector unit)
    // with block t-1's P~V products spread through it (matrix core).  Block t's
    // V bytes are therefore read one iteration after its K codes, and staged
    // one iteration later: K codes of block t+1 and V bytes of block t are
    // copied during iteration t (two LDS slots each; a slot is rewritten only
    // after the barrier that follows its last read).
    v8i P8p[2] = {};       // P~ of the previous block (zero before the first)
    float alpha_p = 1.0f;  // alpha of the previous block
  #pragma clang loop unroll(disable)
    for (int t = tb; t < te; t++) {
      const int slot = (t - tb) & 1;
      const bool ahead = t + 1 < te;
      if (t > tb) __syncthreads();   // block t's K codes, compensation row and scales are in LDS
      if (ahead) issue_k(t + 1, slot ^ 1);
      if (t > tb) stage_v_async<D>(bV(slot), rv, t, wave, voff);
      v16f S[4];
      qk_part<D, BITS>(S, qop, bK(slot), n, h);
      const bool need_mask = (CAUSAL && t >= tmask) || (kTailBranch<D> && ragged && t == nkb - 1);
      v8i P8[2];
      // the previous block's V slot; in the first iteration any valid slot (its
      // products with P8p = 0 add zero)
      const uint8_t* cVp = bV(t > tb ? slot ^ 1 : 0);
      softmax_part<D, CAUSAL, SPLIT, true>(as, S, bDS(slot), bKS(slot), dq, ks, t, klim, h, nk, need_mask, P8, alpha_p, P8p,
                                       cVp, n);
      const v16f rs = row_sum_mfma(P8);
      P8p[0] = P8[0];
      P8p[1] = P8[1];
      wait_vmcnt<0>();   // K codes of block t+1 and V bytes of block t have landed (this wave's copies)
      if (ahead) publish(slot ^ 1, t + 1);
      row_sum_late<D, CAUSAL>(as, rs, alpha_p);
    }
    // the last block's P~V
    rescale<D, CAUSAL>(as, alpha_p);
    __syncthreads();
    {
      const uint8_t* cVl = bV((te - 1 - tb) & 1);
  #pragma unroll
      for (int j = 0; j < 2 * NDT; j++) pv_mfma<D, CAUSAL>(as, P8p, cVl, n, h, j % NDT, j / NDT);
    }
  }

  const int qi = qrow;
  if constexpr (SPLIT) {
    // ---- this range's state for the merge: O (before vscale), m, l'
    if (qi < io.n) {
      const size_t row = (size_t)bh * d.N + qi;
      float* po = sp.part_o + (row * sp.S + rng) * D;
#pragma unroll
      for (int dt = 0; dt < NDT; dt++)
#pragma unroll
        for (int q4 = 0; q4 < 4; q4++)   // 4 consecutive channels per 16-byte store
          *(float4*)(po + 32 * dt + 8 * q4 + 4 * h) =
              make_float4(as.O[dt][4 * q4], as.O[dt][4 * q4 + 1], as.O[dt][4 * q4 + 2], as.O[dt][4 * q4 + 3]);
      if (h == 0) {
        sp.part_ml[(row * sp.S + rng) * 2] = as.m;
        sp.part_ml[(row * sp.S + rng) * 2 + 1] = as.l;
      }
    }
    return;
  }
  // ---- epilogue: O = fma(O_run * vscale, 1 / l', vmean).  The scales and
  //      means come from LDS (global loads here would each wait behind the
  //      stores before them: the output may alias them as far as the compiler
  //      knows); a lane's registers 4q..4q+3 of a tile are 4 consecutive
  //      channels, stored with one 8-byte (16-bit outputs) or 16-byte (fp32)
  //      store when the output is 16-byte aligned.
  if (qi < io.n) {
    const size_t orow = io.base + (size_t)qi * io.stride;
    const float inv_l = 1.0f / as.l;
    const bool vec = ((uintptr_t)o & 15) == 0;
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int q4 = 0; q4 < 4; q4++) {
        const int c0 = 32 * dt + 8 * q4 + 4 * h;
        float y[4];
#pragma unroll
        for (int j = 0; j < 4; j++) y[j] = __builtin_fmaf(as.O[dt][4 * q4 + j] * sVS[c0 + j], inv_l, sVM[c0 + j]);
        if (!vec) {
#pragma unroll
          for (int j = 0; j < 4; j++) store_out(o, orow + c0 + j, y[j], out_dtype);
        } else if (out_dtype == kOutF32) {
          *(float4*)((float*)o + orow + c0) = make_float4(y[0], y[1], y[2], y[3]);
        } else {
          *(uint2*)((uint16_t*)o + orow + c0) = make_uint2(out_pack2(y[0], y[1], out_dtype), out_pack2(y[2], y[3], out_dtype));
        }
      }
  }
  };
  // Dense causal with at most kPairMaxBlocks query blocks per head (the grid
  // then has ceil(NQB/2) workgroups per head): workgroup p takes query blocks
  // NQB-1-p and p (the heaviest with the lightest), so every workgroup has
  // NQB+1 key blocks of work and there are half as many; short workgroups
  // otherwise come faster than the hardware refills their slots.  Otherwise
  // one block per workgroup:
  // dense head-major (the query blocks of a head share an XCD's L2); packed
  // sequences of unequal length query-block-major, so the heaviest blocks of
  // every sequence start first; split: (head, range) pairs take the place of
  // heads, so the query blocks of one key range share an L2.
  // Between the items of a pair only LDS needs ordering (the second one's
  // prologue rewrites the slots and the V statistics the first one's
  // epilogue read): the first one's output stores drain while the second
  // one's prologue loads are in flight.
  // D = 128: one call site of item(), so its code (the key loop with the
  // masked and unmasked softmax) exists once; inlined at each of three call
  // sites the causal kernel took 80 KB and outgrew the instruction cache.
  // D = 64 keeps two call sites: its code is smaller, and the loop would cost
  // it 35 registers and its third wave per SIMD.
  int bh, rng = 0, qb0, qb1 = -1;
  if (QPW == 2) {
    const int np = d.NQB / 2;
    bh = logical / np;
    qb0 = 2 * (logical % np) + half;
  } else if (CAUSAL && !SPLIT && !d.cu && (int)gridDim.x != d.NQB * d.BH()) {
    const int npair = (d.NQB + 1) / 2;
    const int p = logical % npair;
    bh = logical / npair;
    qb0 = d.NQB - 1 - p;
    if (p != qb0) qb1 = p;
  } else {
    const int hs = logical / d.NQB;
    bh = d.cu ? logical % d.BH() : (SPLIT ? hs / sp.S : hs);
    rng = SPLIT ? hs % sp.S : 0;
    const int jq = d.cu ? logical / d.BH() : logical % d.NQB;
    qb0 = CAUSAL ? d.NQB - 1 - jq : jq;
  }
  if constexpr (!CAUSAL || SPLIT) {
    item(bh, rng, qb0);
  } else if constexpr (D == 64) {
    item(bh, rng, qb0);
    if (qb1 >= 0) {
      lds_barrier();
      item(bh, rng, qb1);
    }
  } else {
#pragma clang loop unroll(disable)
    for (int k = 0; k < 2; k++) {
      const int qb = k == 0 ? qb0 : qb1;
      if (qb < 0) break;
      if (k) lds_barrier();
      item(bh, rng, qb);
    }
  }
}

// Debug: exact int32 QK^T for a (nq x nk) window of one head, through the same
// tile function as the fused kernel.  Grid (ceil(nq/32), ceil(nk/32)), 64 threads.
template <int D, int BITS>
__global__ void __launch_bounds__(64) qk_debug_kernel(Bufs b, Dims d, int bh, int q0, int k0, int nq, int nk,
                                                      int32_t* __restrict__ out) {
  constexpr int ROWB = QKCfg<D, BITS>::ROWB;
  const int lane = threadIdx.x, n = lane & 31, h = lane >> 5;
  const int qloc = blockIdx.x * 32 + n;
  const int kbase = blockIdx.y * 32;
  const int qrow = min(q0 + qloc, d.NP - 1);
  QOperand<D, BITS> qop;
  load_q_operand<D, BITS>(b.q_codes + (size_t)bh * d.NP * ROWB, qrow, h, qop);
  const int krow = min(k0 + kbase + n, d.NPk - 1);
  const uint8_t* khead = b.k_codes + (size_t)d.kv_head(bh) * d.NPk * ROWB;
  v16f s;
  if constexpr (BITS == 4) {
    v8i a[D / 64];
    load_fp6_chunk<D>(khead + fp6_chunk_offset(D, krow, h), 32 * h + (krow & 31), a);
    s = qk_tile_fp6<D>(a, qop);
  } else {
    v4i a[D / 32];
#pragma unroll
    for (int m = 0; m < D / 32; m++) a[m] = *(const v4i*)(khead + (size_t)krow * D + m * 32 + h * 16);
    s = qk_tile_i8<D>(a, qop);
  }
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int kloc = kbase + 8 * (r >> 2) + 4 * h + (r & 3);
    if (qloc < nq && kloc < nk) out[(size_t)qloc * nk + kloc] = (int32_t)s[r];
  }
}

// Merge of the key ranges: D/4 threads per query row, four channels each
// (16-byte loads of the partial outputs), 256/(D/4) rows per workgroup.  Row
// i reads the ranges holding a key it sees (range r starts at key
// r*split_keys <= i + Nk - N when causal), M = max m_r, w_r = exp2(m_r - M),
// O = fma(w_r, O_r, O) and l' = fma(w_r, l'_r, l') in range order, then the
// fused kernel's epilogue fma(O * vscale, 1 / l', vmean).  One range gives
// the unsplit kernel's result bit for bit (w = 1).
__global__ void __launch_bounds__(256) split_merge_kernel(Bufs b, Dims d, int causal, SplitParts sp, void* o,
                                                          int out_dtype) {
  const int tpr = d.D / 4;                                  // threads per row
  const int row = blockIdx.x * (256 / tpr) + threadIdx.x / tpr;
  const int c0 = 4 * (threadIdx.x % tpr);
  if (row >= d.BH() * d.N) return;
  const int bh = row / d.N, i = row % d.N, bhk = d.kv_head(bh);
  const int limit = causal ? i + (d.Nk - d.N) : d.Nk - 1;   // last key row i sees
  const int rlast = min(sp.S - 1, limit / (sp.split_blocks * kBK));
  const float* ml = sp.part_ml + (size_t)row * sp.S * 2;
  float M = -__builtin_inff();
  for (int r = 0; r <= rlast; r++) M = fmaxf(M, ml[2 * r]);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, l = 0.0f;
  for (int r = 0; r <= rlast; r++) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * r] - M);
    const float4 p = *(const float4*)(sp.part_o + ((size_t)row * sp.S + r) * d.D + c0);
    acc[0] = __builtin_fmaf(w, p.x, acc[0]);
    acc[1] = __builtin_fmaf(w, p.y, acc[1]);
    acc[2] = __builtin_fmaf(w, p.z, acc[2]);
    acc[3] = __builtin_fmaf(w, p.w, acc[3]);
    l = __builtin_fmaf(w, ml[2 * r + 1], l);
  }
  const float inv_l = 1.0f / l;
  const float4 vs = *(const float4*)(b.v_scale + (size_t)bhk * d.D + c0);
  const float4 vm = *(const float4*)(b.v_mean + (size_t)bhk * d.D + c0);
  const float y0 = __builtin_fmaf(acc[0] * vs.x, inv_l, vm.x), y1 = __builtin_fmaf(acc[1] * vs.y, inv_l, vm.y);
  const float y2 = __builtin_fmaf(acc[2] * vs.z, inv_l, vm.z), y3 = __builtin_fmaf(acc[3] * vs.w, inv_l, vm.w);
  const size_t oi = (size_t)row * d.D + c0;
  if (((uintptr_t)o & 15) != 0) {
    store_out(o, oi, y0, out_dtype);
    store_out(o, oi + 1, y1, out_dtype);
    store_out(o, oi + 2, y2, out_dtype);
    store_out(o, oi + 3, y3, out_dtype);
  } else if (out_dtype == kOutF32) {
    *(float4*)((float*)o + oi) = make_float4(y0, y1, y2, y3);
  } else {
    *(uint2*)((uint16_t*)o + oi) = make_uint2(out_pack2(y0, y1, out_dtype), out_pack2(y2, y3, out_dtype));
  }
}

template <int D, int BITS, bool SPLIT>
hipError_t attn_impl(const Bufs& b, const Dims& d, int causal, float ks, void* o, int out_dtype, const SplitParts& sp,
                     hipStream_t s) {
  // dense causal with few query blocks: one workgroup per pair (see the kernel)
  const int qunits = (causal && !SPLIT && !d.cu && d.NQB <= kPairMaxBlocks) ? (d.NQB + 1) / 2 : d.NQB;
  const dim3 grid(qunits * d.BH() * (SPLIT ? sp.S : 1));
  // The pipelined key loop pays off on short key ranges (measured at D = 128:
  // LLM prefill N 4096 causal +4-8%, DiT N 4608 +2-8%, N 16384 causal +7%)
  // and costs ~2% on long ones (N 16384 non-causal, N 32768 causal); at D = 64
  // its extra registers cost the INT8 kernel its third wave.  Both loops give
  // bit-identical results.
  const int mean_blocks = SPLIT ? sp.split_blocks : (causal ? (d.NQBk + 1) / 2 : d.NQBk);
  bool launched = false;
  // Dense non-causal D = 128 with an even number of query blocks: two query
  // blocks per workgroup, pipelined (measured, bit-identical, builds
  // interleaved; first with three stages and no pipelining against one block
  // per workgroup: N 16384 INT4 +1.6%, INT8 +4.3%; N 32768 +0.4%, +3.7%;
  // against the one-block pipelined loop: DiT +0.7-1.8%, +7%; N 8192
  // +2.7-4.4%, +7-8%; then the four-stage pipelined form against that:
  // INT4 +1.2-2.4% on all four, INT8 within 0.5%).
  // Causal ranges keep one block per workgroup: the two-block form (the
  // first block's waves masked through the second's extra key block, pairs
  // heaviest first) measured 2-3% slower on N 8192-32768 and 16-18% on LLM
  // prefill (B4 H32 N4096), where it replaces the heavy/light pairing.
  if constexpr (D == 128 && !SPLIT) {
    if (!causal && !d.cu && d.NQB % 2 == 0) {
      hipLaunchKernelGGL((attn_kernel<D, BITS, false, false, true, 2>), dim3(d.NQB / 2 * d.BH()), dim3(512), 0, s, b,
                         d, ks, o, out_dtype, sp);
      launched = true;
    }
  }
  if constexpr (D == 128) {
    if (!launched)
    if (mean_blocks <= kPipeMaxBlocks) {
      if (causal)
        hipLaunchKernelGGL((attn_kernel<D, BITS, true, SPLIT, true>), grid, dim3(256), 0, s, b, d, ks, o, out_dtype, sp);
      else
        hipLaunchKernelGGL((attn_kernel<D, BITS, false, SPLIT, true>), grid, dim3(256), 0, s, b, d, ks, o, out_dtype, sp);
      launched = true;
    }
  }
  if (!launched) {
    if (causal)
      hipLaunchKernelGGL((attn_kernel<D, BITS, true, SPLIT, false>), grid, dim3(256), 0, s, b, d, ks, o, out_dtype, sp);
    else
      hipLaunchKernelGGL((attn_kernel<D, BITS, false, SPLIT, false>), grid, dim3(256), 0, s, b, d, ks, o, out_dtype, sp);
  }
  if (SPLIT) {
    const long long rows = (long long)d.BH() * d.N, rpw = 256 / (d.D / 4);
    hipLaunchKernelGGL(split_merge_kernel, dim3((unsigned)((rows + rpw - 1) / rpw)), dim3(256), 0, s, b, d, causal, sp,
                       o, out_dtype);
  }
  return hipGetLastError();
}

template <bool SPLIT>
hipError_t attn_dispatch(const Bufs& b, const Dims& d, int causal, float ks, void* o, int out_dtype,
                         const SplitParts& sp, hipStream_t s) {
  if (d.QB == 8)
    return d.D == 64 ? attn_impl<64, 8, SPLIT>(b, d, causal, ks, o, out_dtype, sp, s)
                     : attn_impl<128, 8, SPLIT>(b, d, causal, ks, o, out_dtype, sp, s);
  return d.D == 64 ? attn_impl<64, 4, SPLIT>(b, d, causal, ks, o, out_dtype, sp, s)
                   : attn_impl<128, 4, SPLIT>(b, d, causal, ks, o, out_dtype, sp, s);
}

}  // namespace

hipError_t launch_attn(const Bufs& b, const Dims& d, int causal, float ks, void* o, int out_dtype, hipStream_t s) {
  return attn_dispatch<false>(b, d, causal, ks, o, out_dtype, SplitParts{}, s);
}

hipError_t launch_attn_split(const Bufs& b, const Dims& d, int causal, float ks, void* o, int out_dtype,
                             const SplitParts& sp, hipStream_t s) {
  return attn_dispatch<true>(b, d, causal, ks, o, out_dtype, sp, s);
}

// One FP8 32x32x64 product d = a*b + c on the matrix core (one wave), with
// the operand and accumulator layouts of the fused kernel's P~V products.
__global__ void __launch_bounds__(64) fp8_mfma_debug_kernel(const uint8_t* __restrict__ a, const uint8_t* __restrict__ b,
                                                            const float* c, float* d) {
  const int l = threadIdx.x, j = l & 31, h = l >> 5;
  v8i av, bv;
#pragma unroll
  for (int w = 0; w < 8; w++) {
    av[w] = *(const int*)(a + j * 64 + 32 * h + 4 * w);
    uint32_t x = 0;
#pragma unroll
    for (int u = 0; u < 4; u++) x |= (uint32_t)b[(32 * h + 4 * w + u) * 32 + j] << (8 * u);
    bv[w] = (int)x;
  }
  v16f acc;
#pragma unroll
  for (int r = 0; r < 16; r++) acc[r] = c[(8 * (r >> 2) + 4 * h + (r & 3)) * 32 + j];
  acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, bv, acc, 0, 0, 0, 0, 0, 0);
#pragma unroll
  for (int r = 0; r < 16; r++) d[(8 * (r >> 2) + 4 * h + (r & 3)) * 32 + j] = acc[r];
}

hipError_t launch_qk_debug(const Bufs& b, const Dims& d, int bh, int q0, int k0, int nq, int nk, int32_t* out,
                           hipStream_t s) {
  const dim3 grid((nq + 31) / 32, (nk + 31) / 32);
  if (d.D == 64 && d.QB == 4) hipLaunchKernelGGL((qk_debug_kernel<64, 4>), grid, dim3(64), 0, s, b, d, bh, q0, k0, nq, nk, out);
  else if (d.D == 64) hipLaunchKernelGGL((qk_debug_kernel<64, 8>), grid, dim3(64), 0, s, b, d, bh, q0, k0, nq, nk, out);
  else if (d.QB == 4) hipLaunchKernelGGL((qk_debug_kernel<128, 4>), grid, dim3(64), 0, s, b, d, bh, q0, k0, nq, nk, out);
  else hipLaunchKernelGGL((qk_debug_kernel<128, 8>), grid, dim3(64), 0, s, b, d, bh, q0, k0, nq, nk, out);
  return hipGetLastError();
}

hipError_t launch_fp8_mfma_debug(const uint8_t* a, const uint8_t* b, const float* c, float* d, hipStream_t s) {
  hipLaunchKernelGGL(fp8_mfma_debug_kernel, dim3(1), dim3(64), 0, s, a, b, c, d);
  return hipGetLastError();
}

}  // namespace sage
