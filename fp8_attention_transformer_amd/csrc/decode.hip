// SageAttention2 decoding step on gfx950: one query token per sequence and
// query head against Nk cached keys and values, grouped-query heads.
//
// The method is the one of the fused kernel (SageAttention2 abstract, arXiv
// 2411.10958 page): smoothed INT4 QK^T with the compensation term, online
// softmax over 128-key blocks, FP8 P~ and V with the two-level accumulation.
// With one query token its 128-token smoothing block holds that token alone,
// so the block mean is the query itself: the smoothed query is zero, its
// codes and scale are zero, and the score of key j is exactly the
// compensation term DeltaS_j = q . (K_j - mean K) (the integer part
// contributes fma(0, 0, DeltaS)).  Key codes are therefore never needed.
// DeltaS_j = q . K_j - q . mean K, and the second term is one constant per
// query head: the softmax cancels it (the same invariance that lets the
// method smooth K at all).  The kernel therefore scores q . K_j in fp32
// straight from the 16-bit keys, with no K mean: every running maximum (and
// every range maximum of the merge) moves by that constant, and the
// max-subtracted exponents, P~, the row sums and O are those of the method
// up to fp32 rounding.
//
// Memory-bound layout.  The V statistics (channel means and scales) need
// every value, so a decoding step streams V twice and K once: the statistics
// kernel of the prepass over V alone, then this kernel, which reads K and V
// in 16-bit form and never writes codes.  Parallelism comes from
// splitting the keys: workgroup (split, K/V head) runs the online softmax of
// all query heads of its group over one key range with its own running
// maximum (the split-key schedule); a second kernel merges the ranges.
//
// Thread layout for one 128-key block (512 threads): thread (kg, cg) owns the
// 8 channels 8cg..8cg+7 of the KPG keys of key group kg, loaded as 16-byte
// row pieces (one load instruction covers 64/CG whole rows).  Groups of more
// than four query heads per K/V head take several workgroups, each reading
// the keys and values again.  Scores: the
// 8-channel partial dot products are summed across the CG lanes of a key with
// row shifts (DPP).  P~V: each thread keeps partial fp32 accumulators for its
// keys and channels (the two-level recurrence is linear, so partials over key
// subsets add up to the whole); they are summed once per split.
#include "sage_internal.h"
#include "sage_device.h"

namespace sage {
namespace {

constexpr float kLog2_448 = 8.80735492205760410744f;

struct DecodeArgs {
  const uint16_t* q;   // [B, Hq, D]
  const uint16_t* k;   // [B, Hk, Nk, D]
  const uint16_t* v;
  const float* v_scale;   // [B*Hk, D]
  const float* v_mean;
  float* part_o;    // [B*Hq, S, D]  per-range unnormalised outputs
  float* part_ml;   // [B*Hq, S, 2]  per-range running maximum (log2 domain) and row sum
  int Hq, Hk, Nk, S, split_blocks, hgroups;
  float ks;         // sm_scale * log2(e)
};

// Sum over groups of CG consecutive lanes (CG = 8 or 16, inside one 16-lane
// row): with zero fill, after shifts by 1, 2, .., CG/2 the last lane of each
// group holds the sum of its group.
template <int SH>
__device__ __forceinline__ float add_row_shr(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x110 + SH, 0xF, 0xF, true));
}
// The same for NV independent values, one shift step at a time for all.
template <int CG, int NV>
__device__ __forceinline__ void group_sum_last_n(float* v) {
  static_assert(CG == 8 || CG == 16, "lanes per group");
#pragma unroll
  for (int i = 0; i < NV; i++) v[i] = add_row_shr<1>(v[i]);
#pragma unroll
  for (int i = 0; i < NV; i++) v[i] = add_row_shr<2>(v[i]);
#pragma unroll
  for (int i = 0; i < NV; i++) v[i] = add_row_shr<4>(v[i]);
  if constexpr (CG == 16) {
#pragma unroll
    for (int i = 0; i < NV; i++) v[i] = add_row_shr<8>(v[i]);
  }
}

// Whole-wave maximum and sum on the VALU (DPP): shifts inside each 16-lane
// row, then row broadcasts 15 and 31 carry the partial results up to lane 63,
// which is read back as a uniform value.  The maximum fills invalid source
// lanes with the lane's own value, the sum with zero.
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max(float v) {
  return fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), CTRL, ROWS, 0xF,
                                                             false)));
}
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_add(float v) {
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROWS, 0xF, true));
}
__device__ __forceinline__ float wave_max_dpp(float v) {
  v = dpp_max<0x111, 0xF>(v);   // row_shr:1
  v = dpp_max<0x112, 0xF>(v);   // row_shr:2
  v = dpp_max<0x114, 0xF>(v);   // row_shr:4
  v = dpp_max<0x118, 0xF>(v);   // row_shr:8
  v = dpp_max<0x142, 0xA>(v);   // row_bcast:15 into rows 1 and 3
  v = dpp_max<0x143, 0xC>(v);   // row_bcast:31 into rows 2 and 3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v = dpp_add<0x111, 0xF>(v);
  v = dpp_add<0x112, 0xF>(v);
  v = dpp_add<0x114, 0xF>(v);
  v = dpp_add<0x118, 0xF>(v);
  v = dpp_add<0x142, 0xA>(v);
  v = dpp_add<0x143, 0xC>(v);
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// e4m3 byte pair (bytes 0-1, or 2-3 with HI) -> two floats (exact).
template <bool HI>
__device__ __forceinline__ void fp8x2_decode(uint32_t w, float& a, float& b) {
  const auto f = __builtin_amdgcn_cvt_pk_f32_fp8((int)w, HI);
  a = f[0];
  b = f[1];
}

// (V - vmean) / vscale for 8 channels with their own scales, correctly
// rounded in fp32 with the sign of zero kept (div_rn_signed), or by true
// divisions when the workgroup holds a zero scale or one outside div_rn's
// exact case (slow: one flag per workgroup, set up front).
__device__ __forceinline__ void fp8_quotients8(float* x, const float* rdv, const float* dv, bool slow) {
  if (slow) {
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = dv[e] == 0.0f ? 0.0f : x[e] / dv[e];
  } else {
#pragma unroll
    for (int e = 0; e < 8; e++) x[e] = div_rn_signed(x[e], dv[e], rdv[e]);
  }
}

// acc + a.lo*b.lo + a.hi*b.hi over packed 16-bit pairs (bf16 or fp16), the
// products exact in fp32
typedef __bf16 v2bf_t __attribute__((ext_vector_type(2)));
typedef _Float16 v2h_t __attribute__((ext_vector_type(2)));
template <int IN>
__device__ __forceinline__ float dot2(int a, int b, float acc) {
  if constexpr (IN == kBF16)
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(v2bf_t, a), __builtin_bit_cast(v2bf_t, b), acc, false);
  else
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(v2h_t, a), __builtin_bit_cast(v2h_t, b), acc, false);
}

template <int IN>
__device__ __forceinline__ void decode8(const v4i& raw, float* x) {
#pragma unroll
  for (int w = 0; w < 4; w++) {
    x[2 * w] = in_to_f32<IN>((uint16_t)((uint32_t)raw[w] & 0xFFFF));
    x[2 * w + 1] = in_to_f32<IN>((uint16_t)((uint32_t)raw[w] >> 16));
  }
}

// grid (S key ranges, B*Hk*hgroups), 512 threads (8 waves, two per SIMD);
// HG <= 4 query heads per workgroup.  A range is processed in chunks of up to
// kChunkBlocks key blocks, each in four phases separated by barriers:
//  S  scores of every block of the chunk into LDS;
//  M  the maximum of each (head, block), one wave per pair;
//  E  per (head, block): the running maximum after that block (from the
//     carried maximum and the block maxima before it, exactly the online
//     recurrence), alpha, p' = exp2(s - m + log2 448), its FP8 rounding
//     (decoded in place of the score) and the block's row sum of those
//     e4m3 values;
//  V  FP8 codes of V on the fly, O = alpha*O, then O += P~ V block by block;
//     one thread per head carries the running maximum and l' = alpha*l' +
//     rowsum into the next chunk.
// K (phase S) and V (phase V) stream through registers, the next block's
// rows loading while one is processed.
constexpr int kThreads = 512;
constexpr int kChunkBlocks = 8;

template <int IN, int D, int HG>
__global__ void __launch_bounds__(kThreads) decode_kernel(DecodeArgs a) {
  static_assert(HG >= 1 && HG <= 4, "heads per workgroup");
  constexpr int CG = D / 8;            // 16-byte channel groups per row
  constexpr int KG = kThreads / CG;    // key groups per block
  constexpr int KPG = kBK / KG;        // keys per group: 4 (D = 128) or 2 (D = 64)
  constexpr int NW = kThreads / 64;
  constexpr int ROWB = 2 * D;          // bytes per 16-bit row
  constexpr int CB = kChunkBlocks, CK = CB * kBK;
  static_assert(NW * D <= CK, "the final reduction fits the score buffer");
  __shared__ float sS[HG][CK];         // scores, then decoded FP8 P~; at the end the cross-wave sums
  __shared__ float sBmax[HG][CB], sAlpha[HG][CB], sRs[HG][CB];
  __shared__ float sM[HG], sL[HG];     // carried running maximum and row sum per head
  __shared__ float sDV[D], sRDV[D], sVB[D];

  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = lane % CG, kg = tid / CG;
  const int split = blockIdx.x;
  const int hgrp = blockIdx.y % a.hgroups, bhk = blockIdx.y / a.hgroups;
  const int b = bhk / a.Hk, hk = bhk % a.Hk;
  const int g = a.Hq / a.Hk;
  const int h0 = hgrp * HG;                 // first head of this workgroup inside its K/V group
  const int nh = min(HG, g - h0);           // heads in use
  const int bhq0 = b * a.Hq + hk * g + h0;  // flat index of head h0
  const size_t kvbase = (size_t)bhk * a.Nk * D;
  const int nkb = (a.Nk + kBK - 1) / kBK;
  const int t0 = split * a.split_blocks, t1 = min(nkb, t0 + a.split_blocks);

  // V scale, its reciprocal and the V mean per channel (LDS: read per key)
  int hard = 0;        // a scale outside div_rn's exact case: true divisions for this workgroup
  bool vslow = false;  // the workgroup-wide verdict, set at the first barrier
  if (tid < D) {
    const float dv = a.v_scale[(size_t)bhk * D + tid];
    hard = (dv == 0.0f || div_rn_hard(dv)) ? 1 : 0;
    sDV[tid] = dv;
    sRDV[tid] = dv == 0.0f ? 0.0f : 1.0f / dv;
    sVB[tid] = a.v_mean[(size_t)bhk * D + tid];
  }
  if (tid < HG) {
    sM[tid] = -__builtin_inff();
    sL[tid] = 0.0f;
  }
  float O[HG][8];
#pragma unroll
  for (int h = 0; h < HG; h++)
#pragma unroll
    for (int e = 0; e < 8; e++) O[h][e] = 0.0f;

  // Buffer resources over this head's keys and values: rows at or past Nk
  // read as zeros, and so does the out-of-range offset used for blocks past
  // the end of a chunk, so every load is unconditional.
  const uint32_t head_bytes = (uint32_t)a.Nk * ROWB;
  const __amdgpu_buffer_rsrc_t rk =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.k + kvbase), (short)0, (int)head_bytes, 0x00020000);
  const __amdgpu_buffer_rsrc_t rv =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a.v + kvbase), (short)0, (int)head_bytes, 0x00020000);
  const int lane_off = KPG * kg * ROWB + 16 * cg;
  auto issue = [&](__amdgpu_buffer_rsrc_t r, int t, int tend, v4i* buf) {
    const int base = t < tend ? t * kBK * ROWB + lane_off : 0x7FFFFFF0;
#pragma unroll
    for (int kk = 0; kk < KPG; kk++)
      buf[kk] = __builtin_bit_cast(v4i, __builtin_amdgcn_raw_buffer_load_b128(r, base + kk * ROWB, 0, 0));
  };

  // ---- scores of block t (slot i of the chunk): partial dot products over
  //      this thread's 8 channels, then the KPG*HG independent sums over the
  //      CG lanes of each key, step by step (the chains hide each other's DPP
  //      latency); the last lane of each group stores its keys' scores.
  auto scores = [&](int t, int i, const v4i* kc, const v4i* qw) {
    float ps[KPG][HG];
#pragma unroll
    for (int kk = 0; kk < KPG; kk++) {
#pragma unroll
      for (int h = 0; h < HG; h++) {
        float p = 0.0f;
#pragma unroll
        for (int w = 0; w < 4; w++) p = dot2<IN>(qw[h][w], kc[kk][w], p);
        ps[kk][h] = p;
      }
    }
    group_sum_last_n<CG, KPG * HG>(&ps[0][0]);
    if (cg == CG - 1) {
#pragma unroll
      for (int h = 0; h < HG; h++) {
        float sc[KPG];
#pragma unroll
        for (int kk = 0; kk < KPG; kk++)
          sc[kk] = (t * kBK + KPG * kg + kk < a.Nk) ? ps[kk][h] * a.ks : -__builtin_inff();
        if constexpr (KPG == 4) *(float4*)&sS[h][i * kBK + KPG * kg] = make_float4(sc[0], sc[1], sc[2], sc[3]);
        else *(float2*)&sS[h][i * kBK + KPG * kg] = make_float2(sc[0], sc[1]);
      }
    }
  };

  // ---- P~V of block t (slot i): O = alpha*O, then V -> FP8 codes of the
  //      method (smoothed, per-channel scale) and O += P~ V over this
  //      thread's keys (the one-level form: the block's products accumulate
  //      into the rescaled running sum)
  auto pv = [&](int t, int i, const v4i* vc) {
    const bool ragged = (t + 1) * kBK > a.Nk;   // the block holds keys past the end
#pragma unroll
    for (int h = 0; h < HG; h++) {
      const float alpha = sAlpha[h][i];
#pragma unroll
      for (int e = 0; e < 8; e++) O[h][e] = O[h][e] * alpha;
    }
    float vbar[8], rdv[8], dvv[8];
#pragma unroll
    for (int e = 0; e < 8; e += 4) {
      *(float4*)&vbar[e] = *(const float4*)&sVB[8 * cg + e];
      *(float4*)&rdv[e] = *(const float4*)&sRDV[8 * cg + e];
      *(float4*)&dvv[e] = *(const float4*)&sDV[8 * cg + e];
    }
#pragma unroll
    for (int kk = 0; kk < KPG; kk++) {
      const int key = KPG * kg + kk;
      float x[8];
      decode8<IN>(vc[kk], x);
#pragma unroll
      for (int e = 0; e < 8; e++) x[e] = x[e] - vbar[e];
      if (ragged) {   // padding keys stay exactly zero
        const bool valid = t * kBK + key < a.Nk;
#pragma unroll
        for (int e = 0; e < 8; e++) x[e] = valid ? x[e] : 0.0f;
      }
      fp8_quotients8(x, rdv, dvv, vslow);
      float vq[8];
#pragma unroll
      for (int w = 0; w < 2; w++) {
        const uint32_t pk = fp8x4(x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3]);
        fp8x2_decode<false>(pk, vq[4 * w], vq[4 * w + 1]);
        fp8x2_decode<true>(pk, vq[4 * w + 2], vq[4 * w + 3]);
      }
#pragma unroll
      for (int h = 0; h < HG; h++) {
        const float p = sS[h][i * kBK + key];
#pragma unroll
        for (int e = 0; e < 8; e++) O[h][e] = __builtin_fmaf(p, vq[e], O[h][e]);   // products of FP8 values are exact
      }
    }
  };

  v4i kA[KPG], kB[KPG], vA[KPG], vB[KPG];
  issue(rk, t0, t1, kA);
  vslow = __syncthreads_or(hard) != 0;   // also publishes sM, sL and the V constants
  for (int tc = t0; tc < t1; tc += CB) {
    const int te = min(t1, tc + CB), nb = te - tc;
    // ---- S (kA holds block tc); the query rows are reloaded per chunk (they
    //      would otherwise hold registers through the V phase)
    {
      v4i qw[HG];   // this thread's 8 query channels per head, packed pairs
#pragma unroll
      for (int h = 0; h < HG; h++) {
        qw[h] = v4i{0, 0, 0, 0};
        if (h < nh) qw[h] = *(const v4i*)(a.q + (size_t)(bhq0 + h) * D + 8 * cg);
      }
      for (int i = 0; i < nb; i += 2) {
        issue(rk, tc + i + 1, te, kB);
        scores(tc + i, i, kA, qw);
        issue(rk, tc + i + 2, te, kA);
        if (i + 1 < nb) scores(tc + i + 1, i + 1, kB, qw);
      }
    }
    issue(rv, tc, te, vA);   // the chunk's first V block loads during M and E
    __syncthreads();
    // ---- M: block maxima, pairs (head p % HG, block p / HG) over the waves
    for (int pr = wave; pr < HG * nb; pr += NW) {
      const int h = pr % HG, i = pr / HG;
      const float bmax = wave_max_dpp(fmaxf(sS[h][i * kBK + 2 * lane], sS[h][i * kBK + 2 * lane + 1]));
      if (lane == 0) sBmax[h][i] = bmax;
    }
    __syncthreads();
    // ---- E: running maximum after block i, alpha, FP8 P~ and row sum
    for (int pr = wave; pr < HG * nb; pr += NW) {
      const int h = pr % HG, i = pr / HG;
      float mprev = sM[h];
      for (int u = 0; u < i; u++) mprev = fmaxf(mprev, sBmax[h][u]);
      const float mnew = fmaxf(mprev, sBmax[h][i]);
      const float alpha = __builtin_amdgcn_exp2f(mprev - mnew);
      const float mm = mnew - kLog2_448;
      float* row = &sS[h][i * kBK + 2 * lane];
      const float p0 = __builtin_amdgcn_exp2f(row[0] - mm), p1 = __builtin_amdgcn_exp2f(row[1] - mm);
      float q0, q1;
      fp8x2_decode<false>(fp8x2(p0, p1), q0, q1);
      const float rs = wave_sum_dpp(q0 + q1);   // the row sum of the e4m3 values that weight V
      row[0] = q0;
      row[1] = q1;
      if (lane == 0) {
        sAlpha[h][i] = alpha;
        sRs[h][i] = rs;
      }
    }
    __syncthreads();
    // ---- V; one thread per head carries the state into the next chunk
    if (tid < HG) {
      float m = sM[tid], l = sL[tid];
      for (int i = 0; i < nb; i++) {
        m = fmaxf(m, sBmax[tid][i]);
        l = sAlpha[tid][i] * l + sRs[tid][i];
      }
      sM[tid] = m;
      sL[tid] = l;
    }
    for (int i = 0; i < nb; i += 2) {
      issue(rv, tc + i + 1, te, vB);
      pv(tc + i, i, vA);
      issue(rv, tc + i + 2, te, vA);
      if (i + 1 < nb) pv(tc + i + 1, i + 1, vB);
    }
    issue(rk, te, t1, kA);   // the next chunk's first K block
    __syncthreads();
  }

  // ---- sum the partial outputs of the key groups: inside the wave (lanes
  //      with the same channel group), then across the waves
#pragma unroll
  for (int h = 0; h < HG; h++)
#pragma unroll
    for (int e = 0; e < 8; e++) {
      float s = O[h][e];
#pragma unroll
      for (int o = CG; o < 64; o <<= 1) s = s + __shfl_xor(s, o);
      O[h][e] = s;
    }
  float* sRed = &sS[0][0];   // [NW][HG][D]
  if (lane < CG) {
#pragma unroll
    for (int h = 0; h < HG; h++)
#pragma unroll
      for (int e = 0; e < 8; e++) sRed[(wave * HG + h) * D + 8 * cg + e] = O[h][e];
  }
  __syncthreads();
  for (int i = tid; i < HG * D; i += kThreads) {
    const int h = i / D, c = i % D;
    if (h < nh) {
      float s = sRed[h * D + c];
#pragma unroll
      for (int w = 1; w < NW; w++) s = s + sRed[(w * HG + h) * D + c];
      a.part_o[((size_t)(bhq0 + h) * a.S + split) * D + c] = s;
    }
  }
  if (tid < nh) {
    a.part_ml[((size_t)(bhq0 + tid) * a.S + split) * 2] = sM[tid];
    a.part_ml[((size_t)(bhq0 + tid) * a.S + split) * 2 + 1] = sL[tid];
  }
}

// Merge of the key ranges: D/4 threads per query head, four channels each
// (16-byte loads of the partial outputs), 256/(D/4) heads per workgroup.
// Per channel: M = max m_s, w_s = exp2(m_s - M), O = fma(w_s, O_s, O) and
// l' = fma(w_s, l'_s, l') in range order, then O * vscale / l' + vmean.
__global__ void __launch_bounds__(256) decode_merge_kernel(const float* __restrict__ part_o,
                                                           const float* __restrict__ part_ml,
                                                           const float* __restrict__ v_scale,
                                                           const float* __restrict__ v_mean, int BHq, int Hq, int Hk,
                                                           int S, int D, void* __restrict__ o, int out_dtype) {
  const int tpr = D / 4;
  const int bhq = blockIdx.x * (256 / tpr) + threadIdx.x / tpr, c0 = 4 * (threadIdx.x % tpr);
  if (bhq >= BHq) return;
  const int g = Hq / Hk, bhk = (bhq / Hq) * Hk + (bhq % Hq) / g;
  const float* ml = part_ml + (size_t)bhq * S * 2;
  float M = -__builtin_inff();
#pragma unroll 8
  for (int s = 0; s < S; s++) M = fmaxf(M, ml[2 * s]);
  float acc[4] = {0.0f, 0.0f, 0.0f, 0.0f}, l = 0.0f;
#pragma unroll 8
  for (int s = 0; s < S; s++) {
    const float w = __builtin_amdgcn_exp2f(ml[2 * s] - M);
    const float4 p = *(const float4*)(part_o + ((size_t)bhq * S + s) * D + c0);
    acc[0] = __builtin_fmaf(w, p.x, acc[0]);
    acc[1] = __builtin_fmaf(w, p.y, acc[1]);
    acc[2] = __builtin_fmaf(w, p.z, acc[2]);
    acc[3] = __builtin_fmaf(w, p.w, acc[3]);
    l = __builtin_fmaf(w, ml[2 * s + 1], l);
  }
  const float4 vs = *(const float4*)(v_scale + (size_t)bhk * D + c0);
  const float4 vm = *(const float4*)(v_mean + (size_t)bhk * D + c0);
  const size_t oi = (size_t)bhq * D + c0;
  store_out(o, oi, (acc[0] * vs.x) / l + vm.x, out_dtype);
  store_out(o, oi + 1, (acc[1] * vs.y) / l + vm.y, out_dtype);
  store_out(o, oi + 2, (acc[2] * vs.z) / l + vm.z, out_dtype);
  store_out(o, oi + 3, (acc[3] * vs.w) / l + vm.w, out_dtype);
}

template <int IN, int D, int HG>
void launch_decode_kernel(const DecodeArgs& a, int BHk, hipStream_t s) {
  hipLaunchKernelGGL((decode_kernel<IN, D, HG>), dim3(a.S, BHk * a.hgroups), dim3(kThreads), 0, s, a);
}

template <int IN, int D>
void launch_decode_hg(const DecodeArgs& a, int BHk, int hg, hipStream_t s) {
  if (hg == 1) launch_decode_kernel<IN, D, 1>(a, BHk, s);
  else if (hg == 2) launch_decode_kernel<IN, D, 2>(a, BHk, s);
  else launch_decode_kernel<IN, D, 4>(a, BHk, s);
}

}  // namespace

int decode_heads_per_group(int g) { return g <= 1 ? 1 : g <= 2 ? 2 : 4; }

hipError_t launch_decode(const void* q, const void* k, const void* v, int in_dtype, const Dims& d, const Bufs& b,
                         const DecodeBufs& db, float ks, void* o, int out_dtype, hipStream_t s) {
  hipError_t e = launch_v_stats(v, in_dtype, d, b, s);
  if (e != hipSuccess) return e;
  const int g = d.H / d.Hk, hg = decode_heads_per_group(g);
  DecodeArgs a;
  a.q = (const uint16_t*)q;
  a.k = (const uint16_t*)k;
  a.v = (const uint16_t*)v;
  a.v_scale = b.v_scale;
  a.v_mean = b.v_mean;
  a.part_o = db.part_o;
  a.part_ml = db.part_ml;
  a.Hq = d.H;
  a.Hk = d.Hk;
  a.Nk = d.Nk;
  a.split_blocks = db.split_keys / kBK;
  a.S = (d.NQBk + a.split_blocks - 1) / a.split_blocks;
  a.hgroups = (g + hg - 1) / hg;
  a.ks = ks;
  if (in_dtype == kBF16) {
    if (d.D == 64) launch_decode_hg<1, 64>(a, d.BHk(), hg, s);
    else launch_decode_hg<1, 128>(a, d.BHk(), hg, s);
  } else {
    if (d.D == 64) launch_decode_hg<0, 64>(a, d.BHk(), hg, s);
    else launch_decode_hg<0, 128>(a, d.BHk(), hg, s);
  }
  const int hpw = 256 / (d.D / 4);   // query heads per merge workgroup
  hipLaunchKernelGGL(decode_merge_kernel, dim3((d.BH() + hpw - 1) / hpw), dim3(256), 0, s, db.part_o, db.part_ml,
                     b.v_scale, b.v_mean, d.BH(), d.H, d.Hk, a.S, d.D, o, out_dtype);
  return hipGetLastError();
}

}  // namespace sage
