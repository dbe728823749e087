// SageAttention2 forward -- CPU oracle (test infrastructure only).
//
// This file is the plain, slow, obviously-correct reference that the GPU path is
// checked against. Only the tests, the smoke check and the benchmark's CPU
// baseline may load it; the product library never links or calls it, and the
// two share no source, header, table or constant generator.
//
// What the method computes comes from the SageAttention2 pages:
//   * "SageAttention2: Efficient Attention with Thorough Outlier Smoothing and
//     Per-thread INT4 Quantization" (arXiv 2411.10958 abstract page):
//     Q,K -> INT4 at a hardware-friendly thread-level granularity; P~,V -> FP8;
//     smoothing of Q to make INT4 QK^T accurate; a two-level accumulation for the
//     FP8 P~V product.  The title's "thorough outlier smoothing" is read as
//     smoothing K as well (per-channel mean over tokens).
//   * "SageAttention2 Technical Report" summary page, Key Contributions 1-2
//     (INT4 Q,K; FP8 P~,V; smoothing).
// Everything the pages leave open is a documented reading, applied identically
// here and in the GPU kernels:
//   - BQ_MEAN = 128 tokens per Q-smoothing block (the tail block averages its
//     valid tokens only); K is smoothed with one mean per channel over all N.
//   - Means: fp32, sequential sums over 128-token chunks in token order, then a
//     sequential sum of the chunk partials, then one IEEE division by the count.
//   - INT4: symmetric, delta = amax/7, code = clamp(rint(x/delta), -7, 7) with
//     true division and round-half-to-even; amax == 0 gives delta = 0, code 0.
//     The adaptive alternative for Q and K ("adaptive quantization method",
//     technical-report summary, Key Contribution 3; 8-bit codes as in the
//     SageAttention v1 page) uses the same rule with 127 in place of 7.
//   - Adaptive width (qk_bits 0): the summary page names an "adaptive
//     quantization method" that keeps end-to-end metrics but does not define
//     it.  Reading: per key/value head (with its query heads), predict the
//     error INT4 adds to the softmax logits and fall back to INT8 where that
//     error would cost more than 0.01 of cosine similarity.  A code error is
//     modelled as uniform over +-delta/2 (variance delta^2/12, delta =
//     amax/7), so a logit q.k gains variance
//        sigma^2 = sm^2/12 * (amax_q^2/49 * |gK|^2 + amax_k^2/49 * |gQ|^2)
//     on average over queries and keys.  Logit noise sigma moves O by about
//     sigma * (spread of the V rows), so the cosine loss against unquantized
//     attention is at most ~ sigma^2/2 * rho with rho = E|V - vbar|^2 /
//     (E|V - vbar|^2 + |vbar|^2) (attention concentrated on one key).  INT4
//     iff sigma^2 * rho <= 0.02.  Statistics (fp32, fixed order):
//       A_Q = sum over query blocks (in order) of the block's sum, in token
//             order, of amax_i^2 (amax of the smoothed token);
//       E_Q = sum over query blocks of sum_c max(0, SSQ_c - SQ_c * qmean_c)
//             (SQ, SSQ: the block's sequential sums of Q and Q^2);
//       A_K = sum over 128-key blocks of the block's sum, in key order, of
//             amax_g(j)^2 (the key's scale group);
//       E_K = sum_c max(0, SSK_c - SK_c * kmean_c), EV likewise for V with
//             vbar_c = SV_c / Nk, V2 = sum_c SV_c * vbar_c (SK, SSK, SV, SSV:
//             chunked sums as for the means);
//     A_Q and E_Q summed over the group's query heads in head order.  Then in
//     fp64: INT4 iff sm^2 * (A_Q*E_K + A_K*E_Q) * EV <= 11.76 * (G*Nq) * Nk *
//     (EV + V2) (11.76 = 0.02 * 12 * 49; G query heads per K/V head).
//   - Q: one scale per token.  K: one scale per 16-key group; inside every
//     32-key tile, group h (0 or 1) holds the keys whose offset o satisfies
//     (o / 4) % 2 == h.  These are the keys that one half of a 64-lane wave holds
//     in a 32x32 matrix-core accumulator when the score tile is built as K*Q^T.
//   - Compensation term DeltaS[qb][j] = sum_c qmean[qb][c] * (K[j][c]-kmean[c]),
//     accumulated in fp64 and rounded once to fp32.
//   - V: FP8 OCP e4m3fn (max 448), one scale per channel = amax/448, RNE.
//     Optional V smoothing (technical-report summary, Key Contribution 2:
//     smoothing of Q and V): the per-channel mean of V over all N tokens
//     (same fp32 chunked order as the K mean) is subtracted before the FP8
//     quantization and added back to the output, which is exact for the
//     unquantized method because every row of softmax(S) sums to one.
//   - Scores in the log2 domain:  ks = sm_scale * log2(e) (fp32),
//     s2 = fma((float)acc, (dq*dk)*ks, DeltaS*ks).
//   - Online softmax over BK = 128-key blocks in ascending order.
//     mm = m_t - log2(448);  p' = exp2(s2 - mm) in [0, 448];  P8 = e4m3(p');
//     l' = alpha*l' + sum(dec(P8)): the row sum of the FP8 P~ that multiplies
//     V (the pages quantize P~ and say nothing of the normalizer; summing the
//     values that weight V keeps every output row a convex combination of the
//     dequantized V rows).  Without P~ quantization the sum is of p' itself.
//   - Two-level P~V: R_t = sum_j dec(P8_j)*dec(V8_j) in a fresh fp32 buffer per
//     block; O_t = fma(alpha_t, O_{t-1}, R_t).
//   - Epilogue: O = (O_T * vscale) / l'_T (+ vmean with V smoothing).
//
// Build: g++ -std=c++17 -O2 -ffp-contract=off -shared -fPIC -pthread
// (no fast-math, no FMA contraction; std::fma only where a step names fma).

#include <cmath>
#include <cstdint>
#include <cstring>
#include <thread>
#include <vector>
#include <algorithm>
#include <limits>
#include <functional>

namespace {

constexpr int ORACLE_CONTRACT = 2;
constexpr int BQ_MEAN = 128;   // tokens per Q-smoothing block and per mean chunk
constexpr int BK = 128;        // keys per online-softmax / two-level block
constexpr float LOG2E = 1.44269504088896340736f;
constexpr float LOG2_448 = 8.80735492205760410744f;

// ---------------------------------------------------------------- decoding ---
float f16_to_f32(uint16_t h) {
  int s = (h >> 15) & 1, e = (h >> 10) & 31, m = h & 1023;
  float v;
  if (e == 0) v = std::ldexp((float)m, -24);
  else if (e == 31) v = m ? std::numeric_limits<float>::quiet_NaN() : std::numeric_limits<float>::infinity();
  else v = std::ldexp((float)(1024 + m), e - 25);
  return s ? -v : v;
}
float bf16_to_f32(uint16_t b) {
  uint32_t u = (uint32_t)b << 16;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}
float in_to_f32(const uint16_t* p, int64_t idx, int dtype) {
  return dtype == 0 ? f16_to_f32(p[idx]) : bf16_to_f32(p[idx]);
}

// ------------------------------------------------------------ e4m3fn codec ---
// OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent (bias 7), 3 mantissa bits; no
// infinities; 0x7F / 0xFF are NaN; largest finite 448; subnormal step 2^-9.
// Encode: round to nearest, ties to even; magnitudes beyond 448 saturate.
uint8_t e4m3_encode(float x) {
  if (std::isnan(x)) return 0x7F;
  uint8_t sign = std::signbit(x) ? 0x80 : 0x00;
  float a = std::fabs(x);
  if (a >= 464.0f) return sign | 0x7E;            // beyond the 448 / 480 midpoint
  if (a < 0.015625f) {                             // below 2^-6: subnormal range
    float m = std::rint(a * 512.0f);               // exact scaling by 2^9, RNE
    return sign | (uint8_t)m;                      // m == 8 is the smallest normal
  }
  int e;
  std::frexp(a, &e);                               // a = f * 2^e, f in [0.5, 1)
  int ex = e - 1;                                  // a in [2^ex, 2^(ex+1))
  float r = std::rint(std::ldexp(a, 3 - ex));      // in [8, 16], RNE
  if (r == 16.0f) { r = 8.0f; ex += 1; }
  int code = ((ex + 7) << 3) | ((int)r - 8);
  if (code > 0x7E) code = 0x7E;
  return sign | (uint8_t)code;
}
float e4m3_decode(uint8_t b) {
  int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
  if (e == 15 && m == 7) return std::numeric_limits<float>::quiet_NaN();
  float v = (e == 0) ? std::ldexp((float)m, -9) : std::ldexp((float)(8 + m), e - 10);
  return s ? -v : v;
}

// ------------------------------------------------------------ quantization ---
// Symmetric integer code with maximum magnitude qmax (7 for INT4, 127 for INT8).
int8_t int_code(float x, float delta, float qmax) {
  if (delta == 0.0f) return 0;
  float r = std::rint(x / delta);
  if (r > qmax) r = qmax;
  if (r < -qmax) r = -qmax;
  return (int8_t)r;
}

// Group of key j: two 16-key groups per 32-key tile (see header comment).
int64_t k_group(int64_t j) { return 2 * (j / 32) + ((j % 32) / 4) % 2; }

void parallel_for(int64_t n, int nthreads, const std::function<void(int64_t)>& fn) {
  if (nthreads <= 1 || n <= 1) {
    for (int64_t i = 0; i < n; i++) fn(i);
    return;
  }
  int nt = (int)std::min<int64_t>(nthreads, n);
  std::vector<std::thread> th;
  for (int t = 0; t < nt; t++)
    th.emplace_back([&, t] {
      for (int64_t i = t; i < n; i += nt) fn(i);
    });
  for (auto& x : th) x.join();
}

}  // namespace

extern "C" {

int oracle_contract_version(void) { return ORACLE_CONTRACT; }
int oracle_bq_mean(void) { return BQ_MEAN; }
int oracle_bk(void) { return BK; }

void oracle_e4m3_encode(const float* x, uint8_t* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = e4m3_encode(x[i]);
}
void oracle_e4m3_decode(const uint8_t* in, float* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = e4m3_decode(in[i]);
}
void oracle_decode_input(const uint16_t* in, int dtype, float* out, int64_t n) {
  for (int64_t i = 0; i < n; i++) out[i] = in_to_f32(in, i, dtype);
}

// Geometry.  Queries: B batches x Hq heads x Nq tokens.  Keys and values:
// B x Hkv heads x Nk tokens, with Hq a multiple of Hkv; query head h reads
// key/value head h / (Hq / Hkv) (grouped-query attention; Hkv == Hq is plain
// multi-head attention, Nk != Nq is cross-attention or decoding against a
// key/value cache).  A causal mask is aligned at the bottom-right corner:
// query i may attend key j iff j <= i + (Nk - Nq), so the last query sees every
// key; causal calls require Nq <= Nk (every query then sees at least key 0).
//
// Prepass: smoothing statistics, INT4 codes and scales for Q and K, FP8 V with
// per-channel scales, and the rank-1 compensation term.  All arrays are in the
// canonical (unpacked, unpadded) layout:
//   q_codes          : int8  [B,Hq,Nq,D]    values in [-7, 7] (qk_bits 4) or [-127, 127] (8)
//   q_scale          : fp32  [B,Hq,Nq]
//   q_mean           : fp32  [B,Hq,ceil(Nq/128),D]
//   k_codes          : int8  [B,Hkv,Nk,D]
//   k_scale          : fp32  [B,Hkv,2*ceil(Nk/32)]
//   k_mean           : fp32  [B,Hkv,D]
//   v_codes          : uint8 [B,Hkv,Nk,D]   e4m3fn bit patterns of (V - vmean)/vscale
//   v_scale          : fp32  [B,Hkv,D]
//   v_mean           : fp32  [B,Hkv,D]      per-channel V mean (zeros without smoothing)
//   delta_s          : fp32  [B,Hq,ceil(Nq/128),Nk]  (query head h against its K head)
// Returns 0, or -1 for invalid arguments.
// qk_bits 4 or 8 for every head, or 0: the width of K/V head bhk (and of its
// query heads) is head_bits[bhk] (4 or 8), as chosen by oracle_adaptive_bits.
int oracle_quant_smooth(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                        int B, int Hq, int Hkv, int Nq, int Nk, int D, int qk_bits, int smooth_v,
                        const int32_t* head_bits,
                        int8_t* q_codes, float* q_scale, int8_t* k_codes, float* k_scale,
                        float* q_mean, float* k_mean, uint8_t* v_codes, float* v_scale, float* v_mean,
                        float* delta_s, int nthreads) {
  if (!q || !k || !v || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Nq < 1 || Nk < 1 || D < 1) return -1;
  if (dtype != 0 && dtype != 1) return -1;
  if (qk_bits != 4 && qk_bits != 8 && qk_bits != 0) return -1;
  if (qk_bits == 0) {
    if (!head_bits) return -1;
    for (int64_t i = 0; i < (int64_t)B * Hkv; i++)
      if (head_bits[i] != 4 && head_bits[i] != 8) return -1;
  }
  if (smooth_v != 0 && smooth_v != 1) return -1;
  // the largest code of K/V head bhk and of its query heads
  auto qmax_of = [&](int64_t bhk) {
    const int bits = qk_bits ? qk_bits : head_bits[bhk];
    return bits == 4 ? 7.0f : 127.0f;
  };
  const int64_t NQB = (Nq + BQ_MEAN - 1) / BQ_MEAN;
  const int64_t G = 2 * ((int64_t)(Nk + 31) / 32);
  const int group = Hq / Hkv;
  // ---- key/value side, one (batch, K/V head) at a time.  The smoothed keys
  // gK are kept for the compensation term of every query head of the group.
  std::vector<std::vector<float>> gK_all((size_t)B * Hkv);
  parallel_for((int64_t)B * Hkv, nthreads, [&](int64_t bhk) {
    const int64_t base = bhk * (int64_t)Nk * D;
    const float qmax = qmax_of(bhk);
    std::vector<float> K((size_t)Nk * D), V((size_t)Nk * D);
    for (int64_t i = 0; i < (int64_t)Nk * D; i++) {
      K[i] = in_to_f32(k, base + i, dtype);
      V[i] = in_to_f32(v, base + i, dtype);
    }
    // K channel mean over all Nk tokens: chunk partials, then their sum.
    std::vector<float> kbar(D);
    for (int c = 0; c < D; c++) {
      float total = 0.0f;
      for (int64_t t0 = 0; t0 < Nk; t0 += BQ_MEAN) {
        float part = 0.0f;
        for (int64_t j = t0; j < std::min<int64_t>(Nk, t0 + BQ_MEAN); j++) part = part + K[j * D + c];
        total = total + part;
      }
      kbar[c] = total / (float)Nk;
      if (k_mean) k_mean[bhk * D + c] = kbar[c];
    }
    std::vector<float>& gK = gK_all[bhk];
    gK.resize((size_t)Nk * D);
    for (int64_t j = 0; j < Nk; j++)
      for (int c = 0; c < D; c++) gK[j * D + c] = K[j * D + c] - kbar[c];
    // K: one scale per 16-key fragment group
    std::vector<float> gamax(G, 0.0f);
    for (int64_t j = 0; j < Nk; j++) {
      int64_t g = k_group(j);
      for (int c = 0; c < D; c++) gamax[g] = std::max(gamax[g], std::fabs(gK[j * D + c]));
    }
    std::vector<float> dk(G);
    for (int64_t g = 0; g < G; g++) {
      dk[g] = gamax[g] / qmax;
      if (k_scale) k_scale[bhk * G + g] = dk[g];
    }
    if (k_codes)
      for (int64_t j = 0; j < Nk; j++)
        for (int c = 0; c < D; c++) k_codes[base + j * D + c] = int_code(gK[j * D + c], dk[k_group(j)], qmax);
    // V: optional smoothing, then FP8 e4m3fn with one scale per channel
    for (int c = 0; c < D; c++) {
      float vbar = 0.0f;
      if (smooth_v) {
        float total = 0.0f;
        for (int64_t t0 = 0; t0 < Nk; t0 += BQ_MEAN) {
          float part = 0.0f;
          for (int64_t j = t0; j < std::min<int64_t>(Nk, t0 + BQ_MEAN); j++) part = part + V[j * D + c];
          total = total + part;
        }
        vbar = total / (float)Nk;
        for (int64_t j = 0; j < Nk; j++) V[j * D + c] = V[j * D + c] - vbar;
      }
      if (v_mean) v_mean[bhk * D + c] = vbar;
      float amax = 0.0f;
      for (int64_t j = 0; j < Nk; j++) amax = std::max(amax, std::fabs(V[j * D + c]));
      float dv = amax / 448.0f;
      if (v_scale) v_scale[bhk * D + c] = dv;
      if (v_codes)
        for (int64_t j = 0; j < Nk; j++)
          v_codes[base + j * D + c] = (dv == 0.0f) ? (uint8_t)0 : e4m3_encode(V[j * D + c] / dv);
    }
  });
  // ---- query side, one (batch, query head) at a time.
  parallel_for((int64_t)B * Hq, nthreads, [&](int64_t bhq) {
    const int64_t base = bhq * (int64_t)Nq * D;
    const int64_t bhk = (bhq / Hq) * Hkv + (bhq % Hq) / group;
    const std::vector<float>& gK = gK_all[bhk];
    const float qmax = qmax_of(bhk);
    std::vector<float> Q((size_t)Nq * D);
    for (int64_t i = 0; i < (int64_t)Nq * D; i++) Q[i] = in_to_f32(q, base + i, dtype);
    // Q block means (128-token blocks, partial tail block).
    std::vector<float> qbar((size_t)NQB * D);
    for (int64_t qb = 0; qb < NQB; qb++) {
      int64_t i0 = qb * BQ_MEAN, i1 = std::min<int64_t>(Nq, i0 + BQ_MEAN);
      for (int c = 0; c < D; c++) {
        float s = 0.0f;
        for (int64_t i = i0; i < i1; i++) s = s + Q[i * D + c];
        qbar[qb * D + c] = s / (float)(i1 - i0);
        if (q_mean) q_mean[(bhq * NQB + qb) * D + c] = qbar[qb * D + c];
      }
    }
    // Q: one scale per token, on the smoothed values
    std::vector<float> gQ(D);
    for (int64_t i = 0; i < Nq; i++) {
      for (int c = 0; c < D; c++) gQ[c] = Q[i * D + c] - qbar[(i / BQ_MEAN) * D + c];
      float amax = 0.0f;
      for (int c = 0; c < D; c++) amax = std::max(amax, std::fabs(gQ[c]));
      float dq = amax / qmax;
      if (q_scale) q_scale[bhq * Nq + i] = dq;
      if (q_codes)
        for (int c = 0; c < D; c++) q_codes[base + i * D + c] = int_code(gQ[c], dq, qmax);
    }
    // rank-1 compensation: DeltaS[qb][j] = qbar[qb] . gK[j]
    if (delta_s)
      for (int64_t qb = 0; qb < NQB; qb++)
        for (int64_t j = 0; j < Nk; j++) {
          double acc = 0.0;
          for (int c = 0; c < D; c++) acc += (double)qbar[qb * D + c] * (double)gK[j * D + c];
          delta_s[(bhq * NQB + qb) * Nk + j] = (float)acc;
        }
  });
  return 0;
}

// Adaptive width (header comment): the statistics and the choice for every
// key/value head.  head_bits[B*Hkv] receives 4 or 8; stats (optional)
// [B*Hkv][6] receives the group totals A_Q, E_Q, A_K, E_K, EV, V2.
int oracle_adaptive_bits(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype, int B, int Hq, int Hkv,
                         int Nq, int Nk, int D, float sm_scale, int32_t* head_bits, float* stats, int nthreads) {
  if (!q || !k || !v || !head_bits || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Nq < 1 || Nk < 1 || D < 1) return -1;
  if (dtype != 0 && dtype != 1) return -1;
  if (!(sm_scale > 0.0f) || !std::isfinite(sm_scale)) return -1;
  const int group = Hq / Hkv;
  // query side: A_Q and E_Q of every query head
  std::vector<float> AQ((size_t)B * Hq), EQ((size_t)B * Hq);
  parallel_for((int64_t)B * Hq, nthreads, [&](int64_t bhq) {
    const int64_t base = bhq * (int64_t)Nq * D;
    float a_tot = 0.0f, e_tot = 0.0f;
    for (int64_t i0 = 0; i0 < Nq; i0 += BQ_MEAN) {
      const int64_t i1 = std::min<int64_t>(Nq, i0 + BQ_MEAN);
      std::vector<float> mean(D);
      float e_blk = 0.0f;
      for (int c = 0; c < D; c++) {
        float sq = 0.0f, ssq = 0.0f;
        for (int64_t i = i0; i < i1; i++) {
          const float x = in_to_f32(q, base + i * D + c, dtype);
          sq = sq + x;
          ssq = ssq + x * x;
        }
        mean[c] = sq / (float)(i1 - i0);
        e_blk = e_blk + std::max(ssq - sq * mean[c], 0.0f);
      }
      float a_blk = 0.0f;
      for (int64_t i = i0; i < i1; i++) {
        float amax = 0.0f;
        for (int c = 0; c < D; c++) amax = std::max(amax, std::fabs(in_to_f32(q, base + i * D + c, dtype) - mean[c]));
        a_blk = a_blk + amax * amax;
      }
      a_tot = a_tot + a_blk;
      e_tot = e_tot + e_blk;
    }
    AQ[bhq] = a_tot;
    EQ[bhq] = e_tot;
  });
  // key/value side and the choice
  parallel_for((int64_t)B * Hkv, nthreads, [&](int64_t bhk) {
    const int64_t base = bhk * (int64_t)Nk * D;
    std::vector<float> kbar(D);
    float EK = 0.0f, EV = 0.0f, V2 = 0.0f;
    for (int c = 0; c < D; c++) {
      float sk = 0.0f, ssk = 0.0f, sv = 0.0f, ssv = 0.0f;
      for (int64_t t0 = 0; t0 < Nk; t0 += BQ_MEAN) {
        float pk = 0.0f, pkk = 0.0f, pv = 0.0f, pvv = 0.0f;
        for (int64_t j = t0; j < std::min<int64_t>(Nk, t0 + BQ_MEAN); j++) {
          const float xk = in_to_f32(k, base + j * D + c, dtype), xv = in_to_f32(v, base + j * D + c, dtype);
          pk = pk + xk;
          pkk = pkk + xk * xk;
          pv = pv + xv;
          pvv = pvv + xv * xv;
        }
        sk = sk + pk;
        ssk = ssk + pkk;
        sv = sv + pv;
        ssv = ssv + pvv;
      }
      kbar[c] = sk / (float)Nk;
      const float vbar = sv / (float)Nk;
      EK = EK + std::max(ssk - sk * kbar[c], 0.0f);
      EV = EV + std::max(ssv - sv * vbar, 0.0f);
      V2 = V2 + sv * vbar;
    }
    // per-group amax of the smoothed keys
    const int64_t G = 2 * ((int64_t)(Nk + 31) / 32);
    std::vector<float> gamax(G, 0.0f);
    for (int64_t j = 0; j < Nk; j++)
      for (int c = 0; c < D; c++)
        gamax[k_group(j)] = std::max(gamax[k_group(j)], std::fabs(in_to_f32(k, base + j * D + c, dtype) - kbar[c]));
    float AK = 0.0f;
    for (int64_t j0 = 0; j0 < Nk; j0 += BK) {
      float part = 0.0f;
      for (int64_t j = j0; j < std::min<int64_t>(Nk, j0 + BK); j++) part = part + gamax[k_group(j)] * gamax[k_group(j)];
      AK = AK + part;
    }
    float AQg = 0.0f, EQg = 0.0f;
    const int64_t b = bhk / Hkv, hk = bhk % Hkv;
    for (int g = 0; g < group; g++) {
      AQg = AQg + AQ[b * Hq + hk * group + g];
      EQg = EQg + EQ[b * Hq + hk * group + g];
    }
    const double sm = (double)sm_scale;
    const double num = (sm * sm) * ((double)AQg * (double)EK + (double)AK * (double)EQg) * (double)EV;
    const double den = 11.76 * ((double)group * (double)Nq * (double)Nk) * ((double)EV + (double)V2);
    head_bits[bhk] = num <= den ? 4 : 8;
    if (stats) {
      float* st = stats + bhk * 6;
      st[0] = AQg;
      st[1] = EQg;
      st[2] = AK;
      st[3] = EK;
      st[4] = EV;
      st[5] = V2;
    }
  });
  return 0;
}

// Exact integer dot products of INT4 codes for one head:
// out[a][b] = sum_c qc[(q0+a)*D + c] * kc[(k0+b)*D + c].
int oracle_qk_int32(const int8_t* qc, const int8_t* kc, int D, int q0, int k0, int nq, int nk, int32_t* out) {
  if (!qc || !kc || !out || D < 1 || nq < 0 || nk < 0) return -1;
  for (int a = 0; a < nq; a++)
    for (int b = 0; b < nk; b++) {
      int64_t acc = 0;
      for (int c = 0; c < D; c++) acc += (int64_t)qc[(int64_t)(q0 + a) * D + c] * kc[(int64_t)(k0 + b) * D + c];
      out[(int64_t)a * nk + b] = (int32_t)acc;
    }
  return 0;
}

// Flags for the mirror mode.
//   1: quantize P~ to FP8 (the method).  Without it, p' itself (fp32) is used.
enum { MIRROR_QUANT_P = 1 };

// Mirror mode: the method step by step, in the same fp32 operations the GPU
// path performs, for a list of query rows.  rows[r] = (b*Hq + h)*Nq + i.
// Inputs are the canonical prepass arrays (geometry as for the prepass).
// Outputs: O[r][c] (fp32) and, per row, slack[r]: an upper bound on how far O
// may move if any P~ element whose value p' lies within relative distance eps
// of an FP8 rounding midpoint were rounded the other way (a diagnostic of exp2
// implementation differences): per such element step * (max|v_j| + 448 *
// max vscale) / l', weighted like the element.  Optional lse[r] = (final running max m, final
// l') for diagnostics.
//
// kv_split (0: none): keys are cut into consecutive ranges of kv_split keys (a
// multiple of the 128-key block).  Each range runs the online softmax of the
// method on its own, from an empty state (its own running max, so its P~
// values are scaled to its own maximum before the FP8 rounding); the ranges
// are then merged in order with fp32 weights w_s = exp2(m_s - M), M the
// largest range maximum:  O = fma(w_s, O_s, O), l' = fma(w_s, l'_s, l').
// Ranges holding no visible key are skipped.  One range is the plain
// schedule, bit for bit.  (The pages fix the block-wise online softmax and
// the per-block FP8 P~ but not the order in which key blocks are visited;
// this is the schedule a split-key kernel uses.)
int oracle_attn_mirror(const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                       const uint8_t* v_codes, const float* v_scale, const float* v_mean, const float* delta_s,
                       int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, float sm_scale, int flags,
                       int kv_split, const int64_t* rows, int64_t nrows, float eps,
                       float* O, float* slack, float* lse, int nthreads) {
  if (!q_codes || !q_scale || !k_codes || !k_scale || !v_codes || !v_scale || !delta_s || !O) return -1;
  if (B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Nq < 1 || Nk < 1 || D < 1 || !(sm_scale > 0.0f)) return -1;
  if (causal && Nq > Nk) return -1;
  if (kv_split < 0 || kv_split % BK) return -1;
  const int64_t NQB = (Nq + BQ_MEAN - 1) / BQ_MEAN;
  const int64_t G = 2 * ((int64_t)(Nk + 31) / 32);
  const int group = Hq / Hkv;
  const float ks = sm_scale * LOG2E;
  const int64_t span = kv_split ? kv_split : Nk;
  const int64_t total = rows ? nrows : (int64_t)B * Hq * Nq;
  parallel_for(total, nthreads, [&](int64_t r) {
    const int64_t flat = rows ? rows[r] : r;
    const int64_t bhq = flat / Nq, i = flat % Nq;
    const int64_t bhk = (bhq / Hq) * Hkv + (bhq % Hq) / group;
    const int8_t* qi = q_codes + flat * D;
    const int8_t* kh = k_codes + bhk * (int64_t)Nk * D;
    const uint8_t* vh = v_codes + bhk * (int64_t)Nk * D;
    const float* ds = delta_s + (bhq * NQB + i / BQ_MEAN) * Nk;
    const float* dvec = v_scale + bhk * D;
    float vbound = 0.0f;   // bound on |O| before V smoothing: every |dec(V8) * vscale| <= 448 * vscale
    for (int c = 0; c < D; c++) vbound = std::max(vbound, 448.0f * dvec[c]);
    const float dq = q_scale[flat];
    const int64_t jend = causal ? i + 1 + (Nk - Nq) : Nk;  // keys j < jend are allowed
    // per-range states, merged below
    std::vector<std::vector<float>> Os;
    std::vector<float> ms, ls, slks;
    std::vector<float> R(D), s2(BK), p(BK);
    for (int64_t r0 = 0; r0 < jend; r0 += span) {
      const int64_t r1 = std::min<int64_t>(r0 + span, Nk);
      std::vector<float> Orun(D, 0.0f);
      float m = -std::numeric_limits<float>::infinity();
      float l = 0.0f, slk = 0.0f;
      for (int64_t t0 = r0; t0 < std::min(r1, jend); t0 += BK) {
        const int64_t t1 = std::min<int64_t>(t0 + BK, r1);
        // scores in the log2 domain
        float bmax = -std::numeric_limits<float>::infinity();
        for (int64_t j = t0; j < t1; j++) {
          float& s = s2[j - t0];
          if (j >= jend) { s = -std::numeric_limits<float>::infinity(); continue; }
          int32_t acc = 0;
          for (int c = 0; c < D; c++) acc += (int32_t)qi[c] * (int32_t)kh[j * D + c];
          float cfac = (dq * k_scale[bhk * G + k_group(j)]) * ks;
          float d = ds[j] * ks;
          s = std::fma((float)acc, cfac, d);
          bmax = std::max(bmax, s);
        }
        const float mnew = std::max(m, bmax);
        const float alpha = std::exp2(m - mnew);
        const float mm = mnew - LOG2_448;
        float rowsum = 0.0f;
        for (int64_t j = t0; j < t1; j++) {
          float pj = (j < jend) ? std::exp2(s2[j - t0] - mm) : 0.0f;
          p[j - t0] = pj;
          rowsum = rowsum + ((flags & MIRROR_QUANT_P) ? e4m3_decode(e4m3_encode(pj)) : pj);
        }
        // P~ -> FP8 and the level-1 partial R_t in a fresh fp32 buffer
        std::fill(R.begin(), R.end(), 0.0f);
        float blk_slack = 0.0f;
        for (int64_t j = t0; j < t1; j++) {
          float pj = p[j - t0];
          float pq = (flags & MIRROR_QUANT_P) ? e4m3_decode(e4m3_encode(pj)) : pj;
          if (pq == 0.0f && pj == 0.0f) continue;
          for (int c = 0; c < D; c++) R[c] = R[c] + pq * e4m3_decode(vh[j * D + c]);
          if ((flags & MIRROR_QUANT_P) && eps > 0.0f && pj > 0.0f) {
            // Is a rounding midpoint of the FP8 grid within relative eps of pj?
            float lo = pj * (1.0f - eps), hi = pj * (1.0f + eps);
            uint8_t clo = e4m3_encode(lo), chi = e4m3_encode(hi);
            if (clo != chi) {
              // the flip moves the numerator by step * v_j and l' by step, so
              // O by step * (v_j - O) / l': bounded with |O| <= 448 * max vscale
              float step = std::fabs(e4m3_decode(chi) - e4m3_decode(clo));
              float vm = 0.0f;
              for (int c = 0; c < D; c++) vm = std::max(vm, std::fabs(e4m3_decode(vh[j * D + c]) * dvec[c]));
              blk_slack += step * (vm + vbound);
            }
          }
        }
        // level 2: fold the block into the fp32 running buffer
        for (int c = 0; c < D; c++) Orun[c] = std::fma(alpha, Orun[c], R[c]);
        l = alpha * l + rowsum;
        slk = alpha * slk + blk_slack;
        m = mnew;
      }
      Os.push_back(Orun);
      ms.push_back(m);
      ls.push_back(l);
      slks.push_back(slk);
    }
    // merge the ranges (a single range passes through unchanged: w = 1)
    float M = -std::numeric_limits<float>::infinity();
    for (float m : ms) M = std::max(M, m);
    std::vector<float> Ofin(D, 0.0f);
    float l = 0.0f, slk = 0.0f;
    for (size_t sidx = 0; sidx < ms.size(); sidx++) {
      const float w = std::exp2(ms[sidx] - M);
      for (int c = 0; c < D; c++) Ofin[c] = std::fma(w, Os[sidx][c], Ofin[c]);
      l = std::fma(w, ls[sidx], l);
      slk = std::fma(w, slks[sidx], slk);
    }
    for (int c = 0; c < D; c++) {
      O[r * D + c] = (Ofin[c] * dvec[c]) / l;
      if (v_mean) O[r * D + c] = O[r * D + c] + v_mean[bhk * D + c];
    }
    if (slack) slack[r] = slk / l;
    if (lse) { lse[2 * r] = M; lse[2 * r + 1] = l; }
  });
  return 0;
}

// Exact mode: softmax(S) V in fp64 with a direct (not online) softmax, for a
// list of rows.  Flags select which parts of the method are applied:
enum {
  EXACT_SMOOTH_K = 1,  // subtract the per-channel K mean (fp64 mean)
  EXACT_SMOOTH_Q = 2,  // subtract the per-block Q mean and add q_mean . gamma(K)
  EXACT_QUANT_QK = 4,  // use the prepass INT4 codes/scales and DeltaS (given)
  EXACT_QUANT_V = 8,   // use the prepass FP8 V and scales (given), plus v_mean if given
  EXACT_SMOOTH_V = 16, // without QUANT_V: subtract the fp64 per-channel V mean, add it back to O
};
// Without EXACT_QUANT_QK the scores are built from the raw inputs in fp64:
//   S_ij = sm_scale * ( gQ_i . gK_j + [SMOOTH_Q] qmean_qb(i) . gK_j )
// With EXACT_QUANT_QK they are built from the canonical prepass arrays:
//   S_ij = sm_scale * ( (dq_i * qc_i) . (dk_g(j) * kc_j) + DeltaS[qb(i)][j] )
// Geometry, head mapping and causal alignment as for the prepass; rows[r] =
// (b*Hq + h)*Nq + i.  Outputs O[r][c] in fp64; optional P row sums in psum[r].
int oracle_attn_exact(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                      const int8_t* q_codes, const float* q_scale, const int8_t* k_codes, const float* k_scale,
                      const uint8_t* v_codes, const float* v_scale, const float* v_mean, const float* delta_s,
                      int B, int Hq, int Hkv, int Nq, int Nk, int D, int causal, double sm_scale, int flags,
                      const int64_t* rows, int64_t nrows, double* O, double* psum, int nthreads) {
  if (!q || !k || !v || !O || B < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv || Nq < 1 || Nk < 1 || D < 1) return -1;
  if (dtype != 0 && dtype != 1) return -1;
  if (causal && Nq > Nk) return -1;
  if ((flags & EXACT_QUANT_QK) && (!q_codes || !q_scale || !k_codes || !k_scale || !delta_s)) return -1;
  if ((flags & EXACT_QUANT_V) && (!v_codes || !v_scale)) return -1;
  const int64_t NQB = (Nq + BQ_MEAN - 1) / BQ_MEAN;
  const int64_t G = 2 * ((int64_t)(Nk + 31) / 32);
  const int group = Hq / Hkv;
  const int64_t total = rows ? nrows : (int64_t)B * Hq * Nq;
  // fp64 statistics: query-block means per query head, K and V channel means
  // per K/V head; computed only for the heads the requested rows touch.
  const int64_t nq_heads = (int64_t)B * Hq, nk_heads = (int64_t)B * Hkv;
  auto kv_head = [&](int64_t bhq) { return (bhq / Hq) * Hkv + (bhq % Hq) / group; };
  std::vector<std::vector<double>> kbar(nk_heads), vbar(nk_heads), qbar(nq_heads);
  std::vector<char> need_q(nq_heads, rows ? 0 : 1), need_k(nk_heads, rows ? 0 : 1);
  if (rows)
    for (int64_t r = 0; r < nrows; r++) {
      need_q[rows[r] / Nq] = 1;
      need_k[kv_head(rows[r] / Nq)] = 1;
    }
  parallel_for(nk_heads, nthreads, [&](int64_t bhk) {
    if (!need_k[bhk]) return;
    const int64_t base = bhk * (int64_t)Nk * D;
    kbar[bhk].assign(D, 0.0);
    vbar[bhk].assign(D, 0.0);
    if ((flags & EXACT_SMOOTH_V) && !(flags & EXACT_QUANT_V))
      for (int c = 0; c < D; c++) {
        double s = 0.0;
        for (int64_t j = 0; j < Nk; j++) s += in_to_f32(v, base + j * D + c, dtype);
        vbar[bhk][c] = s / Nk;
      }
    if (flags & EXACT_SMOOTH_K)
      for (int c = 0; c < D; c++) {
        double s = 0.0;
        for (int64_t j = 0; j < Nk; j++) s += in_to_f32(k, base + j * D + c, dtype);
        kbar[bhk][c] = s / Nk;
      }
  });
  parallel_for(nq_heads, nthreads, [&](int64_t bhq) {
    if (!need_q[bhq]) return;
    const int64_t base = bhq * (int64_t)Nq * D;
    qbar[bhq].assign(NQB * D, 0.0);
    if (flags & EXACT_SMOOTH_Q)
      for (int64_t qb = 0; qb < NQB; qb++) {
        int64_t i0 = qb * BQ_MEAN, i1 = std::min<int64_t>(Nq, i0 + BQ_MEAN);
        for (int c = 0; c < D; c++) {
          double s = 0.0;
          for (int64_t i = i0; i < i1; i++) s += in_to_f32(q, base + i * D + c, dtype);
          qbar[bhq][qb * D + c] = s / (double)(i1 - i0);
        }
      }
  });
  parallel_for(total, nthreads, [&](int64_t r) {
    const int64_t flat = rows ? rows[r] : r;
    const int64_t bhq = flat / Nq, i = flat % Nq, qb = i / BQ_MEAN;
    const int64_t bhk = kv_head(bhq);
    const int64_t qbase = bhq * (int64_t)Nq * D, kbase = bhk * (int64_t)Nk * D;
    const int64_t jend = causal ? i + 1 + (Nk - Nq) : Nk;
    std::vector<double> S(jend);
    std::vector<double> qrow(D), qm(D);
    for (int c = 0; c < D; c++) {
      if (flags & EXACT_QUANT_QK) {
        qrow[c] = (double)q_scale[flat] * (double)q_codes[flat * D + c];
      } else {
        double x = in_to_f32(q, qbase + i * D + c, dtype);
        qm[c] = (flags & EXACT_SMOOTH_Q) ? qbar[bhq][qb * D + c] : 0.0;
        qrow[c] = x - qm[c];
      }
    }
    for (int64_t j = 0; j < jend; j++) {
      double s = 0.0;
      if (flags & EXACT_QUANT_QK) {
        double dk = k_scale[bhk * G + k_group(j)];
        for (int c = 0; c < D; c++) s += qrow[c] * (dk * (double)k_codes[kbase + j * D + c]);
        s += (double)delta_s[(bhq * NQB + qb) * Nk + j];
      } else {
        double comp = 0.0;
        for (int c = 0; c < D; c++) {
          double kj = (double)in_to_f32(k, kbase + j * D + c, dtype) - kbar[bhk][c];
          s += qrow[c] * kj;
          comp += qm[c] * kj;
        }
        s += comp;
      }
      S[j] = sm_scale * s;
    }
    double mx = -std::numeric_limits<double>::infinity();
    for (int64_t j = 0; j < jend; j++) mx = std::max(mx, S[j]);
    double denom = 0.0;
    for (int64_t j = 0; j < jend; j++) { S[j] = std::exp(S[j] - mx); denom += S[j]; }
    double ps = 0.0;
    for (int c = 0; c < D; c++) O[r * D + c] = 0.0;
    for (int64_t j = 0; j < jend; j++) {
      double pj = S[j] / denom;
      ps += pj;
      for (int c = 0; c < D; c++) {
        double vj = (flags & EXACT_QUANT_V) ? (double)v_scale[bhk * D + c] * (double)e4m3_decode(v_codes[kbase + j * D + c])
                                            : (double)in_to_f32(v, kbase + j * D + c, dtype) - vbar[bhk][c];
        O[r * D + c] += pj * vj;
      }
    }
    for (int c = 0; c < D; c++) {
      if (flags & EXACT_QUANT_V) O[r * D + c] += v_mean ? (double)v_mean[bhk * D + c] : 0.0;
      else O[r * D + c] += vbar[bhk][c];
    }
    if (psum) psum[r] = ps;
  });
  return 0;
}

}  // extern "C"
