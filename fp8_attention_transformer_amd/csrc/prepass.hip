// SageAttention2 prepass on gfx950: smoothing statistics, INT4 Q/K codes with
// fine-grained scales, FP8 V with per-channel scales, compensation term.
//
// Method: SageAttention2 abstract (arXiv 2411.10958 page) -- Q,K to INT4 at a
// thread-level granularity, V to FP8, smoothing of Q; the title's "thorough
// outlier smoothing" is read as also removing the per-channel K mean.  The
// readings taken where the pages are silent (block sizes, scale groups, mean
// order, rounding) are the contract constants of sage_internal.h.
//
// All kernels here are HBM-bound except the compensation term (matrix-core
// dot products); they are launched in order on the caller's stream:
//   stats -> finalize -> quant -> delta_s.
// The statistics cover the key/value side (the Q block means come from the
// quant step, which holds each block anyway); the quant step runs once for
// the query side and once for the key/value side, except for packed
// sequences, where one workgroup handles a token block of Q, K and V.
#include "sage_internal.h"
#include "sage_device.h"

#include <type_traits>

namespace sage {
namespace {

// Which inputs a prepass workgroup handles: the query side, the key/value
// side, or both (packed self-attention, where a token block of Q, K and V is
// one work item); kPartV: the V statistics alone (a decoding step, whose
// scores need no K mean).
enum Part { kPartQ = 1, kPartKV = 2, kPartBoth = 3, kPartV = 4 };

// Workgroup barrier for LDS written with ds_write: waits for this wave's LDS
// operations only, so vector-memory loads and stores (including copies into
// LDS that nothing reads yet) stay in flight across it; __syncthreads()
// would wait for those too.  The memory clobber keeps the compiler from
// moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// ---------------------------------------------------------------------------
// stats: 256 threads, one channel pair per thread, 256/(D/2) chunks of 128
// tokens per workgroup.  Each thread walks its chunk in token order (the sums
// are sequential per channel); loads are issued 32 tokens ahead.  Per chunk:
// the K and V sums and the V maxima and minima (kPartV: V only).  The Q block
// means are formed by the quant kernel, which holds the block anyway.
// M2 (adaptive width): also the per-chunk sums of squares of K and V, in the
// same token order, for the width statistics.
template <int IN, int D, int PART, bool M2>
__global__ void __launch_bounds__(256) stats_kernel(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
                                                    Dims d, Bufs b) {
  constexpr int LPC = D / 2;          // lanes per chunk
  constexpr int CPW = 256 / LPC;      // chunks per workgroup
  constexpr int U = 32;               // tokens in flight
  constexpr bool DO_K = PART == kPartKV;
  static_assert(PART == kPartKV || PART == kPartV, "stats cover the key/value side");
  const int tid = threadIdx.x, cp = tid % LPC;
  const int chunk = blockIdx.x * CPW + tid / LPC;
  const int nh = d.BHk(), nb = d.NQBk;
  if (chunk >= nh * nb) return;
  // dense: the chunks of a head are adjacent; packed [T, H, D]: the heads of a
  // token block are adjacent, so neighbouring workgroups read whole rows
  const int bh = d.cu ? chunk % nh : chunk / nb, qb = d.cu ? chunk / nh : chunk % nb;
  const HeadIO io = head_io_kv(d, bh);
  const int i0 = qb * kBQ, i1 = min(io.n, i0 + kBQ);   // i1 <= i0: empty chunk (short sequence)
  const size_t base = io.base + 2 * cp, rs = io.stride;
  float ks0 = 0.0f, ks1 = 0.0f, vs0 = 0.0f, vs1 = 0.0f;
  float vx0 = -__builtin_inff(), vx1 = -__builtin_inff(), vn0 = __builtin_inff(), vn1 = __builtin_inff();
  float kq0 = 0.0f, kq1 = 0.0f, vq0 = 0.0f, vq1 = 0.0f;   // sums of squares (M2)
  auto add = [&](uint32_t kv, uint32_t vv) {
    if constexpr (DO_K) {
      const float k0 = in_to_f32<IN>((uint16_t)(kv & 0xFFFF)), k1 = in_to_f32<IN>((uint16_t)(kv >> 16));
      ks0 = ks0 + k0;
      ks1 = ks1 + k1;
      if constexpr (M2) {
        kq0 = kq0 + k0 * k0;
        kq1 = kq1 + k1 * k1;
      }
    }
    const float v0 = in_to_f32<IN>((uint16_t)(vv & 0xFFFF)), v1 = in_to_f32<IN>((uint16_t)(vv >> 16));
    vs0 = vs0 + v0;
    vs1 = vs1 + v1;
    if constexpr (M2) {
      vq0 = vq0 + v0 * v0;
      vq1 = vq1 + v1 * v1;
    }
    vx0 = fmaxf(vx0, v0);
    vx1 = fmaxf(vx1, v1);
    vn0 = fminf(vn0, v0);
    vn1 = fminf(vn1, v1);
  };
  if (i1 - i0 == kBQ) {
    // full chunk: branch-free, U tokens of loads in flight
    for (int i = i0; i < i1; i += U) {
      uint32_t kv[U], vv[U];
#pragma unroll
      for (int u = 0; u < U; u++) {
        const size_t o = base + (size_t)(i + u) * rs;
        kv[u] = DO_K ? *(const uint32_t*)(k + o) : 0u;
        vv[u] = *(const uint32_t*)(v + o);
      }
#pragma unroll
      for (int u = 0; u < U; u++) add(kv[u], vv[u]);
    }
  } else {
    for (int i = i0; i < i1; i++) {
      const size_t o = base + (size_t)i * rs;
      add(DO_K ? *(const uint32_t*)(k + o) : 0u, *(const uint32_t*)(v + o));
    }
  }
  const size_t o2 = ((size_t)bh * d.NQBk + qb) * 2 * D + 2 * cp;
  b.k_part[o2] = ks0;
  b.k_part[o2 + 1] = ks1;
  b.k_part[o2 + D] = vs0;
  b.k_part[o2 + D + 1] = vs1;
  b.v_part[o2] = vx0;
  b.v_part[o2 + 1] = vx1;
  b.v_part[o2 + D] = vn0;
  b.v_part[o2 + D + 1] = vn1;
  if constexpr (M2) {
    b.m2_part[o2] = kq0;
    b.m2_part[o2 + 1] = kq1;
    b.m2_part[o2 + D] = vq0;
    b.m2_part[o2 + D + 1] = vq1;
  }
}

// acc + src[0] + src[1] + ... + src[n-1], added in index order by one thread,
// 16 values loaded per batch (the loads do not wait for the additions).
__device__ __forceinline__ float lds_ordered_sum(const float* src, int n, float acc = 0.0f) {
  int i = 0;
  for (; i + 16 <= n; i += 16) {
    float x[16];
#pragma unroll
    for (int u = 0; u < 16; u++) x[u] = src[i + u];
#pragma unroll
    for (int u = 0; u < 16; u++) acc = acc + x[u];
  }
  for (; i < n; i++) acc = acc + src[i];
  return acc;
}

// ---------------------------------------------------------------------------
// finalize: grid (B*Hk), D threads.  K mean = (sum of chunk sums, in chunk
// order) / Nk; likewise the V mean when V is smoothed (else 0).  V scale =
// max|V - vmean| / 448, from the chunk maxima and minima: rounding is
// monotonic, so max_j |fl(V_j - m)| = max(|fl(max V - m)|, |fl(min V - m)|).
// AD (adaptive width): also the channel's sums of squares of K and V (chunk
// partials in the same order), its centred sums of squares
// max(0, SS - S * mean) and V mean term S * mean (the V mean S/Nk also
// without V smoothing), summed over channels in channel order into E_K, EV
// and V2 of the head.
template <bool AD>
__global__ void __launch_bounds__(128) finalize_kernel(Dims d, Bufs b) {
  constexpr int U = AD ? 16 : 32;   // chunks whose partials are loaded together
  const int bh = blockIdx.x, c = threadIdx.x, D = d.D;
  const size_t base = (size_t)bh * d.NQBk * 2 * D + c;
  float tot = 0.0f, vtot = 0.0f, vx = -__builtin_inff(), vn = __builtin_inff();
  float ssk = 0.0f, ssv = 0.0f;
  int t = 0;
  for (; t + U <= d.NQBk; t += U) {   // whole batches: unconditional loads, then the in-order sums
    float kp[U], vp[U], xp[U], np[U], kq[AD ? U : 1], vq[AD ? U : 1];
#pragma unroll
    for (int u = 0; u < U; u++) {
      const size_t o = base + (size_t)(t + u) * 2 * D;
      kp[u] = b.k_part[o];
      vp[u] = b.k_part[o + D];
      xp[u] = b.v_part[o];
      np[u] = b.v_part[o + D];
      if constexpr (AD) {
        kq[u] = b.m2_part[o];
        vq[u] = b.m2_part[o + D];
      }
    }
#pragma unroll
    for (int u = 0; u < U; u++) {
      tot = tot + kp[u];
      vtot = vtot + vp[u];
      vx = fmaxf(vx, xp[u]);
      vn = fminf(vn, np[u]);
      if constexpr (AD) {
        ssk = ssk + kq[u];
        ssv = ssv + vq[u];
      }
    }
  }
  for (; t < d.NQBk; t++) {
    const size_t o = base + (size_t)t * 2 * D;
    tot = tot + b.k_part[o];
    vtot = vtot + b.k_part[o + D];
    vx = fmaxf(vx, b.v_part[o]);
    vn = fminf(vn, b.v_part[o + D]);
    if constexpr (AD) {
      ssk = ssk + b.m2_part[o];
      ssv = ssv + b.m2_part[o + D];
    }
  }
  const int n = head_io_kv(d, bh).n;   // 0 only for an empty packed sequence
  const float kbar = n ? tot / (float)n : 0.0f;
  b.k_mean[(size_t)bh * D + c] = kbar;
  const float vbar = (d.SV && n) ? vtot / (float)n : 0.0f;
  b.v_mean[(size_t)bh * D + c] = vbar;
  b.v_scale[(size_t)bh * D + c] = n ? fmaxf(fabsf(vx - vbar), fabsf(vn - vbar)) / 448.0f : 0.0f;
  if constexpr (AD) {
    const float vbs = vtot / (float)n;
    __shared__ float sEK[128], sEV[128], sV2[128];
    sEK[c] = fmaxf(ssk - tot * kbar, 0.0f);
    sEV[c] = fmaxf(ssv - vtot * vbs, 0.0f);
    sV2[c] = vtot * vbs;
    __syncthreads();
    if (c < 3) {   // three threads, one sum each, in channel order
      const float* src = c == 0 ? sEK : (c == 1 ? sEV : sV2);
      b.stat_head[(size_t)bh * 8 + 3 + c] = lds_ordered_sum(src, D);
    }
  }
}

// ---------------------------------------------------------------------------
// decide (adaptive width): grid (B*Hk), 256 threads.  The block statistics are
// summed in order (key blocks; the group's query heads in head order, each
// over its query blocks): the workgroup stages 1024 partials at a time in LDS
// (every load in flight at once) and thread 0 adds them in order.  Then, in
// fp64, INT4 iff
//   sm^2 * (A_Q*E_K + A_K*E_Q) * EV <= 11.76 * (G*Nq) * Nk * (EV + V2),
// i.e. the predicted INT4 logit variance sigma^2 (uniform rounding,
// delta = amax/7) times rho = EV / (EV + V2) is at most 0.02.
constexpr int kDecideChunk = 1024;

// Sum of n values src[i*stride] in index order (the result in thread 0).
__device__ float ordered_sum(const float* __restrict__ src, int stride, int n, float* buf) {
  float acc = 0.0f;
  for (int c0 = 0; c0 < n; c0 += kDecideChunk) {
    const int m = min(kDecideChunk, n - c0);
    for (int i = threadIdx.x; i < m; i += blockDim.x) buf[i] = src[(size_t)(c0 + i) * stride];
    __syncthreads();
    if (threadIdx.x == 0) acc = lds_ordered_sum(buf, m, acc);
    __syncthreads();
  }
  return acc;
}

__global__ void __launch_bounds__(256) decide_kernel(Dims d, Bufs b) {
  __shared__ float buf[kDecideChunk];
  const int bhk = blockIdx.x, G = d.H / d.Hk;
  const int bb = bhk / d.Hk, hk = bhk % d.Hk;
  const float ak = ordered_sum(b.stat_kblk + (size_t)bhk * d.NQBk, 1, d.NQBk, buf);
  float aq = 0.0f, eq = 0.0f;
  for (int g = 0; g < G; g++) {
    const size_t bh = (size_t)bb * d.H + (size_t)hk * G + g;
    const float* qs = b.stat_qblk + bh * d.NQB * 2;
    const float a = ordered_sum(qs, 2, d.NQB, buf);
    const float e = ordered_sum(qs + 1, 2, d.NQB, buf);
    aq = aq + a;
    eq = eq + e;
  }
  if (threadIdx.x != 0) return;
  float* st = b.stat_head + (size_t)bhk * 8;
  const float ek = st[3], ev = st[4], v2 = st[5];
  const double sm = (double)d.sm;
  const double num = (sm * sm) * ((double)aq * (double)ek + (double)ak * (double)eq) * (double)ev;
  const double den = 11.76 * ((double)G * (double)d.N * (double)d.Nk) * ((double)ev + (double)v2);
  b.head_bits[bhk] = num <= den ? 4 : 8;
  st[0] = aq;
  st[1] = eq;
  st[2] = ak;
}

// Position p (0..127) inside a 128-key block of the FP8 V layout holds key
//   64*(p/64) + 32*(s/16) + 8*((s%16)/4) + 4*((p%64)/32) + s%4,  s = p % 32.
// With this order a lane that holds P~ for the keys of one half-wave of the
// 32x32 score accumulators reads its matching 32 V bytes contiguously.
__device__ __forceinline__ int vperm_key(int p) {
  const int s = p & 31;
  return 64 * (p >> 6) + 32 * (s >> 4) + 8 * ((s & 15) >> 2) + 4 * ((p & 63) >> 5) + (s & 3);
}

// 16 consecutive 16-bit inputs (two 16-byte words) -> fp32
template <int IN>
__device__ __forceinline__ void cvt16(const v4i a, const v4i c, float* x) {
#pragma unroll
  for (int w = 0; w < 4; w++) {
    x[2 * w] = in_to_f32<IN>((uint16_t)((uint32_t)a[w] & 0xFFFF));
    x[2 * w + 1] = in_to_f32<IN>((uint16_t)((uint32_t)a[w] >> 16));
    x[8 + 2 * w] = in_to_f32<IN>((uint16_t)((uint32_t)c[w] & 0xFFFF));
    x[8 + 2 * w + 1] = in_to_f32<IN>((uint16_t)((uint32_t)c[w] >> 16));
  }
}

typedef __bf16 v8bf __attribute__((ext_vector_type(8)));

typedef __bf16 v2bf __attribute__((ext_vector_type(2)));

// Two fp32 values -> their three-piece bf16 splits x = p1 + p2 + p3, each
// piece rounded to nearest even from the residual of the ones before
// (v_cvt_pk_bf16_f32 converts a pair per instruction).
__device__ __forceinline__ float bf16_lo_f32(uint32_t w) {   // low bf16 of a packed word, as fp32
  // byte permute (0x0c: zero byte): [0, 0, b0, b1]; a plain shift would be
  // rewritten by the compiler into a second conversion of the low value
  return __uint_as_float(__builtin_amdgcn_perm(0u, w, 0x01000c0cu));
}
__device__ __forceinline__ float bf16_hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }
__device__ __forceinline__ void split3x2(float x0, float x1, uint32_t& p1, uint32_t& p2, uint32_t& p3) {
  p1 = __builtin_bit_cast(uint32_t, v2bf{(__bf16)x0, (__bf16)x1});
  const float r0 = x0 - bf16_lo_f32(p1), r1 = x1 - bf16_hi_f32(p1);
  p2 = __builtin_bit_cast(uint32_t, v2bf{(__bf16)r0, (__bf16)r1});
  const float t0 = r0 - bf16_lo_f32(p2), t1 = r1 - bf16_hi_f32(p2);
  p3 = __builtin_bit_cast(uint32_t, v2bf{(__bf16)t0, (__bf16)t1});
}
// 8 fp32 values -> three v8bf operands
__device__ __forceinline__ void split8(const float* x, v8bf& p1, v8bf& p2, v8bf& p3) {
  v4i w1, w2, w3;
#pragma unroll
  for (int e = 0; e < 4; e++) {
    uint32_t a, bb, c;
    split3x2(x[2 * e], x[2 * e + 1], a, bb, c);
    w1[e] = (int)a;
    w2[e] = (int)bb;
    w3[e] = (int)c;
  }
  p1 = __builtin_bit_cast(v8bf, w1);
  p2 = __builtin_bit_cast(v8bf, w2);
  p3 = __builtin_bit_cast(v8bf, w3);
}

// Integer codes rint(x/delta) of NV values sharing one scale (INT4: |code|
// <= 7, INT8: <= 127), as floats, bit-identical to a true IEEE division per
// element: the correctly rounded quotient from the reciprocal and one
// remainder correction (div_rn), a true division for the whole wave only when
// some lane's scale is outside the exact case.  The codes are clamped to
// [-qmax, qmax]: |x| <= amax, but delta = amax/qmax rounds below the exact
// quotient when it falls among the fp32 subnormals, and x/delta can then
// exceed qmax.  Adding +0 turns a rounded -0 into +0 (code 0 has one pattern).
template <int NV, int BITS>
__device__ __forceinline__ void int_codes_f(const float* x, float delta, float* c) {
  constexpr float qmax = BITS == 4 ? 7.0f : 127.0f;
  const float r = delta == 0.0f ? 0.0f : 1.0f / delta;
  if (__any(div_rn_hard(delta))) {
#pragma unroll
    for (int e = 0; e < NV; e++) c[e] = delta == 0.0f ? 0.0f : rintf(x[e] / delta);
  } else {
#pragma unroll
    for (int e = 0; e < NV; e++) c[e] = rintf(div_rn(x[e], delta, r));
  }
#pragma unroll
  for (int e = 0; e < NV; e++) c[e] = fminf(fmaxf(c[e], -qmax), qmax) + 0.0f;
}
typedef float v16f_t __attribute__((ext_vector_type(16)));
typedef int v6i_t __attribute__((ext_vector_type(6)));

// NF (16 or 32) integer codes in [-7, 7], given as floats, -> 3*NF/16 words
// of FP6 e2m3 fields (field e at bit 6e) with the gfx950 packing conversion
// v_cvt_scalef32_2xpk16_fp6_f32.  It takes its 32 fields from two 16-value
// operands interleaved (field 2i from the first, 2i+1 from the second), so
// even and odd codes go to the two operands; integers of magnitude <= 7 are
// exact in e2m3 (scale 1).  The instruction writes its result while it still
// reads its sources, so the result registers must not overlap them: it is
// issued with an early-clobber output (the builtin lets the register
// allocator place the result on top of the operands), followed by wait
// states before the result is read.
template <int NF>
__device__ __forceinline__ void pack_fp6_hw(const float* c, uint32_t* w) {
  static_assert(NF == 16 || NF == 32, "one or two 16-field halves");
  v16f_t ev, od;
#pragma unroll
  for (int i = 0; i < 16; i++) {
    ev[i] = 2 * i < NF ? c[2 * i] : 0.0f;
    od[i] = 2 * i + 1 < NF ? c[2 * i + 1] : 0.0f;
  }
  v6i_t r;
  asm volatile("v_cvt_scalef32_2xpk16_fp6_f32 %0, %1, %2, 1.0\n\ts_nop 4" : "=&v"(r) : "v"(ev), "v"(od));
#pragma unroll
  for (int i = 0; i < 3 * NF / 16; i++) w[i] = (uint32_t)r[i];
}

// x / dv for FP8 V codes, correctly rounded in fp32 with the sign of zero
// kept (div_rn_signed); a true division for the whole wave when some lane's
// scale is zero (an all-zero channel: +0 codes) or outside the exact case.
template <int NV>
__device__ __forceinline__ void fp8_quotients(float* x, float dv) {
  const float r = dv == 0.0f ? 0.0f : 1.0f / dv;
  if (__any(dv == 0.0f || div_rn_hard(dv))) {
#pragma unroll
    for (int e = 0; e < NV; e++) x[e] = dv == 0.0f ? 0.0f : x[e] / dv;
  } else {
#pragma unroll
    for (int e = 0; e < NV; e++) x[e] = div_rn_signed(x[e], dv, r);
  }
}

// ---------------------------------------------------------------------------
// quant: 256 threads, one 128-token block of one head; grid (blocks, heads):
// (NQB, B*H) for the query side and for self-attention, (NQBk, B*Hk) for the
// key/value side.
//  Q: one scale per token (D/16 lanes per token, 16 channels each);
//  K: one scale per 16-key fragment group (one group = 16 keys x D/32 lanes);
//  V: FP8 with the per-channel scale, written in the permuted channel-major
//     layout through an LDS copy of the block.
// MODE 0: codes of width BITS.  Adaptive width (BITS 8 layout): MODE 1 writes
// INT8 codes for every head and the block statistics of the width rule
// (per query block: the sum of amax^2 over its tokens in token order and the
// sum over channels of max(0, SSQ - SQ * mean); per key block: the sum of the
// keys' group amax^2 in key order); MODE 2 rewrites, for the heads the rule
// gave INT4, the Q and K codes and scales with qmax 7 in the same layout (V
// and the Q block means are unchanged).
template <int IN, int D, int BITS, int PART, int MODE>
__global__ void __launch_bounds__(256) quant_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v, Dims d, Bufs b) {
  static_assert(MODE == 0 || (BITS == 8 && PART != kPartBoth), "adaptive width: int8 layout, dense geometry");
  constexpr int CB = MODE == 2 ? 4 : BITS;   // code width of this pass
  constexpr float kQmax = CB == 4 ? 7.0f : 127.0f;
  constexpr bool DO_Q = PART & kPartQ, DO_KV = PART & kPartKV;
  constexpr bool DO_V = DO_KV && MODE != 2;
  __shared__ __align__(16) uint16_t sV[DO_V ? kBK * D : 8];
  __shared__ float sStat[MODE == 1 ? kBQ + D : 1];   // amax^2 per token or key; centred squares per channel
  __shared__ __align__(16) float sKM[DO_KV ? D : 4];   // K means of the head
  __shared__ __align__(16) uint16_t sQ[DO_Q ? 64 * D : 8];   // half a block of raw Q rows
  __shared__ __align__(16) float sQM[DO_Q ? D : 4];          // the block's Q means
  // packed [T, H, D] inputs: grid (B*H, NQB), heads of a token block adjacent
  const int qb = d.cu ? blockIdx.y : blockIdx.x, bh = d.cu ? blockIdx.x : blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int i0 = qb * kBQ;
  // input tokens of this head (query head, or key/value head for the K/V side)
  const HeadIO io = DO_Q ? head_io(d, bh) : head_io_kv(d, bh);
  // past the end of a shorter packed sequence: nothing here is ever read
  if (d.cu && i0 >= io.n) return;
  if constexpr (MODE == 2) {
    if (b.head_bits[DO_Q ? d.kv_head(bh) : bh] != 4) return;   // an INT8 head keeps the first pass
  }
  const size_t qrowp = (size_t)bh * d.NP;    // first padded query row of this head
  const size_t krowp = (size_t)bh * d.NPk;   // first padded key row of this head

  // Every global load of the block is issued up front (one memory round
  // trip): V by direct copies into LDS, this thread's Q and K rows into
  // registers.  Rows past the head's tokens load its last row instead; Q and
  // K zero them below, the V codes mask them by key.
  const int nlast = io.n - 1;
  const bool ragged = i0 + kBQ > io.n;   // the block holds rows past the head's tokens
  constexpr int LPT = D / 16, TPP = 256 / LPT, NQP = kBQ / TPP;   // Q: lanes per token, tokens per pass, passes
  constexpr int LPK = D / 32, LPG = 16 * LPK;                      // K: lanes per key / per scale group
  constexpr int GPW = 64 / LPG, NKI = kBK / kKGroup / (4 * GPW);   // K: groups per wave, rounds
  if constexpr (DO_V) {
    constexpr int VPT = kBK * D / 8 / 256;   // 16-byte chunks per thread
#pragma unroll
    for (int p = 0; p < VPT; p++) {
      const int wbase = 256 * p + 64 * wave, e = wbase + lane;
      const int r = e / (D / 8), c8 = e % (D / 8);
      const uint16_t* src = v + io.base + (size_t)min(i0 + r, nlast) * io.stride + 8 * c8;
      __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(sV + 8 * wbase), 16,
                                       0, 0);
    }
  }
  if constexpr (DO_KV) {
    if (wave == 0 && lane < D / 4)
      __builtin_amdgcn_global_load_lds((const void*)(b.k_mean + (size_t)bh * D + 4 * lane),
                                       (__attribute__((address_space(3))) void*)sKM, 16, 0, 0);
  }
  // V scale and mean of this thread's channel in the FP8 step (ch = tid mod D)
  const float dv_ch = DO_V ? b.v_scale[(size_t)bh * D + tid % D] : 0.0f;
  const float vbar_ch = DO_V ? b.v_mean[(size_t)bh * D + tid % D] : 0.0f;   // 0 without V smoothing
  v4i qraw[DO_Q ? NQP : 1][2];
  if constexpr (DO_Q) {
    const int c0 = 16 * (tid % LPT);
#pragma unroll
    for (int p = 0; p < NQP; p++) {
      const uint16_t* src = q + io.base + (size_t)min(i0 + tid / LPT + TPP * p, nlast) * io.stride + c0;
      qraw[p][0] = *(const v4i*)src;
      qraw[p][1] = *(const v4i*)(src + 8);
    }
  }
  v4i kraw[DO_KV ? NKI : 1][4];
  if constexpr (DO_KV) {
    const int c0 = 32 * (lane % LPK), ki = (lane % LPG) / LPK;
#pragma unroll
    for (int it = 0; it < NKI; it++) {
      const int grp = wave * GPW + lane / LPG + 4 * GPW * it, T = grp >> 1, hh = grp & 1;
      const int j = i0 + 32 * T + 8 * (ki >> 2) + 4 * hh + (ki & 3);
      const uint16_t* src = k + io.base + (size_t)min(j, nlast) * io.stride + c0;
#pragma unroll
      for (int w = 0; w < 4; w++) kraw[it][w] = *(const v4i*)(src + 8 * w);
    }
  }

  // ---- Q: LPT lanes per token, 16 channels per lane
  if constexpr (DO_Q) {
    const int sub = tid % LPT, c0 = 16 * sub;
    // Block means: thread c < D sums channel c over the block's tokens in
    // token order (fp32, one chain), then divides once by the count.  The raw
    // rows pass through LDS in two halves of 64 tokens; rows past the head's
    // tokens are staged too but not summed.
    const int nval = min(kBQ, io.n - i0);
    constexpr int PPH = NQP / 2;   // Q passes per half (64 tokens)
    static_assert(PPH * TPP == 64, "a half is 64 tokens");
    float qs = 0.0f, qss = 0.0f;   // qss: sum of squares (MODE 1)
#pragma unroll
    for (int h = 0; h < 2; h++) {
      if (h) lds_barrier();   // the first half has been summed
#pragma unroll
      for (int p = 0; p < PPH; p++) {
        uint16_t* dst = sQ + (tid / LPT + TPP * p) * D + c0;
        *(v4i*)dst = qraw[PPH * h + p][0];
        *(v4i*)(dst + 8) = qraw[PPH * h + p][1];
      }
      lds_barrier();
      if (tid < D) {
        const int nh = min(64, nval - 64 * h);   // tokens of this half to sum (may be <= 0)
        if (nh == 64) {
#pragma unroll
          for (int t0 = 0; t0 < 64; t0 += 16) {
            uint16_t x[16];
#pragma unroll
            for (int t = 0; t < 16; t++) x[t] = sQ[(t0 + t) * D + tid];
#pragma unroll
            for (int t = 0; t < 16; t++) {
              const float xf = in_to_f32<IN>(x[t]);
              qs = qs + xf;
              if constexpr (MODE == 1) qss = qss + xf * xf;
            }
          }
        } else {
          for (int t = 0; t < nh; t++) {
            const float xf = in_to_f32<IN>(sQ[t * D + tid]);
            qs = qs + xf;
            if constexpr (MODE == 1) qss = qss + xf * xf;
          }
        }
      }
    }
    if (tid < D) {
      const float m = qs / (float)nval;
      sQM[tid] = m;
      if constexpr (MODE != 2) b.q_mean[((size_t)bh * d.NQB + qb) * D + tid] = m;
      if constexpr (MODE == 1) sStat[kBQ + tid] = fmaxf(qss - qs * m, 0.0f);
    }
    lds_barrier();
    float qm[16];
#pragma unroll
    for (int e = 0; e < 16; e += 4) {
      const float4 m = *(const float4*)(sQM + c0 + e);
      qm[e] = m.x;
      qm[e + 1] = m.y;
      qm[e + 2] = m.z;
      qm[e + 3] = m.w;
    }
    // three bf16 pieces of this block's channel means for the compensation
    // kernel: pieces 1 and 2 in k_part, piece 3 in v_part (both are free once
    // the K means and V scales are final)
    if (MODE != 2 && tid < LPT) {
      uint16_t* p12 = (uint16_t*)b.k_part + ((size_t)bh * d.NQB + qb) * 2 * D;
      uint16_t* p3s = (uint16_t*)b.v_part + ((size_t)bh * d.NQB + qb) * D;
#pragma unroll
      for (int e = 0; e < 16; e += 2) {
        uint32_t p1, p2, p3;
        split3x2(qm[e], qm[e + 1], p1, p2, p3);
        *(uint32_t*)(p12 + c0 + e) = p1;
        *(uint32_t*)(p12 + D + c0 + e) = p2;
        *(uint32_t*)(p3s + c0 + e) = p3;
      }
    }
#pragma unroll
    for (int p = 0; p < NQP; p++) {
      const int i = i0 + tid / LPT + TPP * p;
      float g[16];
      cvt16<IN>(qraw[p][0], qraw[p][1], g);
#pragma unroll
      for (int e = 0; e < 16; e++) g[e] = g[e] - qm[e];
      if (ragged) {
#pragma unroll
        for (int e = 0; e < 16; e++) g[e] = i < io.n ? g[e] : 0.0f;
      }
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; e++) amax = fmaxf(amax, fabsf(g[e]));
      amax = group_max<LPT>(amax);
      if constexpr (MODE == 1) {
        if (sub == 0) sStat[tid / LPT + TPP * p] = amax * amax;   // 0 past the head's tokens
      }
      const float dq = amax / kQmax;
      float cq[16];
      int_codes_f<16, CB>(g, dq, cq);
      if constexpr (BITS == 4) {
        // FP6 tile layout: this lane's 16 channels are fields 16*(sub&1)..+15
        // of group c0/64 in half (c0/32)&1 of the row's chunk
        uint32_t w[3];
        pack_fp6_hw<16>(cq, w);
        const int hq = (c0 >> 5) & 1, odd = sub & 1;
        uint32_t* chunk = (uint32_t*)(b.q_codes + fp6_chunk_offset(D, qrowp + i, hq));
        if constexpr (D == 128) {
          const int d0 = 6 * (c0 >> 6) + 3 * odd;
#pragma unroll
          for (int k2 = 0; k2 < 3; k2++) chunk[d0 + k2] = w[k2];
        } else {
          const int rot = 4 * (((32 * hq + (i & 31)) >> 3) & 1);   // swapped halves
#pragma unroll
          for (int k2 = 0; k2 < 3; k2++) chunk[(3 * odd + k2 + rot) & 7] = w[k2];
          if (odd) {
            chunk[(6 + rot) & 7] = 0u;
            chunk[(7 + rot) & 7] = 0u;
          }
        }
      } else {
        v4i pk;
#pragma unroll
        for (int w = 0; w < 4; w++) {
          uint32_t word = 0;
#pragma unroll
          for (int e = 0; e < 4; e++) word |= ((uint32_t)(int)cq[4 * w + e] & 0xFFu) << (8 * e);
          pk[w] = (int)word;
        }
        *(v4i*)(b.q_codes + (qrowp + i) * D + 16 * sub) = pk;
      }
      if (sub == 0) b.q_scale[qrowp + i] = dq;
    }
    if constexpr (MODE == 1) {
      // the block's statistics: token order, channel order (two waves)
      lds_barrier();
      if (tid == 0 || tid == 64) {
        const float acc = tid == 0 ? lds_ordered_sum(sStat, kBQ) : lds_ordered_sum(sStat + kBQ, D);
        b.stat_qblk[((size_t)bh * d.NQB + qb) * 2 + (tid == 0 ? 0 : 1)] = acc;
      }
    }
  }
  // ---- K: a group (T, hh) holds keys 32T + 8u + 4hh + w (u, w in 0..3);
  //      LPK lanes per key, 32 channels per lane.
  if constexpr (DO_KV) {
    const int sub = lane % LPK, c0 = 32 * sub;
    const int ki = (lane % LPG) / LPK;
    wait_vmcnt<0>();   // the V and K-mean copies (and this thread's loads) have landed
    __syncthreads();
    float km[32];
#pragma unroll
    for (int e = 0; e < 32; e += 4) {
      const float4 m = *(const float4*)(sKM + c0 + e);
      km[e] = m.x;
      km[e + 1] = m.y;
      km[e + 2] = m.z;
      km[e + 3] = m.w;
    }
#pragma unroll
    for (int it = 0; it < NKI; it++) {
      const int grp = wave * GPW + lane / LPG + 4 * GPW * it, T = grp >> 1, hh = grp & 1;
      const int j = i0 + 32 * T + 8 * (ki >> 2) + 4 * hh + (ki & 3);
      float g[32];
      cvt16<IN>(kraw[it][0], kraw[it][1], g);
      cvt16<IN>(kraw[it][2], kraw[it][3], g + 16);
#pragma unroll
      for (int e = 0; e < 32; e++) g[e] = g[e] - km[e];
      if (ragged) {
#pragma unroll
        for (int e = 0; e < 32; e++) g[e] = j < io.n ? g[e] : 0.0f;
      }
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 32; e++) amax = fmaxf(amax, fabsf(g[e]));
      amax = group_max<LPG>(amax);
      if constexpr (MODE == 1) {
        if (sub == 0) sStat[j - i0] = j < io.n ? amax * amax : 0.0f;   // keys past the head count 0
      }
      const float dk = amax / kQmax;
      float ck[32];
      int_codes_f<32, CB>(g, dk, ck);
      if constexpr (BITS == 4) {
        // FP6 tile layout: this lane's 32 channels are group sub/2 of half sub&1
        uint32_t w[6];
        pack_fp6_hw<32>(ck, w);
        const int hk = sub & 1;
        uint8_t* chunk = b.k_codes + fp6_chunk_offset(D, krowp + j, hk);
        if constexpr (D == 128) {
#pragma unroll
          for (int k2 = 0; k2 < 3; k2++) {
            uint2 u;
            u.x = w[2 * k2];
            u.y = w[2 * k2 + 1];
            *(uint2*)(chunk + 24 * (sub >> 1) + 8 * k2) = u;
          }
        } else {
          const int ci = 32 * hk + (j & 31);
          const v4i lo = {(int)w[0], (int)w[1], (int)w[2], (int)w[3]};
          const v4i hi = {(int)w[4], (int)w[5], 0, 0};
          *(v4i*)(chunk + fp6_half_offset(ci, 0)) = lo;
          *(v4i*)(chunk + fp6_half_offset(ci, 1)) = hi;
        }
      } else {
#pragma unroll
        for (int half = 0; half < 2; half++) {
          v4i pk;
#pragma unroll
          for (int w = 0; w < 4; w++) {
            uint32_t word = 0;
#pragma unroll
            for (int e = 0; e < 4; e++) word |= ((uint32_t)(int)ck[16 * half + 4 * w + e] & 0xFFu) << (8 * e);
            pk[w] = (int)word;
          }
          *(v4i*)(b.k_codes + (krowp + j) * D + 32 * sub + 16 * half) = pk;
        }
      }
      if ((lane % LPG) == 0) b.k_scale[krowp / kKGroup + (i0 / kKGroup) + grp] = dk;
    }
    if constexpr (MODE == 1) {
      lds_barrier();
      if (tid == 0) b.stat_kblk[(size_t)bh * d.NQBk + qb] = lds_ordered_sum(sStat, kBK);
    }
  }
  // ---- V: 16-key chunks of one channel -> 16 FP8 bytes (channel tid mod D,
  //      chunks tid / D + (256 / D) i); the block is in LDS since the K step
  if constexpr (DO_V) {
    static_assert(256 % D == 0, "whole channels per pass");
    uint8_t* vout = b.v_codes + ((size_t)bh * d.NQBk + qb) * D * kBK;
    const int ch = tid % D;
#pragma unroll
    for (int c = tid / D; c < kBK / 16; c += 256 / D) {
      uint16_t raw[16];
#pragma unroll
      for (int u = 0; u < 16; u++) raw[u] = sV[vperm_key(16 * c + u) * D + ch];
      float x[16];
#pragma unroll
      for (int u = 0; u < 16; u++) {
        // padding keys stay exactly zero (also when V is smoothed)
        const int key = vperm_key(16 * c + u);
        x[u] = i0 + key < io.n ? in_to_f32<IN>(raw[u]) - vbar_ch : 0.0f;
      }
      fp8_quotients<16>(x, dv_ch);
      v4i pk;
#pragma unroll
      for (int w = 0; w < 4; w++) pk[w] = (int)fp8x4(x[4 * w], x[4 * w + 1], x[4 * w + 2], x[4 * w + 3]);
      *(v4i*)(vout + ch * kBK + 16 * c) = pk;
    }
  }
}

// ---------------------------------------------------------------------------
// delta_s: grid (NQBk key blocks, B*H query heads), 256 threads; wave w owns
// keys j0 + 32w .. +31 of the query head's K/V head and all Q blocks.
// DeltaS = qmean . gamma(K) on the bf16 matrix core: every fp32 operand is
// split into three bf16 pieces (x = x1 + x2 + x3 up to 2^-24 |x|) and the six
// products x_a*y_b with a + b <= 4 are accumulated in fp32, which reproduces
// an fp32 dot product to within a few units in the last place.
// Cache-policy operand of the raw buffer stores: bit 1 marks a store
// non-temporal (streamed past the caches).
constexpr int kStoreNT = 2;

template <int IN, int D>
__global__ void __launch_bounds__(256, 3) delta_s_kernel(const uint16_t* __restrict__ k, Dims d, Bufs b) {
  constexpr int NK = D / 16;   // k-steps of the 32x32x16 bf16 MFMA
  const int kb = d.cu ? blockIdx.y : blockIdx.x, bh = d.cu ? blockIdx.x : blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6, n = lane & 31, h = lane >> 5;
  const int j = kb * kBK + 32 * wave + n;        // this lane's key (B operand column)
  const int bhk = d.kv_head(bh);
  const HeadIO io = head_io_kv(d, bhk);
  // packed sequences: only key blocks and query blocks inside the sequence
  const int nkb = d.cu ? (io.n + kBK - 1) / kBK : d.NQBk;
  const int nqb = d.cu ? (head_io(d, bh).n + kBQ - 1) / kBQ : d.NQB;
  if (kb >= nkb) return;
  const float* km = b.k_mean + (size_t)bhk * D;
  // A operands: the three bf16 pieces of the Q-block means (pieces 1, 2:
  // [NQB][2][D] in k_part; piece 3: [NQB][D] in v_part), staged per 32-block
  // Q tile into LDS by direct copies, double-buffered.  LDS tile layout
  // [piece][row][D] with 16-byte chunks XOR-swizzled by row.
  constexpr int CPR = D / 8;                       // 16-byte chunks per row
  constexpr int TILE = 3 * 32 * D;                 // bf16 elements per staged tile
  constexpr int NCH = TILE / 8 / 256;              // chunks per thread
  __shared__ __align__(16) uint16_t sA0[TILE], sA1[TILE];
  const uint16_t* p12 = (const uint16_t*)b.k_part + (size_t)bh * d.NQB * 2 * D;
  const uint16_t* p3s = (const uint16_t*)b.v_part + (size_t)bh * d.NQB * D;
  auto stage = [&](int qt, uint16_t* dst) {
#pragma unroll
    for (int i = 0; i < NCH; i++) {
      const int wbase = 256 * i + 64 * wave;
      const int e = wbase + lane;
      const int piece = e / (32 * CPR), rem = e % (32 * CPR), r = rem / CPR, c = (rem % CPR) ^ (r & (CPR - 1));
      const int qrow = min(qt + r, d.NQB - 1);
      const uint16_t* src = piece < 2 ? p12 + ((size_t)qrow * 2 + piece) * D + 8 * c : p3s + (size_t)qrow * D + 8 * c;
      __builtin_amdgcn_global_load_lds((const void*)src, (__attribute__((address_space(3))) void*)(dst + 8 * wbase), 16,
                                       0, 0);
    }
  };
  // The first Q tile and the K means stream into LDS while this lane's key
  // row loads: all eight 16-byte chunks at once, from a valid row (keys past
  // the head read its last row and are zeroed below).
  __shared__ __align__(16) float sM[D];
  stage(0, sA0);
  if (tid < D) sM[tid] = km[tid];
  const bool valid = j < io.n, ragged = kb * kBK + kBK > io.n;   // ragged: this block has keys past the head
  const uint16_t* krow = k + io.base + (size_t)min(j, io.n - 1) * io.stride + 8 * h;
  v4i raw[NK];
#pragma unroll
  for (int kk = 0; kk < NK; kk++) raw[kk] = *(const v4i*)(krow + 16 * kk);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  // B operands: gamma(K) pieces for all k-steps (slot s of step kk = channel
  // 16kk + 8h + s), built during the first Q tile just before the k-step that
  // uses them, so this VALU work overlaps the tile's matrix-core work.
  v8bf B1[NK], B2[NK], B3[NK];
  auto build_b = [&](int kk) {
    const int c0 = 16 * kk + 8 * h;
    const float4 m0 = *(const float4*)(sM + c0);
    const float4 m1 = *(const float4*)(sM + c0 + 4);
    const float mv[8] = {m0.x, m0.y, m0.z, m0.w, m1.x, m1.y, m1.z, m1.w};
    float g[8];
#pragma unroll
    for (int w = 0; w < 4; w++) {
      g[2 * w] = in_to_f32<IN>((uint16_t)((uint32_t)raw[kk][w] & 0xFFFF)) - mv[2 * w];
      g[2 * w + 1] = in_to_f32<IN>((uint16_t)((uint32_t)raw[kk][w] >> 16)) - mv[2 * w + 1];
    }
    if (ragged) {
#pragma unroll
      for (int e = 0; e < 8; e++) g[e] = valid ? g[e] : 0.0f;
    }
    split8(g, B1[kk], B2[kk], B3[kk]);
  };
  // Output rows [NQB][NPk] of this head through one buffer resource: a 32-bit
  // per-lane offset (key, and the row half h) instead of a 64-bit address per
  // store; the row of each store is a scalar offset.  Every store is in range.
  const __amdgpu_buffer_rsrc_t ro = head_rsrc(b.delta_s + (size_t)bh * d.NQB * d.NPk, (uint32_t)d.NQB * d.NPk * 4);
  const uint32_t obase = ((uint32_t)(4 * h) * d.NPk + j) * 4;
  auto tile = [&](int qt, int it, auto first) {
    const bool more = qt + 32 < nqb;
    if (more) stage(qt + 32, (it & 1) ? sA0 : sA1);
    const uint16_t* A = (it & 1) ? sA1 : sA0;
    v16f acc;
#pragma unroll
    for (int r = 0; r < 16; r++) acc[r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < NK; kk++) {
      if constexpr (decltype(first)::value) build_b(kk);
      const int c = (2 * kk + h) ^ (n & (CPR - 1));
      const v8bf A1 = __builtin_bit_cast(v8bf, *(const v4i*)(A + (0 * 32 + n) * D + 8 * c));
      const v8bf A2 = __builtin_bit_cast(v8bf, *(const v4i*)(A + (1 * 32 + n) * D + 8 * c));
      const v8bf A3 = __builtin_bit_cast(v8bf, *(const v4i*)(A + (2 * 32 + n) * D + 8 * c));
      // smallest products first
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A3, B1[kk], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A2, B2[kk], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B3[kk], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A2, B1[kk], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B2[kk], acc, 0, 0, 0);
      acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A1, B1[kk], acc, 0, 0, 0);
    }
    if (more) {
      // A whole tile: exactly 16 stores, issued after the next tile's copies.
      // The wait below lets those stores stay in flight and holds only for
      // the copies (the counter retires in issue order).  The compensation
      // array is written once and read once by the attention kernel: its
      // stores are non-temporal (cache policy bit 1, "nt"; measured, values
      // unchanged: headline prepass 145.7 -> 138.1 us, LLM prefill -1.2%,
      // DiT -1.7%, the attention kernel unchanged).
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const uint32_t row = (uint32_t)(qt + 8 * (r >> 2) + (r & 3));
        __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[r]), ro, obase, row * d.NPk * 4, kStoreNT);
      }
      wait_vmcnt<16>();
      // A bare barrier: the release fence of __syncthreads() would wait for
      // every outstanding store as well.  Every LDS read of this tile has
      // returned (its matrix-core instructions consumed them), and the memory
      // clobber keeps the compiler from moving LDS accesses across it.
      asm volatile("s_barrier" ::: "memory");
    } else {
      // the last tile (possibly partial): rows past the head's query blocks are not stored
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int q2 = qt + 8 * (r >> 2) + 4 * h + (r & 3);
        if (q2 < nqb) {
          const uint32_t row = (uint32_t)(qt + 8 * (r >> 2) + (r & 3));
          __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(acc[r]), ro, obase, row * d.NPk * 4, kStoreNT);
        }
      }
    }
  };
  tile(0, 0, std::true_type{});
  for (int qt = 32, it = 1; qt < nqb; qt += 32, it++) tile(qt, it, std::false_type{});
}

__global__ void fp8_encode_kernel(const float* __restrict__ in, uint8_t* __restrict__ out, size_t n) {
  const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 4 <= n) {
    *(uint32_t*)(out + i) = fp8x4(in[i], in[i + 1], in[i + 2], in[i + 3]);
  } else {
    for (size_t e = i; e < n; e++) out[e] = (uint8_t)fp8x2(in[e], 0.0f);
  }
}

template <int IN, int D, int BITS, int MODE = 0>
void launch_quant(const uint16_t* q, const uint16_t* k, const uint16_t* v, const Dims& d, const Bufs& b,
                  hipStream_t s) {
  // Packed sequences quantize a token block of Q, K and V in one workgroup
  // (heads of a block adjacent in the grid).  Dense inputs run the query side
  // and the key/value side as two launches: their smaller workgroups (92 and
  // 133 VGPRs against 138 with 50 KB of LDS) keep more bytes in flight (LLM
  // prefill B4 H32 N4096: prepass 234 -> 227 us; the headline unchanged).
  if constexpr (MODE == 0) {
    if (d.self_attention() && d.cu) {
      hipLaunchKernelGGL((quant_kernel<IN, D, BITS, kPartBoth, 0>), dim3(d.BH(), d.NQB), dim3(256), 0, s, q, k, v, d,
                         b);
      return;
    }
  }
  hipLaunchKernelGGL((quant_kernel<IN, D, BITS, kPartQ, MODE>), dim3(d.NQB, d.BH()), dim3(256), 0, s, q, k, v, d, b);
  hipLaunchKernelGGL((quant_kernel<IN, D, BITS, kPartKV, MODE>), dim3(d.NQBk, d.BHk()), dim3(256), 0, s, q, k, v, d,
                     b);
}

template <int IN, int D>
hipError_t prepass_impl(const void* q, const void* k, const void* v, const Dims& d, const Bufs& b, hipStream_t s) {
  const uint16_t* q16 = (const uint16_t*)q;
  const uint16_t* k16 = (const uint16_t*)k;
  const uint16_t* v16 = (const uint16_t*)v;
  constexpr int CPW = 256 / (D / 2);
  auto nstat = [](long long chunks) { return dim3((unsigned)((chunks + CPW - 1) / CPW)); };
  if (d.AD) {
    // adaptive width: statistics with the INT8 pass, the choice per K/V head,
    // then the INT4 heads' codes rewritten
    hipLaunchKernelGGL((stats_kernel<IN, D, kPartKV, true>), nstat((long long)d.BHk() * d.NQBk), dim3(256), 0, s, k16,
                       v16, d, b);
    hipLaunchKernelGGL(finalize_kernel<true>, dim3(d.BHk()), dim3(D), 0, s, d, b);
    launch_quant<IN, D, 8, 1>(q16, k16, v16, d, b, s);
    hipLaunchKernelGGL(decide_kernel, dim3(d.BHk()), dim3(256), 0, s, d, b);
    launch_quant<IN, D, 8, 2>(q16, k16, v16, d, b, s);
  } else {
    hipLaunchKernelGGL((stats_kernel<IN, D, kPartKV, false>), nstat((long long)d.BHk() * d.NQBk), dim3(256), 0, s,
                       k16, v16, d, b);
    hipLaunchKernelGGL(finalize_kernel<false>, dim3(d.BHk()), dim3(D), 0, s, d, b);
    if (d.QB == 8) launch_quant<IN, D, 8>(q16, k16, v16, d, b, s);
    else launch_quant<IN, D, 4>(q16, k16, v16, d, b, s);
  }
  const dim3 ds_grid = d.cu ? dim3(d.BH(), d.NQBk) : dim3(d.NQBk, d.BH());
  hipLaunchKernelGGL((delta_s_kernel<IN, D>), ds_grid, dim3(256), 0, s, k16, d, b);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepass(const void* q, const void* k, const void* v, int in_dtype, const Dims& d, const Bufs& b,
                          hipStream_t s) {
  if (in_dtype == kBF16) return d.D == 64 ? prepass_impl<1, 64>(q, k, v, d, b, s) : prepass_impl<1, 128>(q, k, v, d, b, s);
  return d.D == 64 ? prepass_impl<0, 64>(q, k, v, d, b, s) : prepass_impl<0, 128>(q, k, v, d, b, s);
}

// Value statistics alone (V channel sums, maxima and minima per chunk, then V
// means and V scales per K/V head; the K sums and so the K means are left
// zero): the first half of a decoding step.
hipError_t launch_v_stats(const void* v, int in_dtype, const Dims& d, const Bufs& b, hipStream_t s) {
  const uint16_t* v16 = (const uint16_t*)v;
  const int cpw = 256 / (d.D / 2);
  const dim3 grid((unsigned)(((long long)d.BHk() * d.NQBk + cpw - 1) / cpw));
  if (in_dtype == kBF16) {
    if (d.D == 64) hipLaunchKernelGGL((stats_kernel<1, 64, kPartV, false>), grid, dim3(256), 0, s, nullptr, v16, d, b);
    else hipLaunchKernelGGL((stats_kernel<1, 128, kPartV, false>), grid, dim3(256), 0, s, nullptr, v16, d, b);
  } else {
    if (d.D == 64) hipLaunchKernelGGL((stats_kernel<0, 64, kPartV, false>), grid, dim3(256), 0, s, nullptr, v16, d, b);
    else hipLaunchKernelGGL((stats_kernel<0, 128, kPartV, false>), grid, dim3(256), 0, s, nullptr, v16, d, b);
  }
  hipLaunchKernelGGL(finalize_kernel<false>, dim3(d.BHk()), dim3(d.D), 0, s, d, b);
  return hipGetLastError();
}

hipError_t launch_fp8_encode(const float* in, uint8_t* out, size_t n, hipStream_t s) {
  const size_t threads = (n + 3) / 4;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(fp8_encode_kernel, dim3(blocks), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

}  // namespace sage
