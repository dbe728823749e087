// SageAttention2 prepass on gfx950: smoothing statistics, INT4 Q/K codes with
// fine-grained scales, FP8 V with per-channel scales, compensation term.
//
// Method: SageAttention2 abstract (arXiv 2411.10958 page) -- Q,K to INT4 at a
// thread-level granularity, V to FP8, smoothing of Q; the title's "thorough
// outlier smoothing" is read as also removing the per-channel K mean.  The
// readings taken where the pages are silent (block sizes, scale groups, mean
// order, rounding) are the contract constants of sage_internal.h.
//
// All kernels here are HBM-bound except the compensation term (VALU-bound
// dot products); they are launched in order on the caller's stream:
//   stats -> finalize -> quant -> delta_s.
#include "sage_internal.h"
#include "sage_device.h"

namespace sage {
namespace {

// ---------------------------------------------------------------------------
// stats: grid (NQB, B*H), D threads.  Thread c walks the 128 tokens of its
// chunk in order: Q block sum -> Q block mean, K chunk sum, V chunk absmax.
template <int IN, int D>
__global__ void __launch_bounds__(D) stats_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                  const uint16_t* __restrict__ v, Dims d, Bufs b) {
  const int qb = blockIdx.x, bh = blockIdx.y, c = threadIdx.x;
  const int i0 = qb * kBQ, i1 = min(d.N, i0 + kBQ);
  const size_t base = ((size_t)bh * d.N) * D + c;
  float qs = 0.0f, ks = 0.0f, vm = 0.0f;
  int i = i0;
  for (; i + 8 <= i1; i += 8) {
    uint16_t qv[8], kv[8], vv[8];
#pragma unroll
    for (int u = 0; u < 8; u++) {
      qv[u] = q[base + (size_t)(i + u) * D];
      kv[u] = k[base + (size_t)(i + u) * D];
      vv[u] = v[base + (size_t)(i + u) * D];
    }
#pragma unroll
    for (int u = 0; u < 8; u++) {
      qs = qs + in_to_f32<IN>(qv[u]);
      ks = ks + in_to_f32<IN>(kv[u]);
      vm = fmaxf(vm, fabsf(in_to_f32<IN>(vv[u])));
    }
  }
  for (; i < i1; i++) {
    qs = qs + in_to_f32<IN>(q[base + (size_t)i * D]);
    ks = ks + in_to_f32<IN>(k[base + (size_t)i * D]);
    vm = fmaxf(vm, fabsf(in_to_f32<IN>(v[base + (size_t)i * D])));
  }
  const size_t o = ((size_t)bh * d.NQB + qb) * D + c;
  b.q_mean[o] = qs / (float)(i1 - i0);
  b.k_part[o] = ks;
  b.v_part[o] = vm;
}

// ---------------------------------------------------------------------------
// finalize: grid (B*H), D threads.  K mean = (sum of chunk sums, in chunk
// order) / N; V scale = (max of chunk absmax) / 448.
__global__ void finalize_kernel(Dims d, Bufs b) {
  const int bh = blockIdx.x, c = threadIdx.x, D = d.D;
  float tot = 0.0f, vm = 0.0f;
  for (int t = 0; t < d.NQB; t++) {
    const size_t o = ((size_t)bh * d.NQB + t) * D + c;
    tot = tot + b.k_part[o];
    vm = fmaxf(vm, b.v_part[o]);
  }
  b.k_mean[(size_t)bh * D + c] = tot / (float)d.N;
  b.v_scale[(size_t)bh * D + c] = vm / 448.0f;
}

// Position p (0..127) inside a 128-key block of the FP8 V layout holds key
//   64*(p/64) + 32*(s/16) + 8*((s%16)/4) + 4*((p%64)/32) + s%4,  s = p % 32.
// With this order a lane that holds P~ for the keys of one half-wave of the
// 32x32 score accumulators reads its matching 32 V bytes contiguously.
__device__ __forceinline__ int vperm_key(int p) {
  const int s = p & 31;
  return 64 * (p >> 6) + 32 * (s >> 4) + 8 * ((s & 15) >> 2) + 4 * ((p & 63) >> 5) + (s & 3);
}

// ---------------------------------------------------------------------------
// quant: grid (NQB, B*H), 256 threads.  One 128-token block of one head:
//  Q: one scale per token; K: one scale per 16-key fragment group; V: FP8.
template <int IN, int D>
__global__ void __launch_bounds__(256) quant_kernel(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                    const uint16_t* __restrict__ v, Dims d, Bufs b) {
  constexpr int LPR = D / 2;          // lanes per row: one lane per channel pair
  constexpr int ROWS = 256 / LPR;     // rows handled in parallel
  __shared__ float sV[kBK][D + 1];
  const int qb = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int lb = tid % LPR, slot = tid / LPR;
  const int i0 = qb * kBQ;
  const size_t hrow = (size_t)bh * d.N;      // first input row of this head
  const size_t hrowp = (size_t)bh * d.NP;    // first padded row of this head

  // ---- Q: per token
  {
    const float m0 = b.q_mean[((size_t)bh * d.NQB + qb) * D + 2 * lb];
    const float m1 = b.q_mean[((size_t)bh * d.NQB + qb) * D + 2 * lb + 1];
    for (int r = slot; r < kBQ; r += ROWS) {
      const int i = i0 + r;
      float g0 = 0.0f, g1 = 0.0f;
      if (i < d.N) {
        const uint32_t pr = *(const uint32_t*)(q + (hrow + i) * D + 2 * lb);
        g0 = in_to_f32<IN>((uint16_t)(pr & 0xFFFF)) - m0;
        g1 = in_to_f32<IN>((uint16_t)(pr >> 16)) - m1;
      }
      const float amax = group_max<LPR>(fmaxf(fabsf(g0), fabsf(g1)));
      const float dq = amax / 7.0f;
      b.q_codes[(hrowp + i) * (D / 2) + lb] = (uint8_t)pack_pair(int4_code(g0, dq), int4_code(g1, dq));
      if (lb == 0) b.q_scale[hrowp + i] = dq;
    }
  }
  // ---- K: per 16-key group.  Group (T, hh) of the block holds keys
  //      32*T + 8*u + 4*hh + w, u, w in 0..3.
  {
    const float m0 = b.k_mean[(size_t)bh * D + 2 * lb];
    const float m1 = b.k_mean[(size_t)bh * D + 2 * lb + 1];
    for (int grp = slot; grp < kBK / kKGroup; grp += ROWS) {
      const int T = grp >> 1, hh = grp & 1;
      float g[16][2];
      float amax = 0.0f;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int j = i0 + 32 * T + 8 * (e >> 2) + 4 * hh + (e & 3);
        g[e][0] = 0.0f;
        g[e][1] = 0.0f;
        if (j < d.N) {
          const uint32_t pr = *(const uint32_t*)(k + (hrow + j) * D + 2 * lb);
          g[e][0] = in_to_f32<IN>((uint16_t)(pr & 0xFFFF)) - m0;
          g[e][1] = in_to_f32<IN>((uint16_t)(pr >> 16)) - m1;
        }
        amax = fmaxf(amax, fmaxf(fabsf(g[e][0]), fabsf(g[e][1])));
      }
      amax = group_max<LPR>(amax);
      const float dk = amax / 7.0f;
#pragma unroll
      for (int e = 0; e < 16; e++) {
        const int j = i0 + 32 * T + 8 * (e >> 2) + 4 * hh + (e & 3);
        b.k_codes[(hrowp + j) * (D / 2) + lb] = (uint8_t)pack_pair(int4_code(g[e][0], dk), int4_code(g[e][1], dk));
      }
      if (lb == 0) b.k_scale[hrowp / kKGroup + (i0 / kKGroup) + grp] = dk;
    }
  }
  // ---- V: stage the block in LDS as fp32, then write FP8 in the permuted,
  //      channel-major layout [D][128].
  for (int e = tid; e < kBK * D / 2; e += 256) {
    const int r = e / (D / 2), cp = e % (D / 2);
    const int j = i0 + r;
    float a = 0.0f, c2 = 0.0f;
    if (j < d.N) {
      const uint32_t pr = *(const uint32_t*)(v + (hrow + j) * D + 2 * cp);
      a = in_to_f32<IN>((uint16_t)(pr & 0xFFFF));
      c2 = in_to_f32<IN>((uint16_t)(pr >> 16));
    }
    sV[r][2 * cp] = a;
    sV[r][2 * cp + 1] = c2;
  }
  __syncthreads();
  uint32_t* vout = (uint32_t*)(b.v_codes + ((size_t)bh * d.NQB + qb) * D * kBK);
  for (int w = tid; w < D * kBK / 4; w += 256) {
    const int ch = w % D, p4 = w / D;
    const float dv = b.v_scale[(size_t)bh * D + ch];
    float x[4];
#pragma unroll
    for (int u = 0; u < 4; u++) {
      const int key = vperm_key(4 * p4 + u);
      x[u] = (dv == 0.0f || i0 + key >= d.N) ? 0.0f : sV[key][ch] / dv;
    }
    vout[(ch * kBK) / 4 + p4] = fp8x4(x[0], x[1], x[2], x[3]);
  }
}

// ---------------------------------------------------------------------------
// delta_s: grid (NQB key blocks, B*H), 256 threads.  For the 128 keys of the
// block and every Q block qb: sum_c qmean[qb][c] * (K[j][c] - kmean[c]), an
// fp32 fma chain in channel order, times ds_scale.
template <int IN, int D>
__global__ void __launch_bounds__(256) delta_s_kernel(const uint16_t* __restrict__ k, Dims d, Bufs b, float ds_scale) {
  constexpr int QC = 16;  // Q blocks per pass
  __shared__ float sG[D][kBK];
  __shared__ float sQ[QC][D];
  const int kb = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
  const int j0 = kb * kBK;
  const size_t hrow = (size_t)bh * d.N;
  for (int e = tid; e < kBK * D; e += 256) {
    const int r = e / D, c = e % D;
    const int j = j0 + r;
    float g = 0.0f;
    if (j < d.N) g = in_to_f32<IN>(k[(hrow + j) * D + c]) - b.k_mean[(size_t)bh * D + c];
    sG[c][r] = g;
  }
  const int jl = tid % kBK, half = tid / kBK;   // 2 groups of 128 threads
  for (int qc0 = 0; qc0 < d.NQB; qc0 += QC) {
    __syncthreads();
    for (int e = tid; e < QC * D; e += 256) {
      const int qq = e / D, c = e % D;
      sQ[qq][c] = (qc0 + qq < d.NQB) ? b.q_mean[((size_t)bh * d.NQB + qc0 + qq) * D + c] : 0.0f;
    }
    __syncthreads();
    float acc[QC / 2];
#pragma unroll
    for (int u = 0; u < QC / 2; u++) acc[u] = 0.0f;
    for (int c = 0; c < D; c++) {
      const float g = sG[c][jl];
#pragma unroll
      for (int u = 0; u < QC / 2; u++) acc[u] = __builtin_fmaf(sQ[half + 2 * u][c], g, acc[u]);
    }
#pragma unroll
    for (int u = 0; u < QC / 2; u++) {
      const int qb = qc0 + half + 2 * u;
      if (qb < d.NQB) b.delta_s[((size_t)bh * d.NQB + qb) * d.NP + j0 + jl] = acc[u] * ds_scale;
    }
  }
}

__global__ void fp8_encode_kernel(const float* __restrict__ in, uint8_t* __restrict__ out, size_t n) {
  const size_t i = ((size_t)blockIdx.x * blockDim.x + threadIdx.x) * 4;
  if (i + 4 <= n) {
    *(uint32_t*)(out + i) = fp8x4(in[i], in[i + 1], in[i + 2], in[i + 3]);
  } else {
    for (size_t e = i; e < n; e++) out[e] = (uint8_t)fp8x2(in[e], 0.0f);
  }
}

template <int IN, int D>
hipError_t prepass_impl(const void* q, const void* k, const void* v, const Dims& d, const Bufs& b, float ds_scale,
                        hipStream_t s) {
  const dim3 grid(d.NQB, d.BH());
  const uint16_t* q16 = (const uint16_t*)q;
  const uint16_t* k16 = (const uint16_t*)k;
  const uint16_t* v16 = (const uint16_t*)v;
  hipLaunchKernelGGL((stats_kernel<IN, D>), grid, dim3(D), 0, s, q16, k16, v16, d, b);
  hipLaunchKernelGGL(finalize_kernel, dim3(d.BH()), dim3(D), 0, s, d, b);
  hipLaunchKernelGGL((quant_kernel<IN, D>), grid, dim3(256), 0, s, q16, k16, v16, d, b);
  hipLaunchKernelGGL((delta_s_kernel<IN, D>), grid, dim3(256), 0, s, k16, d, b, ds_scale);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prepass(const void* q, const void* k, const void* v, int in_dtype, const Dims& d, const Bufs& b,
                          float ds_scale, hipStream_t s) {
  if (in_dtype == kBF16) {
    return d.D == 64 ? prepass_impl<1, 64>(q, k, v, d, b, ds_scale, s) : prepass_impl<1, 128>(q, k, v, d, b, ds_scale, s);
  }
  return d.D == 64 ? prepass_impl<0, 64>(q, k, v, d, b, ds_scale, s) : prepass_impl<0, 128>(q, k, v, d, b, ds_scale, s);
}

hipError_t launch_fp8_encode(const float* in, uint8_t* out, size_t n, hipStream_t s) {
  const size_t threads = (n + 3) / 4;
  const unsigned blocks = (unsigned)((threads + 255) / 256);
  hipLaunchKernelGGL(fp8_encode_kernel, dim3(blocks), dim3(256), 0, s, in, out, n);
  return hipGetLastError();
}

}  // namespace sage
