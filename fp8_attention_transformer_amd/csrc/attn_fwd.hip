// SageAttention2 fused attention forward on gfx950.
//
// Method (SageAttention2 abstract, arXiv 2411.10958 page): INT4 QK^T with
// fine-grained scales, online softmax, FP8 P~ and V, and a two-level
// accumulation of P~V (a per-block partial in a fresh FP32 buffer, then added
// into an FP32 running buffer).
//
// gfx950 mapping.  A workgroup owns one 128-query block of one head (4 waves x
// 32 queries).  Scores are built transposed, S^T = K * Q^T, with the INT8
// matrix core (v_mfma_i32_32x32x32_i8): every lane then holds one query and 16
// keys of each 32-key tile, so the dequantization factor is one scalar per
// lane and tile (per-token Q scale times the scale of the lane's 16-key K
// group) and row reductions of the online softmax stay inside a lane plus one
// exchange with the partner lane 32 away.  P~ stays in registers: converted to
// e4m3 it is directly the B operand of the FP8 matrix core
// (v_mfma_f32_32x32x64_f8f6f4) computing O^T += V^T P~^T, with V stored by the
// prepass in the matching permuted channel-major layout.
//
// INT4 on the INT8 matrix core without unpacking.  A packed byte holds the
// pair (c_even, c_odd) as 16*c_odd + c_even + 8.  Read as int8, byte b is
// 16*c_odd + u with u = c_even + 8; masked with 0xF0 it is 16*c_odd.  With the
// query operands x = 16*q_even and y = q_odd - 16*q_even (both within int8),
//   raw*x + masked*y = 16*(c_odd*q_odd + c_even*q_even) + 128*q_even,
// so two MFMAs over the raw and masked K bytes give 16 times the integer dot
// product plus a per-query constant 128*sum(q_even).  That constant is removed
// by starting the accumulation from a register block holding -128*sum(q_even)
// (MFMA C operand distinct from D), so each K byte costs a quarter of an AND.
#include "sage_internal.h"
#include "sage_device.h"

namespace sage {
namespace {

constexpr float kLog2_448 = 8.80735492205760410744f;

template <int D>
struct QOperand {
  static constexpr int NPAIR = D / 64;
  v4i x[NPAIR];
  v4i y[NPAIR];
  v16i cinit;
};

// Build the query operands for lane (query row `qrow` in padded coordinates,
// half h) from the packed codes.  Both lanes of a query end with the same
// correction block.
template <int D>
__device__ __forceinline__ void load_q_operand(const uint8_t* __restrict__ q_codes_head, int qrow, int h,
                                               QOperand<D>& op) {
  constexpr int KROW = D / 2;
  int corr = 0;
#pragma unroll
  for (int pr = 0; pr < QOperand<D>::NPAIR; pr++) {
    const v4i raw = *(const v4i*)(q_codes_head + (size_t)qrow * KROW + pr * 32 + h * 16);
#pragma unroll
    for (int w = 0; w < 4; w++) {
      uint32_t xw = 0, yw = 0;
#pragma unroll
      for (int bb = 0; bb < 4; bb++) {
        const int v = (int)(int8_t)((uint32_t)raw[w] >> (8 * bb));
        const int ce = (v & 15) - 8;
        const int co = v >> 4;
        corr += ce;
        xw |= ((uint32_t)(16 * ce) & 0xFFu) << (8 * bb);
        yw |= ((uint32_t)(co - 16 * ce) & 0xFFu) << (8 * bb);
      }
      op.x[pr][w] = (int)xw;
      op.y[pr][w] = (int)yw;
    }
  }
  corr += __shfl_xor(corr, 32);
#pragma unroll
  for (int r = 0; r < 16; r++) op.cinit[r] = -128 * corr;
}

// One 32-key tile of S^T (times 16): `a[pr]` holds this lane's 16 packed K
// bytes (key row lane%32, half h) for channel pair-block pr.
template <int D>
__device__ __forceinline__ v16i qk_tile(const v4i* a, const QOperand<D>& op) {
  v16i s = op.cinit;
#pragma unroll
  for (int pr = 0; pr < QOperand<D>::NPAIR; pr++) {
    s = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[pr], op.x[pr], s, 0, 0, 0);
    const v4i hi = a[pr] & (int)0xF0F0F0F0;
    s = __builtin_amdgcn_mfma_i32_32x32x32_i8(hi, op.y[pr], s, 0, 0, 0);
  }
  return s;
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

// Map the hardware workgroup id to (head, query block).  Workgroups are
// dealt round-robin to the 8 XCDs; renumbering gives every XCD a contiguous
// range of logical ids, so the query blocks of one head share an L2.
__device__ __forceinline__ int xcd_logical_id(int pid, int nwg) {
  const int xcd = pid & 7, idx = pid >> 3;
  const int per = nwg >> 3, rem = nwg & 7;
  return xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
}

template <int D, bool CAUSAL>
__global__ void __launch_bounds__(256, 2) attn_kernel(Bufs b, Dims d, float ks, void* __restrict__ o, int out_dtype) {
  constexpr int KROW = D / 2;
  constexpr int NPAIR = D / 64;
  constexpr int NDT = D / 32;
  __shared__ __align__(16) uint8_t sK[kBK * KROW];
  __shared__ __align__(16) uint8_t sV[D * kBK];
  __shared__ float sDS[kBK];
  __shared__ float sKS[kBK / kKGroup];

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5;

  const int logical = xcd_logical_id(blockIdx.x, gridDim.x);
  const int bh = logical / d.NQB;
  const int jq = logical % d.NQB;
  const int qb = CAUSAL ? d.NQB - 1 - jq : jq;
  const int qrow = qb * kBQ + wave * 32 + n;     // padded query index of this lane
  const size_t hrowp = (size_t)bh * d.NP;

  QOperand<D> qop;
  load_q_operand<D>(b.q_codes + hrowp * KROW, qrow, h, qop);
  const float dq = b.q_scale[hrowp + qrow];
  const float* dsrow = b.delta_s + ((size_t)bh * d.NQB + qb) * d.NP;
  const uint8_t* kblk = b.k_codes + hrowp * KROW;
  const uint8_t* vblk = b.v_codes + (size_t)bh * d.NQB * D * kBK;
  const float* kscl = b.k_scale + hrowp / kKGroup;

  v16f O[NDT];
#pragma unroll
  for (int dt = 0; dt < NDT; dt++)
#pragma unroll
    for (int r = 0; r < 16; r++) O[dt][r] = 0.0f;
  float m = -__builtin_inff(), l = 0.0f;

  const int tend = CAUSAL ? qb + 1 : d.NQB;
  for (int t = 0; t < tend; t++) {
    __syncthreads();
    {  // stage this key block: K codes, FP8 V, compensation row (times ks), K scales
      const v4i* gk = (const v4i*)(kblk + (size_t)t * kBK * KROW);
      v4i* lk = (v4i*)sK;
#pragma unroll
      for (int e = tid; e < kBK * KROW / 16; e += 256) lk[e] = gk[e];
      const v4i* gv = (const v4i*)(vblk + (size_t)t * D * kBK);
      v4i* lv = (v4i*)sV;
#pragma unroll
      for (int e = tid; e < D * kBK / 16; e += 256) lv[e] = gv[e];
      if (tid < kBK) sDS[tid] = dsrow[t * kBK + tid] * ks;
      if (tid < kBK / kKGroup) sKS[tid] = kscl[t * (kBK / kKGroup) + tid];
    }
    __syncthreads();

    // ---- S^T for 4 tiles of 32 keys
    v16i S[4];
#pragma unroll
    for (int T = 0; T < 4; T++) {
      v4i a[NPAIR];
#pragma unroll
      for (int pr = 0; pr < NPAIR; pr++) a[pr] = *(const v4i*)(sK + (32 * T + n) * KROW + pr * 32 + h * 16);
      S[T] = qk_tile<D>(a, qop);
    }

    // ---- dequantize into the log2 domain, mask, block max
    float s2[4][16];
    float bmax = -__builtin_inff();
    const bool need_mask = (CAUSAL && t == qb) || (t == d.NQB - 1 && d.N != d.NP);
#pragma unroll
    for (int T = 0; T < 4; T++) {
      const float c = ((dq * sKS[2 * T + h]) * ks) * 0.0625f;
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int key = 32 * T + 8 * (r >> 2) + 4 * h + (r & 3);
        s2[T][r] = __builtin_fmaf((float)S[T][r], c, sDS[key]);
      }
      if (need_mask) {
#pragma unroll
        for (int r = 0; r < 16; r++) {
          const int key = t * kBK + 32 * T + 8 * (r >> 2) + 4 * h + (r & 3);
          const bool bad = (key >= d.N) || (CAUSAL && key > qrow);
          if (bad) s2[T][r] = -__builtin_inff();
        }
      }
#pragma unroll
      for (int r = 0; r < 16; r++) bmax = fmaxf(bmax, s2[T][r]);
    }
    bmax = fmaxf(bmax, __shfl_xor(bmax, 32));
    const float mnew = fmaxf(m, bmax);
    const float alpha = __builtin_amdgcn_exp2f(m - mnew);
    const float mm = mnew - kLog2_448;

    // ---- p' = exp2(s2 - mm) in [0, 448]; row sum; P~ -> e4m3 B operands
    float rowsum = 0.0f;
    v8i P8[2];
#pragma unroll
    for (int T = 0; T < 4; T++) {
      float p[16];
#pragma unroll
      for (int r = 0; r < 16; r++) {
        p[r] = __builtin_amdgcn_exp2f(s2[T][r] - mm);
        rowsum += p[r];
      }
#pragma unroll
      for (int w = 0; w < 4; w++) P8[T >> 1][4 * (T & 1) + w] = (int)fp8x4(p[4 * w], p[4 * w + 1], p[4 * w + 2], p[4 * w + 3]);
    }
    rowsum += __shfl_xor(rowsum, 32);
    l = alpha * l + rowsum;
    m = mnew;

    // ---- two-level P~V: fresh FP32 partial R per d-tile, then O = alpha*O + R
#pragma unroll
    for (int dt = 0; dt < NDT; dt++) {
      v16f R;
#pragma unroll
      for (int r = 0; r < 16; r++) R[r] = 0.0f;
#pragma unroll
      for (int kh = 0; kh < 2; kh++) {
        const v8i av = *(const v8i*)(sV + (32 * dt + n) * kBK + kh * 64 + h * 32);
        R = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(av, P8[kh], R, 0, 0, 0, 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < 16; r++) O[dt][r] = __builtin_fmaf(alpha, O[dt][r], R[r]);
    }
  }

  // ---- epilogue: O = (O_run * vscale) / l'
  const int qi = qrow;
  if (qi < d.N) {
    const float* vs = b.v_scale + (size_t)bh * D;
    const size_t orow = ((size_t)bh * d.N + qi) * D;
#pragma unroll
    for (int dt = 0; dt < NDT; dt++)
#pragma unroll
      for (int r = 0; r < 16; r++) {
        const int ch = 32 * dt + 8 * (r >> 2) + 4 * h + (r & 3);
        store_out(o, orow + ch, (O[dt][r] * vs[ch]) / l, out_dtype);
      }
  }
}

// Debug: exact int32 QK^T for a (nq x nk) window of one head, through the same
// tile function as the fused kernel.  Grid (ceil(nq/32), ceil(nk/32)), 64 threads.
template <int D>
__global__ void __launch_bounds__(64) qk_debug_kernel(Bufs b, Dims d, int bh, int q0, int k0, int nq, int nk,
                                                      int32_t* __restrict__ out) {
  constexpr int KROW = D / 2;
  const int lane = threadIdx.x, n = lane & 31, h = lane >> 5;
  const size_t hrowp = (size_t)bh * d.NP;
  const int qloc = blockIdx.x * 32 + n;
  const int kbase = blockIdx.y * 32;
  const int qrow = min(q0 + qloc, d.NP - 1);
  QOperand<D> qop;
  load_q_operand<D>(b.q_codes + hrowp * KROW, qrow, h, qop);
  const int krow = min(k0 + kbase + n, d.NP - 1);
  v4i a[D / 64];
#pragma unroll
  for (int pr = 0; pr < D / 64; pr++) a[pr] = *(const v4i*)(b.k_codes + (hrowp + krow) * KROW + pr * 32 + h * 16);
  const v16i s = qk_tile<D>(a, qop);
#pragma unroll
  for (int r = 0; r < 16; r++) {
    const int kloc = kbase + 8 * (r >> 2) + 4 * h + (r & 3);
    if (qloc < nq && kloc < nk) out[(size_t)qloc * nk + kloc] = s[r] >> 4;
  }
}

template <int D>
hipError_t attn_impl(const Bufs& b, const Dims& d, int causal, float ks, void* o, int out_dtype, hipStream_t s) {
  const dim3 grid(d.NQB * d.BH());
  if (causal) hipLaunchKernelGGL((attn_kernel<D, true>), grid, dim3(256), 0, s, b, d, ks, o, out_dtype);
  else hipLaunchKernelGGL((attn_kernel<D, false>), grid, dim3(256), 0, s, b, d, ks, o, out_dtype);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn(const Bufs& b, const Dims& d, int causal, float ks, void* o, int out_dtype, hipStream_t s) {
  return d.D == 64 ? attn_impl<64>(b, d, causal, ks, o, out_dtype, s) : attn_impl<128>(b, d, causal, ks, o, out_dtype, s);
}

hipError_t launch_qk_debug(const Bufs& b, const Dims& d, int bh, int q0, int k0, int nq, int nk, int32_t* out,
                           hipStream_t s) {
  const dim3 grid((nq + 31) / 32, (nk + 31) / 32);
  if (d.D == 64) hipLaunchKernelGGL(qk_debug_kernel<64>, grid, dim3(64), 0, s, b, d, bh, q0, k0, nq, nk, out);
  else hipLaunchKernelGGL(qk_debug_kernel<128>, grid, dim3(64), 0, s, b, d, bh, q0, k0, nq, nk, out);
  return hipGetLastError();
}

}  // namespace sage
