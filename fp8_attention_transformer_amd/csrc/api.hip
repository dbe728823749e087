// C ABI of libsage (declarations and documentation in include/sage.h).
#include "sage.h"

#include <cmath>
#include <cstring>
#include <mutex>

#include "sage_internal.h"

namespace {

using sage::Bufs;
using sage::Dims;

constexpr size_t kAlign = 256;
constexpr int kMaxDevices = 64;

size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

bool mul_ok(size_t a, size_t b, size_t* out) {
  if (a != 0 && b > SIZE_MAX / a) return false;
  *out = a * b;
  return true;
}

// Queries [B, Hq, Nq, D], keys and values [B, Hkv, Nk, D].
bool shape_ok(int B, int Hq, int Hkv, int Nq, int Nk, int D) {
  if (B < 1 || Hq < 1 || Hkv < 1 || Nq < 1 || Nk < 1) return false;
  if (Hq % Hkv) return false;
  if (D != 64 && D != 128) return false;
  // keep every index computed in 32-bit arithmetic inside the kernels in range,
  // and every buffer resource within its 32-bit byte range: the 16-bit K or
  // V rows of a head (decoding step, 2*D bytes a row) and the DeltaS rows of
  // a query head (NQB * NPk fp32, written through one resource)
  const long long NPq = ((long long)Nq + 127) / 128 * 128, NPk = ((long long)Nk + 127) / 128 * 128;
  if (NPq > (1LL << 23) || NPk > (1LL << 23)) return false;
  if (NPq / 128 * NPk >= (1LL << 30)) return false;
  if ((long long)B * Hq > 65535) return false;   // grid y dimension of the prepass
  if ((long long)B * Hq * (NPq / 128) > (1LL << 30)) return false;
  if ((long long)B * Hkv * (NPk / 128) > (1LL << 30)) return false;
  return true;
}

bool bits_ok(int qk_bits) { return qk_bits == 4 || qk_bits == 8; }
// also 0, the adaptive width (dense entry points; the codes use the 8-bit layout)
bool bits_ok_ad(int qk_bits) { return qk_bits == 0 || bits_ok(qk_bits); }

Dims make_dims(int B, int Hq, int Hkv, int Nq, int Nk, int D, int qk_bits = 8, int smooth_v = 0,
               float sm_scale = 0.0f) {
  Dims d;
  d.B = B;
  d.H = Hq;
  d.N = Nq;
  d.D = D;
  d.NP = (Nq + 127) / 128 * 128;
  d.NQB = d.NP / 128;
  d.Hk = Hkv;
  d.Nk = Nk;
  d.NPk = (Nk + 127) / 128 * 128;
  d.NQBk = d.NPk / 128;
  d.QB = qk_bits ? qk_bits : 8;
  d.SV = smooth_v;
  d.AD = qk_bits == 0;
  d.sm = sm_scale;
  d.cu = nullptr;
  d.T = 0;
  return d;
}

constexpr int kNumArrays = 15;

// Sizes of the workspace arrays, in the order of sage_quant_bufs.  The code
// arrays are sized for 8-bit codes so that one layout serves both code widths.
bool layout(const Dims& d, size_t sizes[kNumArrays]) {
  const size_t D = (size_t)d.D;
  const size_t bhq = (size_t)d.B * d.H, bhk = (size_t)d.B * d.Hk;
  size_t qrows, krows, qblk, kblk, t;
  if (!mul_ok(bhq, (size_t)d.NP, &qrows) || !mul_ok(bhk, (size_t)d.NPk, &krows)) return false;
  if (!mul_ok(bhq, (size_t)d.NQB, &qblk) || !mul_ok(bhk, (size_t)d.NQBk, &kblk)) return false;
  if (!mul_ok(qrows, D, &sizes[0])) return false;           // q_codes
  if (!mul_ok(krows, D, &sizes[1])) return false;           // k_codes
  if (!mul_ok(qrows, 4, &sizes[2])) return false;           // q_scale
  sizes[3] = krows / 16 * 4;                                 // k_scale
  if (!mul_ok(qblk, D * 4, &sizes[4])) return false;        // q_mean
  sizes[5] = bhk * D * 4;                                    // k_mean
  if (!mul_ok(krows, D, &sizes[6])) return false;           // v_codes
  sizes[7] = bhk * D * 4;                                    // v_scale
  if (!mul_ok(qblk, (size_t)d.NPk, &t) || !mul_ok(t, 4, &sizes[8])) return false;  // delta_s
  // per-chunk K/V statistics, later the bf16 pieces of the Q block means
  if (!mul_ok(kblk, 2 * D * 4, &t)) return false;
  sizes[9] = t > qblk * 2 * D * 2 ? t : qblk * 2 * D * 2;   // k_part
  sizes[10] = t > qblk * D * 2 ? t : qblk * D * 2;          // v_part
  sizes[11] = bhk * D * 4;                                   // v_mean
  // adaptive width: per-chunk sums of squares, statistics, chosen widths
  sizes[12] = t;                                             // m2_part
  if (!mul_ok(bhk * 8 + qblk * 2 + kblk, 4, &sizes[13])) return false;   // adapt_stat
  sizes[14] = bhk * 4;                                       // head_bits
  return true;
}

size_t total_bytes(const Dims& d) {
  size_t s[kNumArrays];
  if (!layout(d, s)) return 0;
  size_t tot = 0;
  for (int i = 0; i < kNumArrays; i++) {
    const size_t a = align_up(s[i]);
    if (a < s[i] || tot + a < tot) return 0;
    tot += a;
  }
  return tot;
}

void carve(void* ws, const Dims& d, sage_quant_bufs* out) {
  size_t s[kNumArrays];
  layout(d, s);
  char* p = (char*)ws;
  void** slots[kNumArrays] = {(void**)&out->q_codes, (void**)&out->k_codes, (void**)&out->q_scale,
                              (void**)&out->k_scale, (void**)&out->q_mean,  (void**)&out->k_mean,
                              (void**)&out->v_codes, (void**)&out->v_scale, (void**)&out->delta_s,
                              (void**)&out->k_part,  (void**)&out->v_part,  (void**)&out->v_mean,
                              (void**)&out->m2_part, (void**)&out->adapt_stat, (void**)&out->head_bits};
  for (int i = 0; i < kNumArrays; i++) {
    *slots[i] = p;
    p += align_up(s[i]);
  }
}

// The buffer set of shape d (the adaptive statistics are carved from
// adapt_stat: [B*Hkv][8] per head, [B*Hq*NQB][2] per query block, [B*Hkv*NQBk]
// per key block).
Bufs to_internal(const sage_quant_bufs& q, const Dims& d) {
  Bufs b = {};
  b.q_codes = q.q_codes;
  b.k_codes = q.k_codes;
  b.q_scale = q.q_scale;
  b.k_scale = q.k_scale;
  b.q_mean = q.q_mean;
  b.k_mean = q.k_mean;
  b.v_codes = q.v_codes;
  b.v_scale = q.v_scale;
  b.delta_s = q.delta_s;
  b.k_part = q.k_part;
  b.v_part = q.v_part;
  b.v_mean = q.v_mean;
  b.m2_part = q.m2_part;
  b.stat_head = q.adapt_stat;
  b.stat_qblk = q.adapt_stat + (size_t)d.BHk() * 8;
  b.stat_kblk = b.stat_qblk + (size_t)d.BH() * d.NQB * 2;
  b.head_bits = q.head_bits;
  return b;
}

// 16-byte boundary: the kernels read inputs, codes and workspace arrays in
// 16-byte pieces
bool a16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool a16(const void* a, const void* b, const void* c) { return a16(a) && a16(b) && a16(c); }

bool bufs_ok(const sage_quant_bufs* q) {
  return q && q->q_codes && q->k_codes && q->q_scale && q->k_scale && q->q_mean && q->k_mean && q->v_codes &&
         q->v_scale && q->delta_s && q->k_part && q->v_part && q->v_mean && q->m2_part && q->adapt_stat &&
         q->head_bits && a16(q->q_codes, q->k_codes, q->q_scale) && a16(q->k_scale, q->q_mean, q->k_mean) &&
         a16(q->v_codes, q->v_scale, q->delta_s) && a16(q->k_part, q->v_part, q->v_mean) &&
         a16(q->m2_part, q->adapt_stat, q->head_bits);
}

// gfx950 check, cached once per device.
std::once_flag g_once[kMaxDevices];
int g_is_gfx950[kMaxDevices];

sage_status device_check() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return SAGE_ERR_HIP;
  if (dev < 0 || dev >= kMaxDevices) return SAGE_ERR_UNSUPPORTED;
  std::call_once(g_once[dev], [dev] {
    hipDeviceProp_t p;
    g_is_gfx950[dev] = (hipGetDeviceProperties(&p, dev) == hipSuccess && std::strncmp(p.gcnArchName, "gfx950", 6) == 0)
                           ? 1
                           : 0;
  });
  return g_is_gfx950[dev] ? SAGE_OK : SAGE_ERR_UNSUPPORTED;
}

bool ranges_overlap(const void* a, size_t na, const void* b, size_t nb) {
  const char* pa = (const char*)a;
  const char* pb = (const char*)b;
  return pa < pb + nb && pb < pa + na;
}

// ---------------------------------------------------------------- decoding --
// Workspace of a decoding step: K/V statistics (k_part, v_part, k_mean,
// v_scale, v_mean) and the per-range partial outputs.
constexpr int kDecodeArrays = 7;

bool split_ok(int split_keys) { return split_keys >= 0 && split_keys % 128 == 0; }

// The decoding kernel addresses one head's keys with 31-bit byte offsets.
bool decode_shape_ok(int B, int Hq, int Hkv, int Nk, int D) {
  return shape_ok(B, Hq, Hkv, 1, Nk, D) && (long long)Nk * D * 2 < (1LL << 31);
}

// MI355X compute units: the default key ranges aim at one round of
// workgroups, the fewest ranges that still fill the chip (measured, B16 Hq32
// Hkv8 Nk8192 D128 decoding: 153 us per step with one round of 256
// workgroups, 159 with two, 165 with four; chunked prefill Hq32 Hkv8 Nq512
// Nk8192 through the split path: 116 us with one round of 512, 128 with two).
constexpr int kComputeUnits = 256;

int default_split_keys(const Dims& d) {
  const int g = d.H / d.Hk, hg = sage::decode_heads_per_group(g);
  const long long wgy = (long long)d.BHk() * ((g + hg - 1) / hg);
  // about one 8-wave workgroup per compute unit, at least one block per range
  long long S = (kComputeUnits + wgy - 1) / wgy;
  if (S > d.NQBk) S = d.NQBk;
  if (S < 1) S = 1;
  return 128 * (int)((d.NQBk + S - 1) / S);
}

bool decode_layout(const Dims& d, int split_keys, size_t sizes[kDecodeArrays]) {
  const size_t D = (size_t)d.D, bhk = (size_t)d.BHk(), bhq = (size_t)d.BH();
  const size_t S = ((size_t)d.Nk + split_keys - 1) / split_keys;
  size_t t;
  if (!mul_ok(bhk * (size_t)d.NQBk, 2 * D * 4, &sizes[0])) return false;   // k_part
  sizes[1] = sizes[0];                                                     // v_part
  sizes[2] = sizes[3] = sizes[4] = bhk * D * 4;                            // k_mean, v_scale, v_mean
  if (!mul_ok(bhq * S, D * 4, &sizes[5])) return false;                    // part_o
  if (!mul_ok(bhq * S, 8, &t)) return false;                               // part_ml
  sizes[6] = t;
  return true;
}

size_t decode_total(const Dims& d, int split_keys) {
  size_t s[kDecodeArrays];
  if (!decode_layout(d, split_keys, s)) return 0;
  size_t tot = 0;
  for (int i = 0; i < kDecodeArrays; i++) {
    const size_t a = align_up(s[i]);
    if (a < s[i] || tot + a < tot) return 0;
    tot += a;
  }
  return tot;
}

// ------------------------------------------------- split key ranges (fused) --
int default_split_fused(const Dims& d) {
  // about two workgroups per compute unit (one round)
  const long long wg = (long long)d.NQB * d.BH();
  long long S = (2 * kComputeUnits + wg - 1) / wg;
  if (S > d.NQBk) S = d.NQBk;
  if (S < 1) S = 1;
  return 128 * (int)((d.NQBk + S - 1) / S);
}

// Partial-state arrays after the prepass buffers: O [B*H*N, S, D] and (m, l')
// [B*H*N, S, 2], fp32.
bool split_sizes(const Dims& d, int split_keys, size_t* o_bytes, size_t* ml_bytes) {
  const size_t S = ((size_t)d.Nk + split_keys - 1) / split_keys;
  const size_t rows = (size_t)d.BH() * d.N;
  if ((long long)d.NQB * d.BH() * (long long)S >= (1LL << 31) || rows >= (1ULL << 31)) return false;
  size_t t;
  if (!mul_ok(rows * S, (size_t)d.D * 4, o_bytes) || !mul_ok(rows * S, 8, &t)) return false;
  *ml_bytes = t;
  return true;
}

size_t split_total(const Dims& d, int split_keys) {
  size_t ob, mb;
  const size_t base = total_bytes(d);
  if (base == 0 || !split_sizes(d, split_keys, &ob, &mb)) return 0;
  const size_t tot = base + align_up(ob) + align_up(mb);
  return tot < base ? 0 : tot;
}

}  // namespace

extern "C" {

int sage_contract_version(void) { return sage::kContractVersion; }

const char* sage_status_string(sage_status st) {
  switch (st) {
    case SAGE_OK: return "SAGE_OK";
    case SAGE_ERR_INVALID: return "SAGE_ERR_INVALID: invalid argument";
    case SAGE_ERR_UNSUPPORTED: return "SAGE_ERR_UNSUPPORTED: device is not gfx950";
    case SAGE_ERR_WORKSPACE: return "SAGE_ERR_WORKSPACE: workspace too small";
    case SAGE_ERR_HIP: return "SAGE_ERR_HIP: HIP runtime or launch failure";
  }
  return "unknown sage_status";
}

size_t sage_workspace_bytes_cross(int B, int Hq, int Hkv, int Nq, int Nk, int D) {
  if (!shape_ok(B, Hq, Hkv, Nq, Nk, D)) return 0;
  return total_bytes(make_dims(B, Hq, Hkv, Nq, Nk, D));
}

sage_status sage_quant_bufs_from_workspace_cross(void* ws, size_t bytes, int B, int Hq, int Hkv, int Nq, int Nk,
                                                 int D, sage_quant_bufs* out) {
  if (!ws || !out || !a16(ws) || !shape_ok(B, Hq, Hkv, Nq, Nk, D)) return SAGE_ERR_INVALID;
  const Dims d = make_dims(B, Hq, Hkv, Nq, Nk, D);
  const size_t need = total_bytes(d);
  if (need == 0) return SAGE_ERR_INVALID;
  if (bytes < need) return SAGE_ERR_WORKSPACE;
  carve(ws, d, out);
  return SAGE_OK;
}

}  // extern "C"

namespace {
// The prepass into caller buffers; qk_bits 0 (adaptive width) uses sm_scale.
sage_status quant_smooth_impl(const void* q, const void* k, const void* v, sage_dtype in_dtype, int B, int Hq,
                              int Hkv, int Nq, int Nk, int D, int qk_bits, float sm_scale, int smooth_v,
                              const sage_quant_bufs* out, hipStream_t stream) {
  if (!q || !k || !v || !a16(q, k, v) || !bufs_ok(out) || !shape_ok(B, Hq, Hkv, Nq, Nk, D) || !bits_ok_ad(qk_bits))
    return SAGE_ERR_INVALID;
  if (smooth_v != 0 && smooth_v != 1) return SAGE_ERR_INVALID;
  if (in_dtype != SAGE_F16 && in_dtype != SAGE_BF16) return SAGE_ERR_INVALID;
  if (qk_bits == 0 && (!std::isfinite(sm_scale) || !(sm_scale > 0.0f))) return SAGE_ERR_INVALID;
  const Dims d = make_dims(B, Hq, Hkv, Nq, Nk, D, qk_bits, smooth_v, sm_scale);
  if (total_bytes(d) == 0) return SAGE_ERR_INVALID;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  const hipError_t e = sage::launch_prepass(q, k, v, (int)in_dtype, d, to_internal(*out, d), stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}
}  // namespace

extern "C" {

sage_status sage_quant_smooth_cross(const void* q, const void* k, const void* v, sage_dtype in_dtype, int B, int Hq,
                                    int Hkv, int Nq, int Nk, int D, int qk_bits, int smooth_v,
                                    const sage_quant_bufs* out, hipStream_t stream) {
  if (!bits_ok(qk_bits)) return SAGE_ERR_INVALID;
  return quant_smooth_impl(q, k, v, in_dtype, B, Hq, Hkv, Nq, Nk, D, qk_bits, 0.0f, smooth_v, out, stream);
}

sage_status sage_quant_smooth_adaptive_cross(const void* q, const void* k, const void* v, sage_dtype in_dtype, int B,
                                             int Hq, int Hkv, int Nq, int Nk, int D, float sm_scale, int smooth_v,
                                             const sage_quant_bufs* out, hipStream_t stream) {
  return quant_smooth_impl(q, k, v, in_dtype, B, Hq, Hkv, Nq, Nk, D, 0, sm_scale, smooth_v, out, stream);
}

sage_status sage_attn_fwd_cross(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Nq,
                                int Nk, int D, int causal, float sm_scale, int qk_bits, int smooth_v,
                                sage_dtype in_dtype, sage_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (!q || !k || !v || !o || !workspace || !a16(q, k, v) || !a16(workspace) || !shape_ok(B, Hq, Hkv, Nq, Nk, D) ||
      !bits_ok_ad(qk_bits))
    return SAGE_ERR_INVALID;
  if (causal && Nq > Nk) return SAGE_ERR_INVALID;
  if (smooth_v != 0 && smooth_v != 1) return SAGE_ERR_INVALID;
  if (in_dtype != SAGE_F16 && in_dtype != SAGE_BF16) return SAGE_ERR_INVALID;
  if (out_dtype != SAGE_F16 && out_dtype != SAGE_BF16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID;
  const Dims d = make_dims(B, Hq, Hkv, Nq, Nk, D, qk_bits, smooth_v, sm_scale);
  const size_t need = total_bytes(d);
  if (need == 0) return SAGE_ERR_INVALID;
  if (workspace_bytes < need) return SAGE_ERR_WORKSPACE;
  size_t qel, kel, obytes, qbytes, kbytes;
  if (!mul_ok((size_t)B * Hq * Nq, (size_t)D, &qel) || !mul_ok((size_t)B * Hkv * Nk, (size_t)D, &kel))
    return SAGE_ERR_INVALID;
  if (!mul_ok(qel, out_dtype == SAGE_F32 ? 4 : 2, &obytes) || !mul_ok(qel, 2, &qbytes) || !mul_ok(kel, 2, &kbytes))
    return SAGE_ERR_INVALID;
  if (ranges_overlap(o, obytes, q, qbytes) || ranges_overlap(o, obytes, k, kbytes) ||
      ranges_overlap(o, obytes, v, kbytes) || ranges_overlap(o, obytes, workspace, need))
    return SAGE_ERR_INVALID;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  sage_quant_bufs qb;
  carve(workspace, d, &qb);
  const Bufs b = to_internal(qb, d);
  const float ks = sm_scale * 1.44269504088896340736f;
  hipError_t e = sage::launch_prepass(q, k, v, (int)in_dtype, d, b, stream);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  e = sage::launch_attn(b, d, causal ? 1 : 0, ks, o, (int)out_dtype, stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

sage_status sage_attn_quantized_cross(const sage_quant_bufs* qb, void* o, int B, int Hq, int Hkv, int Nq, int Nk,
                                      int D, int causal, float sm_scale, int qk_bits, sage_dtype out_dtype,
                                      hipStream_t stream) {
  if (!bufs_ok(qb) || !o || !shape_ok(B, Hq, Hkv, Nq, Nk, D) || !bits_ok_ad(qk_bits)) return SAGE_ERR_INVALID;
  if (causal && Nq > Nk) return SAGE_ERR_INVALID;
  if (out_dtype != SAGE_F16 && out_dtype != SAGE_BF16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID;
  const Dims d = make_dims(B, Hq, Hkv, Nq, Nk, D, qk_bits);
  if (total_bytes(d) == 0) return SAGE_ERR_INVALID;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  const float ks = sm_scale * 1.44269504088896340736f;
  const hipError_t e = sage::launch_attn(to_internal(*qb, d), d, causal ? 1 : 0, ks, o, (int)out_dtype, stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int sage_decode_split_keys(int B, int Hq, int Hkv, int Nk, int D) {
  if (!decode_shape_ok(B, Hq, Hkv, Nk, D)) return 0;
  return default_split_keys(make_dims(B, Hq, Hkv, 1, Nk, D));
}

size_t sage_decode_workspace_bytes(int B, int Hq, int Hkv, int Nk, int D, int split_keys) {
  if (!decode_shape_ok(B, Hq, Hkv, Nk, D) || !split_ok(split_keys)) return 0;
  const Dims d = make_dims(B, Hq, Hkv, 1, Nk, D);
  return decode_total(d, split_keys ? split_keys : default_split_keys(d));
}

sage_status sage_attn_decode(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Nk,
                             int D, float sm_scale, int smooth_v, int split_keys, sage_dtype in_dtype,
                             sage_dtype out_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !workspace || !a16(q, k, v) || !a16(workspace) || !decode_shape_ok(B, Hq, Hkv, Nk, D) ||
      !split_ok(split_keys))
    return SAGE_ERR_INVALID;
  if (smooth_v != 0 && smooth_v != 1) return SAGE_ERR_INVALID;
  if (in_dtype != SAGE_F16 && in_dtype != SAGE_BF16) return SAGE_ERR_INVALID;
  if (out_dtype != SAGE_F16 && out_dtype != SAGE_BF16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID;
  const Dims d = make_dims(B, Hq, Hkv, 1, Nk, D, 4, smooth_v);
  const int sk = split_keys ? split_keys : default_split_keys(d);
  const size_t need = decode_total(d, sk);
  if (need == 0) return SAGE_ERR_INVALID;
  if (workspace_bytes < need) return SAGE_ERR_WORKSPACE;
  size_t qel, kel, obytes, qbytes, kbytes;
  if (!mul_ok((size_t)B * Hq, (size_t)D, &qel) || !mul_ok((size_t)B * Hkv * Nk, (size_t)D, &kel))
    return SAGE_ERR_INVALID;
  if (!mul_ok(qel, out_dtype == SAGE_F32 ? 4 : 2, &obytes) || !mul_ok(qel, 2, &qbytes) || !mul_ok(kel, 2, &kbytes))
    return SAGE_ERR_INVALID;
  if (ranges_overlap(o, obytes, q, qbytes) || ranges_overlap(o, obytes, k, kbytes) ||
      ranges_overlap(o, obytes, v, kbytes) || ranges_overlap(o, obytes, workspace, need))
    return SAGE_ERR_INVALID;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  size_t sz[kDecodeArrays];
  decode_layout(d, sk, sz);
  char* p = (char*)workspace;
  float* arr[kDecodeArrays];
  for (int i = 0; i < kDecodeArrays; i++) {
    arr[i] = (float*)p;
    p += align_up(sz[i]);
  }
  Bufs b = {};
  b.k_part = arr[0];
  b.v_part = arr[1];
  b.k_mean = arr[2];
  b.v_scale = arr[3];
  b.v_mean = arr[4];
  sage::DecodeBufs db;
  db.part_o = arr[5];
  db.part_ml = arr[6];
  db.split_keys = sk;
  const float ks = sm_scale * 1.44269504088896340736f;
  const hipError_t e = sage::launch_decode(q, k, v, (int)in_dtype, d, b, db, ks, o, (int)out_dtype, stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

int sage_split_keys(int B, int Hq, int Hkv, int Nq, int Nk, int D) {
  if (!shape_ok(B, Hq, Hkv, Nq, Nk, D)) return 0;
  return default_split_fused(make_dims(B, Hq, Hkv, Nq, Nk, D));
}

size_t sage_split_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D, int split_keys) {
  if (!shape_ok(B, Hq, Hkv, Nq, Nk, D) || !split_ok(split_keys)) return 0;
  const Dims d = make_dims(B, Hq, Hkv, Nq, Nk, D);
  return split_total(d, split_keys ? split_keys : default_split_fused(d));
}

sage_status sage_attn_fwd_split(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Nq,
                                int Nk, int D, int causal, float sm_scale, int qk_bits, int smooth_v, int split_keys,
                                sage_dtype in_dtype, sage_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                hipStream_t stream) {
  if (!q || !k || !v || !o || !workspace || !a16(q, k, v) || !a16(workspace) || !shape_ok(B, Hq, Hkv, Nq, Nk, D) ||
      !bits_ok_ad(qk_bits) || !split_ok(split_keys))
    return SAGE_ERR_INVALID;
  if (causal && Nq > Nk) return SAGE_ERR_INVALID;
  if (smooth_v != 0 && smooth_v != 1) return SAGE_ERR_INVALID;
  if (in_dtype != SAGE_F16 && in_dtype != SAGE_BF16) return SAGE_ERR_INVALID;
  if (out_dtype != SAGE_F16 && out_dtype != SAGE_BF16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID;
  const Dims d = make_dims(B, Hq, Hkv, Nq, Nk, D, qk_bits, smooth_v, sm_scale);
  const int sk = split_keys ? split_keys : default_split_fused(d);
  const size_t need = split_total(d, sk);
  if (need == 0) return SAGE_ERR_INVALID;
  if (workspace_bytes < need) return SAGE_ERR_WORKSPACE;
  size_t qel, kel, obytes, qbytes, kbytes;
  if (!mul_ok((size_t)B * Hq * Nq, (size_t)D, &qel) || !mul_ok((size_t)B * Hkv * Nk, (size_t)D, &kel))
    return SAGE_ERR_INVALID;
  if (!mul_ok(qel, out_dtype == SAGE_F32 ? 4 : 2, &obytes) || !mul_ok(qel, 2, &qbytes) || !mul_ok(kel, 2, &kbytes))
    return SAGE_ERR_INVALID;
  if (ranges_overlap(o, obytes, q, qbytes) || ranges_overlap(o, obytes, k, kbytes) ||
      ranges_overlap(o, obytes, v, kbytes) || ranges_overlap(o, obytes, workspace, need))
    return SAGE_ERR_INVALID;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  sage_quant_bufs qb;
  carve(workspace, d, &qb);
  const Bufs b = to_internal(qb, d);
  size_t ob, mb;
  split_sizes(d, sk, &ob, &mb);
  char* p = (char*)workspace + total_bytes(d);
  sage::SplitParts sp;
  sp.part_o = (float*)p;
  sp.part_ml = (float*)(p + align_up(ob));
  sp.split_blocks = sk / 128;
  sp.S = (d.NQBk + sp.split_blocks - 1) / sp.split_blocks;
  const float ks = sm_scale * 1.44269504088896340736f;
  hipError_t e = sage::launch_prepass(q, k, v, (int)in_dtype, d, b, stream);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  e = sage::launch_attn_split(b, d, causal ? 1 : 0, ks, o, (int)out_dtype, sp, stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

// Self-attention: the same calls with Hq = Hkv = H and Nq = Nk = N.
size_t sage_workspace_bytes(int B, int H, int N, int D) { return sage_workspace_bytes_cross(B, H, H, N, N, D); }

sage_status sage_quant_bufs_from_workspace(void* ws, size_t bytes, int B, int H, int N, int D, sage_quant_bufs* out) {
  return sage_quant_bufs_from_workspace_cross(ws, bytes, B, H, H, N, N, D, out);
}

sage_status sage_quant_smooth(const void* q, const void* k, const void* v, sage_dtype in_dtype, int B, int H, int N,
                              int D, int qk_bits, int smooth_v, const sage_quant_bufs* out, hipStream_t stream) {
  return sage_quant_smooth_cross(q, k, v, in_dtype, B, H, H, N, N, D, qk_bits, smooth_v, out, stream);
}

sage_status sage_quant_smooth_adaptive(const void* q, const void* k, const void* v, sage_dtype in_dtype, int B, int H,
                                       int N, int D, float sm_scale, int smooth_v, const sage_quant_bufs* out,
                                       hipStream_t stream) {
  return sage_quant_smooth_adaptive_cross(q, k, v, in_dtype, B, H, H, N, N, D, sm_scale, smooth_v, out, stream);
}

sage_status sage_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int D,
                          int causal, float sm_scale, int qk_bits, int smooth_v, sage_dtype in_dtype,
                          sage_dtype out_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream) {
  return sage_attn_fwd_cross(q, k, v, o, B, H, H, N, N, D, causal, sm_scale, qk_bits, smooth_v, in_dtype, out_dtype,
                             workspace, workspace_bytes, stream);
}

sage_status sage_attn_quantized(const sage_quant_bufs* qb, void* o, int B, int H, int N, int D, int causal,
                                float sm_scale, int qk_bits, sage_dtype out_dtype, hipStream_t stream) {
  return sage_attn_quantized_cross(qb, o, B, H, H, N, N, D, causal, sm_scale, qk_bits, out_dtype, stream);
}

sage_status sage_qk_int32_debug(const sage_quant_bufs* qb, int B, int H, int N, int D, int qk_bits, int bh, int q0,
                                int k0, int nq, int nk, int32_t* out, hipStream_t stream) {
  if (!bufs_ok(qb) || !out || !shape_ok(B, H, H, N, N, D) || !bits_ok_ad(qk_bits)) return SAGE_ERR_INVALID;
  if (bh < 0 || bh >= B * H || q0 < 0 || k0 < 0 || nq < 1 || nk < 1) return SAGE_ERR_INVALID;
  if ((long long)q0 + nq > N || (long long)k0 + nk > N) return SAGE_ERR_INVALID;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  const Dims d = make_dims(B, H, H, N, N, D, qk_bits);
  const hipError_t e = sage::launch_qk_debug(to_internal(*qb, d), d, bh, q0, k0, nq, nk, out, stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

// Packed variable-length batches: nseq sequences of at most max_seqlen tokens
// in token-major [T, H, D] tensors, workspace of the dense shape
// (nseq, H, max_seqlen, D).
static bool varlen_ok(const int* cu, int nseq, int max_seqlen, int total, int H, int D) {
  // the prepass grids put the 128-token blocks in the y dimension (<= 65535)
  return cu && total >= 1 && shape_ok(nseq, H, H, max_seqlen, max_seqlen, D) && (max_seqlen + 127) / 128 <= 65535;
}

sage_status sage_quant_smooth_varlen(const void* q, const void* k, const void* v, sage_dtype in_dtype,
                                     const int* cu_seqlens, int nseq, int max_seqlen, int total_tokens, int H, int D,
                                     int qk_bits, int smooth_v, const sage_quant_bufs* out, hipStream_t stream) {
  if (!q || !k || !v || !a16(q, k, v) || !bufs_ok(out) || !varlen_ok(cu_seqlens, nseq, max_seqlen, total_tokens, H, D))
    return SAGE_ERR_INVALID;
  if (!bits_ok(qk_bits) || (smooth_v != 0 && smooth_v != 1)) return SAGE_ERR_INVALID;
  if (in_dtype != SAGE_F16 && in_dtype != SAGE_BF16) return SAGE_ERR_INVALID;
  Dims d = make_dims(nseq, H, H, max_seqlen, max_seqlen, D, qk_bits, smooth_v);
  if (total_bytes(d) == 0) return SAGE_ERR_INVALID;
  d.cu = cu_seqlens;
  d.T = total_tokens;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  const hipError_t e = sage::launch_prepass(q, k, v, (int)in_dtype, d, to_internal(*out, d), stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

sage_status sage_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, const int* cu_seqlens,
                                 int nseq, int max_seqlen, int total_tokens, int H, int D, int causal, float sm_scale,
                                 int qk_bits, int smooth_v, sage_dtype in_dtype, sage_dtype out_dtype,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream) {
  if (!q || !k || !v || !o || !workspace || !a16(q, k, v) || !a16(workspace) ||
      !varlen_ok(cu_seqlens, nseq, max_seqlen, total_tokens, H, D))
    return SAGE_ERR_INVALID;
  if (!bits_ok(qk_bits) || (smooth_v != 0 && smooth_v != 1)) return SAGE_ERR_INVALID;
  if (in_dtype != SAGE_F16 && in_dtype != SAGE_BF16) return SAGE_ERR_INVALID;
  if (out_dtype != SAGE_F16 && out_dtype != SAGE_BF16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID;
  Dims d = make_dims(nseq, H, H, max_seqlen, max_seqlen, D, qk_bits, smooth_v);
  const size_t need = total_bytes(d);
  if (need == 0) return SAGE_ERR_INVALID;
  if (workspace_bytes < need) return SAGE_ERR_WORKSPACE;
  size_t elems, obytes, ibytes;
  if (!mul_ok((size_t)total_tokens * H, (size_t)D, &elems)) return SAGE_ERR_INVALID;
  if (!mul_ok(elems, out_dtype == SAGE_F32 ? 4 : 2, &obytes) || !mul_ok(elems, 2, &ibytes)) return SAGE_ERR_INVALID;
  if (ranges_overlap(o, obytes, q, ibytes) || ranges_overlap(o, obytes, k, ibytes) ||
      ranges_overlap(o, obytes, v, ibytes) || ranges_overlap(o, obytes, workspace, need))
    return SAGE_ERR_INVALID;
  d.cu = cu_seqlens;
  d.T = total_tokens;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  sage_quant_bufs qb;
  carve(workspace, d, &qb);
  const Bufs b = to_internal(qb, d);
  const float ks = sm_scale * 1.44269504088896340736f;
  hipError_t e = sage::launch_prepass(q, k, v, (int)in_dtype, d, b, stream);
  if (e != hipSuccess) return SAGE_ERR_HIP;
  e = sage::launch_attn(b, d, causal ? 1 : 0, ks, o, (int)out_dtype, stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

sage_status sage_attn_quantized_varlen(const sage_quant_bufs* qb, void* o, const int* cu_seqlens, int nseq,
                                       int max_seqlen, int total_tokens, int H, int D, int causal, float sm_scale,
                                       int qk_bits, sage_dtype out_dtype, hipStream_t stream) {
  if (!bufs_ok(qb) || !o || !varlen_ok(cu_seqlens, nseq, max_seqlen, total_tokens, H, D) || !bits_ok(qk_bits))
    return SAGE_ERR_INVALID;
  if (out_dtype != SAGE_F16 && out_dtype != SAGE_BF16 && out_dtype != SAGE_F32) return SAGE_ERR_INVALID;
  if (!std::isfinite(sm_scale) || !(sm_scale > 0.0f)) return SAGE_ERR_INVALID;
  Dims d = make_dims(nseq, H, H, max_seqlen, max_seqlen, D, qk_bits);
  if (total_bytes(d) == 0) return SAGE_ERR_INVALID;
  d.cu = cu_seqlens;
  d.T = total_tokens;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  const float ks = sm_scale * 1.44269504088896340736f;
  const hipError_t e = sage::launch_attn(to_internal(*qb, d), d, causal ? 1 : 0, ks, o, (int)out_dtype, stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

sage_status sage_fp8_encode_debug(const float* in, uint8_t* out, size_t n, hipStream_t stream) {
  if (!in || !out || n == 0 || n > ((size_t)1 << 40)) return SAGE_ERR_INVALID;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  const hipError_t e = sage::launch_fp8_encode(in, out, n, stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

sage_status sage_fp8_mfma_debug(const uint8_t* a, const uint8_t* b, const float* c, float* d, hipStream_t stream) {
  if (!a || !b || !c || !d) return SAGE_ERR_INVALID;
  const sage_status dc = device_check();
  if (dc != SAGE_OK) return dc;
  const hipError_t e = sage::launch_fp8_mfma_debug(a, b, c, d, stream);
  return e == hipSuccess ? SAGE_OK : SAGE_ERR_HIP;
}

}  // extern "C"
