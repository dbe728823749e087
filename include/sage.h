/*
 * sage.h -- C ABI of libsage: the SageAttention2 quantized attention forward
 * pass for AMD Instinct MI355X (gfx950).
 *
 * The method is the one of "SageAttention2: Efficient Attention with Thorough
 * Outlier Smoothing and Per-thread INT4 Quantization" (arXiv 2411.10958,
 * abstract page): Q and K are smoothed and quantized to INT4 with fine-grained
 * scales, S = QK^T is computed in integer arithmetic and dequantized, an online
 * softmax produces P~, and P~ and V are quantized to FP8 with a two-level
 * accumulation of P~V.  The "SageAttention2 Technical Report" summary page
 * (Key Contributions 1-2) describes the same INT4 QK / FP8 P~V split.
 *
 * Conventions for every entry point
 *  - Tensors are contiguous, row-major [B, H, N, D] device buffers (self
 *    attention: queries and keys share N).  D must be 64 or 128; B, H, N >= 1.
 *  - q, k, v and workspaces start on a 16-byte boundary (the
 *    kernels read them in 16-byte pieces), as do the arrays of a
 *    sage_quant_bufs; otherwise the call returns SAGE_ERR_INVALID.  Outputs
 *    may start anywhere (a misaligned one is written element by element).
 *  - Every buffer is owned by the caller.  The library allocates no device
 *    memory, keeps no pointer after returning and holds no mutable state
 *    (the gfx950 check is cached once per device).
 *  - Work is enqueued on `stream` (NULL = the default stream) and the call
 *    returns without synchronising; results are valid after the stream is.
 *  - Arguments are validated before anything is launched; on error nothing is
 *    written.  Launch failures return SAGE_ERR_HIP; faults inside a kernel
 *    surface at the caller's next synchronisation.
 *  - Results are deterministic: the same inputs give bit-identical outputs.
 *  - Contract constants (they fix the method's rounding; any change bumps
 *    sage_contract_version): Q-smoothing block and mean chunk = 128 tokens;
 *    online-softmax block = 128 keys (also the level-1 block of the two-level
 *    P~V accumulation); K scale groups of 16 keys (two per 32-key tile).
 *  - qk_bits selects the width of the Q and K codes: 4 (INT4 in [-7, 7], the
 *    method's default) or 8 (INT8 in [-127, 127], the more accurate choice
 *    the adaptive quantization of SageAttention2 (summary page, Key
 *    Contribution 3) falls back to where INT4 loses accuracy; same
 *    granularity, scale = amax/qmax), or 0 where an entry point says so: the
 *    adaptive width.  Any other value is SAGE_ERR_INVALID.  Buffers written
 *    with one qk_bits must be read with the same value (0 and 8 share the
 *    8-bit layout).
 *  - Adaptive width (qk_bits 0).  The summary page names an adaptive
 *    quantization that keeps end-to-end metrics but does not define it.
 *    Here, per key/value head (with its query heads), the prepass predicts
 *    the variance INT4 codes add to the softmax logits, modelling a code
 *    error as uniform over half a step (delta = amax/7):
 *      sigma^2 = sm_scale^2/12 * (mean amax_q^2/49 * mean |K - kmean|^2
 *                                 + mean amax_k^2/49 * mean |Q - qmean|^2),
 *    and weights it by rho = E|V - vmean|^2 / (E|V - vmean|^2 + |vmean|^2)
 *    (the cosine loss of O is about sigma^2 * rho / 2 when attention falls
 *    on one key).  The head gets INT4 codes (values in [-7, 7], scale
 *    amax/7) iff sigma^2 * rho <= 0.02, else INT8; both are stored in the
 *    8-bit layout and multiplied on the INT8 matrix core, so one launch
 *    serves heads of both widths.  The statistics are fp32 sums in a fixed
 *    order (see head_bits / adapt_stat below), the comparison is in fp64;
 *    the choice is deterministic.  Supported by the dense entry points
 *    (self-attention, cross-attention, grouped heads, split key ranges), not
 *    by packed sequences or the decoding step.
 *  - smooth_v (0 or 1): smooth V before its FP8 quantization by subtracting
 *    the per-channel mean over all N tokens, added back to O in the epilogue
 *    (the smoothing of Q and V of the technical-report summary, Key
 *    Contribution 2; exact for unquantized softmax, whose rows sum to one).
 */
#ifndef SAGE_H_
#define SAGE_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  SAGE_OK = 0,
  SAGE_ERR_INVALID = -1,      /* null pointer, bad size, bad dtype, bad sm_scale, overflow */
  SAGE_ERR_UNSUPPORTED = -2,  /* current device is not gfx950                               */
  SAGE_ERR_WORKSPACE = -3,    /* workspace smaller than sage_workspace_bytes()              */
  SAGE_ERR_HIP = -4           /* a HIP runtime call or kernel launch failed                 */
} sage_status;

typedef enum { SAGE_F16 = 0, SAGE_BF16 = 1, SAGE_F32 = 2 } sage_dtype;

/*
 * Device buffers written by sage_quant_smooth (and by the prepass inside
 * sage_attn_fwd).  NP = N rounded up to a multiple of 128, NQB = NP / 128.
 * Rows or keys at index >= N are padding: codes 0, scales 0, V bytes 0.
 *
 *  q_codes, k_codes  uint8, B*H*NP*D bytes reserved (the INT8 size); a head
 *                    starts at byte (b*H + h) * NP * RB with RB the row bytes
 *                    qk_bits 8: int8 [NP][D], codes in [-127,127], RB = D.
 *                    qk_bits 4: INT4 codes in [-7,7] stored as OCP FP6 e2m3
 *                    bit patterns (magnitudes 0..7 -> 0,8,16,20,24,26,28,30;
 *                    sign in bit 5), grouped in tiles of 32 rows.  Tile t of
 *                    a head is 64 chunks of LB bytes (LB = 48 for D = 128, 32
 *                    for D = 64; RB = 2*LB): chunk 32*h + (r % 32) of tile
 *                    r / 32 holds, for m < D/64, a 24-byte group with the
 *                    codes of row r, channels 64m + 32h + i (i < 32), as
 *                    6-bit fields starting at bit 6i (little endian).  D = 64:
 *                    bytes 24-31 of a chunk are zero, and the two 16-byte
 *                    halves of chunk c are stored swapped when (c >> 3) & 1.
 *  q_scale           fp32  [B,H,NP]      one scale per token (amax/7 or
 *                    amax/127)
 *  k_scale           fp32  [B,H,NP/16]   one scale per 16-key group; in a
 *                    32-key tile starting at key 32u, group 2u+h holds the keys
 *                    32u + o with (o/4) % 2 == h
 *  q_mean            fp32  [B,H,NQB,D]   per-block Q channel means (tail block
 *                    averages its valid tokens only)
 *  k_mean            fp32  [B,H,D]       K channel means over all N tokens
 *  v_codes           uint8 [B,H,NQB,D,128] OCP e4m3fn codes of (V - v_mean)/v_scale,
 *                    channel-major per 128-key block; position p of a block
 *                    holds key 64(p/64) + 32(s/16) + 8((s%16)/4) + 4((p%64)/32)
 *                    + s%4 with s = p%32
 *  v_scale           fp32  [B,H,D]       per-channel scale (max|V - v_mean|/448)
 *  delta_s           fp32  [B,H,NQB,NP]  compensation term
 *                    DeltaS[qb][j] = q_mean[qb] . (K[j] - k_mean), fp32
 *                    accumulation (not scaled by sm_scale)
 *  k_part, v_part    fp32  [B,H,NQB,2,D] scratch: per-chunk K and V sums, V
 *                    maxima and minima, later reused for bf16 pieces of q_mean
 *  v_mean            fp32  [B,H,D]       V channel means over all N tokens with
 *                    smooth_v, zeros without; added to O by the fused kernel
 *  m2_part           fp32  [B,H,NQB,2,D] scratch (adaptive width): per-chunk K
 *                    and V sums of squares
 *  adapt_stat        fp32  [B*H*8 + B*H*NQB*2 + B*H*NQB] (adaptive width):
 *                    first [B,H,8]: per head A_Q, E_Q, A_K, E_K, EV, V2, -, -
 *                    (A_Q: sum over tokens of amax^2 of the smoothed query,
 *                    summed per 128-token block in token order, then over
 *                    blocks in order; E_Q: per block the sum over channels
 *                    of max(0, SSQ - SQ * qmean) with SQ, SSQ the block's
 *                    sequential sums of Q and Q^2, over blocks in order; A_K:
 *                    per 128-key block the sum in key order of the key's
 *                    group amax^2, over blocks in order; E_K, EV: sums over
 *                    channels of max(0, SS - S * mean) with S, SS the chunked
 *                    sums of K, V and K^2, V^2 and mean = S/N; V2: sum over
 *                    channels of S_V * vmean), then scratch
 *  head_bits         int32 [B,H]         code width chosen per head (4 or 8),
 *                    written by the adaptive width
 * For grouped or cross-attention shapes the key/value-side arrays (k_*,
 * v_*, m2_part, head_bits, the per-head statistics) use Hkv and Nk.
 */
typedef struct {
  uint8_t* q_codes;
  uint8_t* k_codes;
  float* q_scale;
  float* k_scale;
  float* q_mean;
  float* k_mean;
  uint8_t* v_codes;
  float* v_scale;
  float* delta_s;
  float* k_part;
  float* v_part;
  float* v_mean;
  float* m2_part;
  float* adapt_stat;
  int32_t* head_bits;
} sage_quant_bufs;

/* Version of the contract constants above (2 = 128/128/16 blocks and groups,
 * the adaptive width rule above, this sage_quant_bufs layout). */
int sage_contract_version(void);

/* Human-readable name of a status code (static storage). */
const char* sage_status_string(sage_status st);

/*
 * Bytes of device workspace sage_attn_fwd needs for this shape (all
 * sage_quant_bufs arrays, each 256-byte aligned).  Returns 0 for an invalid
 * shape or on size_t overflow.
 */
size_t sage_workspace_bytes(int B, int H, int N, int D);

/*
 * Host-only pointer carving: fill *out with the sage_quant_bufs layout inside
 * a workspace of `bytes` bytes at device address `ws`.  Touches no device.
 * Errors: SAGE_ERR_INVALID (null pointers, bad shape), SAGE_ERR_WORKSPACE.
 */
sage_status sage_quant_bufs_from_workspace(void* ws, size_t bytes, int B, int H, int N, int D,
                                           sage_quant_bufs* out);

/*
 * Prepass (smoothing, INT4/INT8 Q/K quantization and packing, FP8 V with
 * per-channel scales, compensation term): the smoothing of the method and
 * the quantization of Q, K to INT4 and V to FP8 (SageAttention2 abstract).
 * q, k, v: device [B,H,N,D] of in_dtype (SAGE_F16 or SAGE_BF16); qk_bits 4 or
 * 8; smooth_v 0 or 1.  All arrays of *out must be device buffers of the sizes
 * listed above (for example carved by sage_quant_bufs_from_workspace).
 */
sage_status sage_quant_smooth(const void* q, const void* k, const void* v, sage_dtype in_dtype, int B, int H,
                              int N, int D, int qk_bits, int smooth_v, const sage_quant_bufs* out,
                              hipStream_t stream);

/*
 * The prepass with the adaptive width (qk_bits 0 above): the per-head
 * choice needs the softmax scale sm_scale (> 0, finite).  Writes the code
 * arrays in the 8-bit layout, the scales of each head's width, head_bits and
 * the statistics of adapt_stat.  Read the buffers with qk_bits 0 (or 8).
 */
sage_status sage_quant_smooth_adaptive(const void* q, const void* k, const void* v, sage_dtype in_dtype, int B, int H,
                                       int N, int D, float sm_scale, int smooth_v, const sage_quant_bufs* out,
                                       hipStream_t stream);

/*
 * Attention forward: O = SageAttention2(Q, K, V), i.e. the prepass above
 * followed by the fused kernel (INT4 QK^T on the FP6 matrix core, exact,
 * dequantization with the compensation term, online softmax over 128-key
 * blocks, FP8 P~ and V on the FP8 matrix core with two-level accumulation).
 *  q, k, v   device [B,H,N,D] of in_dtype (SAGE_F16 / SAGE_BF16)
 *  o         device [B,H,N,D] of out_dtype (SAGE_F16 / SAGE_BF16 / SAGE_F32);
 *            must not alias q, k, v or the workspace
 *  causal    nonzero: query i attends to keys j <= i
 *  sm_scale  softmax scale (> 0, finite), usually 1/sqrt(D)
 *  qk_bits   4 (INT4 Q/K codes), 8 (INT8) or 0 (adaptive width per head)
 *  smooth_v  1: subtract the V channel means before FP8, add them to O
 *  workspace device buffer of at least sage_workspace_bytes(B,H,N,D) bytes;
 *            afterwards it holds the sage_quant_bufs of this call
 * Equivalent to sage_quant_smooth followed by sage_attn_quantized.
 */
sage_status sage_attn_fwd(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int D,
                          int causal, float sm_scale, int qk_bits, int smooth_v, sage_dtype in_dtype,
                          sage_dtype out_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * sage_attn_fwd without a workspace argument.  The prepass buffers live in a
 * fixed device array of SAGE_STATIC_SCRATCH_BYTES that the library holds on
 * every GPU it runs on until the process ends; the call allocates nothing.
 * Shapes whose sage_workspace_bytes exceeds the array return
 * SAGE_ERR_WORKSPACE (128 MiB: for example B1 H16 N8192 D128 fits, B1 H16
 * N16384 D128 does not).  All calls on one GPU share its array and it keeps
 * the last call's buffers: calls that overlap on one GPU (several streams or
 * threads) race.  Other arguments, results and errors as for sage_attn_fwd.
 */
#define SAGE_STATIC_SCRATCH_BYTES ((size_t)128 << 20)
sage_status sage_attn_fwd_static(const void* q, const void* k, const void* v, void* o, int B, int H, int N, int D,
                                 int causal, float sm_scale, int qk_bits, int smooth_v, sage_dtype in_dtype,
                                 sage_dtype out_dtype, hipStream_t stream);

/*
 * The fused attention kernel alone, over prepass buffers already written by
 * sage_quant_smooth (or by an earlier sage_attn_fwd): INT4 QK^T,
 * dequantization with the compensation term, online softmax, FP8 P~V with
 * two-level accumulation (SageAttention2 abstract).  Arguments as for
 * sage_attn_fwd; qb must describe buffers of this B, H, N, D written with
 * this qk_bits (v_mean, written by the prepass, carries the V smoothing).
 */
sage_status sage_attn_quantized(const sage_quant_bufs* qb, void* o, int B, int H, int N, int D, int causal,
                                float sm_scale, int qk_bits, sage_dtype out_dtype, hipStream_t stream);

/*
 * Separate query and key/value geometry: cross-attention, decoding or chunked
 * prefill against a key/value cache (Nq != Nk), and grouped-query / multi-
 * query heads (Hq = g * Hkv).  The pages define the method for one attention
 * call; these calls apply it unchanged to
 *  q, o     [B, Hq, Nq, D]     k, v   [B, Hkv, Nk, D]
 * with Hq a multiple of Hkv: query head h attends K/V head h / (Hq / Hkv).
 * Smoothing statistics follow the tensors they describe: Q block means over
 * the query tokens of each query head; the K mean, K scale groups, V scales
 * and V mean over the Nk tokens of each K/V head; DeltaS per (query block,
 * key).  Causal: the mask is aligned at the bottom-right corner, query i
 * attends key j iff j <= i + (Nk - Nq) (the last query sees every key), and
 * causal calls require Nq <= Nk (SAGE_ERR_INVALID otherwise).
 * The buffers of sage_quant_bufs take the query-side shapes with (Hq, Nq):
 * q_codes, q_scale, q_mean, and delta_s [B,Hq,NQB,NPk]; the key/value-side
 * ones with (Hkv, Nk): k_codes, k_scale, k_mean, v_codes, v_scale, v_mean
 * (NPk = Nk rounded up to 128).  Size the workspace with
 * sage_workspace_bytes_cross.  With Hq = Hkv = H and Nq = Nk = N every call
 * below is the self-attention call above (the same layout and results).
 * Limits: B*Hq <= 65535; Nq and Nk rounded up to 128 at most 2^23; and
 * (Nq rounded up to 128) / 128 * (Nk rounded up to 128) below 2^30 (the
 * DeltaS rows of one query head: self-attention N up to ~370k tokens).
 * qk_bits 0 (adaptive width) is accepted by sage_attn_fwd_cross,
 * sage_attn_quantized_cross (the 8-bit layout) and sage_attn_fwd_split;
 * sage_quant_smooth_cross takes 4 or 8, sage_quant_smooth_adaptive_cross the
 * adaptive width.
 */
size_t sage_workspace_bytes_cross(int B, int Hq, int Hkv, int Nq, int Nk, int D);

sage_status sage_quant_bufs_from_workspace_cross(void* ws, size_t bytes, int B, int Hq, int Hkv, int Nq, int Nk,
                                                 int D, sage_quant_bufs* out);

sage_status sage_quant_smooth_cross(const void* q, const void* k, const void* v, sage_dtype in_dtype, int B, int Hq,
                                    int Hkv, int Nq, int Nk, int D, int qk_bits, int smooth_v,
                                    const sage_quant_bufs* out, hipStream_t stream);

/* The adaptive-width prepass of this geometry: one width per K/V head, its
 * statistics pooling the query heads of its group (head order). */
sage_status sage_quant_smooth_adaptive_cross(const void* q, const void* k, const void* v, sage_dtype in_dtype, int B,
                                             int Hq, int Hkv, int Nq, int Nk, int D, float sm_scale, int smooth_v,
                                             const sage_quant_bufs* out, hipStream_t stream);

sage_status sage_attn_fwd_cross(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Nq,
                                int Nk, int D, int causal, float sm_scale, int qk_bits, int smooth_v,
                                sage_dtype in_dtype, sage_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

sage_status sage_attn_quantized_cross(const sage_quant_bufs* qb, void* o, int B, int Hq, int Hkv, int Nq, int Nk,
                                      int D, int causal, float sm_scale, int qk_bits, sage_dtype out_dtype,
                                      hipStream_t stream);

/*
 * The full call with split key ranges, for shapes with few 128-query blocks
 * per head (a prefill chunk against a long cache, cross-attention with few
 * queries), where one workgroup per query block leaves the chip idle.
 * Arguments, geometry and errors as for sage_attn_fwd_cross, plus
 * split_keys: keys per range (a non-negative multiple of 128; 0 selects
 * sage_split_keys).  Each (query block, key range) is processed by its own
 * workgroup running the method over that range from an empty state (its own
 * running maximum scales its P~ before the FP8 rounding); a merge then
 * combines, for each query, the ranges holding a key it sees, in order, with
 * weights exp2(m_r - M) (M the largest range maximum) and applies the
 * epilogue.  One range covering every key gives sage_attn_fwd_cross's result
 * bit for bit; more ranges change the FP8 rounding of P~ only.
 * workspace: at least sage_split_workspace_bytes(...) bytes: the
 * sage_quant_bufs of the cross geometry first (as written by the prepass, the
 * layout of sage_quant_bufs_from_workspace_cross), then scratch for the range
 * states (contents unspecified afterwards).
 */
int sage_split_keys(int B, int Hq, int Hkv, int Nq, int Nk, int D);

size_t sage_split_workspace_bytes(int B, int Hq, int Hkv, int Nq, int Nk, int D, int split_keys);

sage_status sage_attn_fwd_split(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Nq,
                                int Nk, int D, int causal, float sm_scale, int qk_bits, int smooth_v, int split_keys,
                                sage_dtype in_dtype, sage_dtype out_dtype, void* workspace, size_t workspace_bytes,
                                hipStream_t stream);

/*
 * Decoding step: one query token per sequence and query head against Nk
 * cached keys and values (q [B, Hq, 1, D], k and v [B, Hkv, Nk, D], o
 * [B, Hq, 1, D]; Hq a multiple of Hkv; no causal flag: the single query sees
 * every key under the bottom-right alignment above).
 * The method is unchanged; with one query token its smoothing block holds
 * that token alone, so the smoothed query is zero, the Q codes and scale are
 * zero for either code width (no qk_bits argument) and the score of key j is
 * the compensation term q . (K_j - mean K) alone.  Its second part is one
 * constant per query head, which the softmax does not see (the invariance
 * behind smoothing K), so this call scores q . K_j in fp32 from the 16-bit
 * keys with no K mean and skips the key codes: it computes the V statistics
 * of the prepass (V mean with smooth_v, V scales), then the scores and the
 * FP8 V codes of the method on the fly, reading K once and V twice in all and
 * writing no codes.  The result equals the method's up to fp32 rounding.
 * Key blocks are processed in ranges of split_keys keys (a multiple of 128;
 * 0 selects sage_decode_split_keys), each range with its own online softmax
 * (its own running maximum scales its P~ before the FP8 rounding), merged at
 * the end with weights exp2(m_s - M) in range order.  The result is that of
 * the method under this schedule; it differs from sage_attn_fwd_cross on the
 * same inputs by the FP8 rounding of P~ (one range covering every key gives
 * the plain schedule).
 * workspace: at least sage_decode_workspace_bytes(B, Hq, Hkv, Nk, D,
 * split_keys) bytes, scratch for the call (its contents are unspecified
 * afterwards).  Errors as for sage_attn_fwd; split_keys not a non-negative
 * multiple of 128, or Nk * D * 2 >= 2^31 (one head's keys), is
 * SAGE_ERR_INVALID.
 */
int sage_decode_split_keys(int B, int Hq, int Hkv, int Nk, int D);

size_t sage_decode_workspace_bytes(int B, int Hq, int Hkv, int Nk, int D, int split_keys);

sage_status sage_attn_decode(const void* q, const void* k, const void* v, void* o, int B, int Hq, int Hkv, int Nk,
                             int D, float sm_scale, int smooth_v, int split_keys, sage_dtype in_dtype,
                             sage_dtype out_dtype, void* workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Packed variable-length batches (the varlen form of the drop-in call; the
 * code record of the SageAttention2 paper names `sageattn_varlen`).  nseq
 * independent self-attention problems share one launch:
 *  q, k, v, o   token-major [T, H, D] with T = total_tokens; sequence s owns
 *               tokens cu_seqlens[s] .. cu_seqlens[s+1]-1 of every head
 *  cu_seqlens   DEVICE int32 [nseq+1], non-decreasing, cu_seqlens[0] = 0,
 *               cu_seqlens[nseq] <= T, every length <= max_seqlen.  It is read
 *               only by the kernels: lengths are clamped to [0, max_seqlen]
 *               and to the tensor, so malformed offsets give wrong results
 *               but no access outside the buffers.  Empty sequences are
 *               allowed.
 *  max_seqlen   >= every sequence length; the workspace and the prepass
 *               buffers have the dense shape (B = nseq, H, N = max_seqlen, D):
 *               size them with sage_workspace_bytes(nseq, H, max_seqlen, D).
 *               Row r of head b*H + h in the buffers is token r of sequence b.
 * Each sequence is smoothed, quantized and attended on its own (its own K and
 * V means, 128-token Q blocks from its first token, compensation rows, causal
 * mask), exactly as a dense call with B = 1, N = its length would do.
 * qk_bits 4 or 8 (the adaptive width is not offered for packed sequences).
 */
sage_status sage_quant_smooth_varlen(const void* q, const void* k, const void* v, sage_dtype in_dtype,
                                     const int* cu_seqlens, int nseq, int max_seqlen, int total_tokens, int H, int D,
                                     int qk_bits, int smooth_v, const sage_quant_bufs* out, hipStream_t stream);

sage_status sage_attn_fwd_varlen(const void* q, const void* k, const void* v, void* o, const int* cu_seqlens,
                                 int nseq, int max_seqlen, int total_tokens, int H, int D, int causal, float sm_scale,
                                 int qk_bits, int smooth_v, sage_dtype in_dtype, sage_dtype out_dtype,
                                 void* workspace, size_t workspace_bytes, hipStream_t stream);

/* The fused kernel alone over buffers written by sage_quant_smooth_varlen
 * with the same cu_seqlens, nseq, max_seqlen, total_tokens, H, D, qk_bits. */
sage_status sage_attn_quantized_varlen(const sage_quant_bufs* qb, void* o, const int* cu_seqlens, int nseq,
                                       int max_seqlen, int total_tokens, int H, int D, int causal, float sm_scale,
                                       int qk_bits, sage_dtype out_dtype, hipStream_t stream);

/*
 * Debug: the exact integer dot products of the Q/K codes (qk_bits as written
 * by the prepass), computed by the same matrix-core tile routine as the fused
 * kernel.  For head bh = b*H + h:
 *   out[a][c] = sum_ch qcode[q0+a][ch] * kcode[k0+c][ch],  a < nq, c < nk
 * out: device int32 [nq, nk].  Requires 0 <= q0, q0+nq <= N, 0 <= k0,
 * k0+nk <= N, nq, nk >= 1.
 */
sage_status sage_qk_int32_debug(const sage_quant_bufs* qb, int B, int H, int N, int D, int qk_bits, int bh,
                                int q0, int k0, int nq, int nk, int32_t* out, hipStream_t stream);

/*
 * Debug: fp32 -> OCP e4m3fn with the device conversion the kernels use for P~
 * and V (round to nearest even).  in: device fp32 [n]; out: device uint8 [n].
 */
sage_status sage_fp8_encode_debug(const float* in, uint8_t* out, size_t n, hipStream_t stream);

/*
 * Debug: one FP8 (OCP e4m3fn) 32x32x64 matrix-core product with fp32
 * accumulator, the instruction of the fused kernel's P~V products and row
 * sums (the arXiv abstract page's FP8 P~V): d = a * b + c.
 * a: device uint8 [32][64] (e4m3 codes, row-major), b: device uint8 [64][32],
 * c, d: device fp32 [32][32] row-major (d may equal c).  Lane l of the wave
 * feeds row l%32 of a and column l%32 of b with k = 32*(l/32) .. +31 in byte
 * order.  For tests of how the products are accumulated.
 */
sage_status sage_fp8_mfma_debug(const uint8_t* a, const uint8_t* b, const float* c, float* d, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* SAGE_H_ */
