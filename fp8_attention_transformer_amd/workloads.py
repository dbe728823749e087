"""Seeded synthetic attention inputs.

The SageAttention2 pages measure end-to-end quality on language, image and
video generation models (arXiv 2411.10958 abstract page).  Those models are not
available here, so attention inputs are synthesised with the shapes and value
structure of such layers: LLM prefill, DiT image generation, video generation
with a long token sequence, and a long-context sweep.

This module holds no step of the attention method.  It draws random numbers
(numpy PCG64 via ``default_rng(seed)``), adds per-channel offsets and outlier
channels, and rounds to the 16-bit input dtype with round-to-nearest-even.  The
same bits feed the GPU path and the CPU oracle.
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

F16 = "f16"
BF16 = "bf16"


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    D: int
    dtype: str            # "f16" or "bf16"
    causal: bool
    seed: int
    k_offset_std: float = 0.0       # shared per-(b,h) channel offset added to every K token
    v_offset_std: float = 0.0       # same for V
    outlier_channels: int = 0       # channels scaled by outlier_scale
    outlier_scale: float = 1.0
    outliers_in_k: bool = False     # same channel indices in K as in Q
    t_noise_scale: float = 0.0      # Student-t(3) noise added to Q and K
    sm_scale: float | None = None   # default 1/sqrt(D)
    note: str = ""
    Hkv: int = 0                    # key/value heads (0: same as H); H must be a multiple
    Nk: int = 0                     # key/value tokens (0: same as N)

    @property
    def scale(self) -> float:
        return self.sm_scale if self.sm_scale is not None else 1.0 / math.sqrt(self.D)

    @property
    def hkv(self) -> int:
        return self.Hkv or self.H

    @property
    def nk(self) -> int:
        return self.Nk or self.N

    @property
    def self_attention(self) -> bool:
        return self.hkv == self.H and self.nk == self.N

    @property
    def ops(self) -> float:
        """Attention operations 4*B*H*N*Nk*D; causal (aligned at the last key)
        drops the upper triangle of the N x N corner: 4*B*H*D*(N*Nk - N^2/2)."""
        pairs = self.N * self.nk - (self.N * self.N / 2 if self.causal else 0)
        return 4.0 * self.B * self.H * pairs * self.D

    def with_(self, **kw) -> "Workload":
        d = dict(self.__dict__)
        d.update(kw)
        return Workload(**d)


# The five workload families (sizes and distributions of the method's target
# layers).  The long-context family has three lengths, causal and not.
TINY = Workload("tiny_b1h2n256d64_f16", 1, 2, 256, 64, F16, False, seed=1, k_offset_std=3.0,
                note="tiny non-causal; fp16; K channel offset ~N(0,3)")
LLM = Workload("llm_prefill_b4h32n4096d128_causal", 4, 32, 4096, 128, BF16, True, seed=2, k_offset_std=4.0,
               outlier_channels=4, outlier_scale=20.0,
               note="LLM prefill; causal; K offset ~N(0,4); 4 Q outlier channels x20")
DIT = Workload("dit_b1h24n4608d128", 1, 24, 4608, 128, BF16, False, seed=3, k_offset_std=4.0, v_offset_std=1.0,
               note="DiT image generation; K offset ~N(0,4); V offset ~N(0,1)")
VIDEO = Workload("video_b2h48n17776d64", 2, 48, 17776, 64, BF16, False, seed=4, k_offset_std=5.0,
                 outlier_channels=8, outlier_scale=15.0, outliers_in_k=True,
                 note="video generation; 8 outlier channels x15 in Q and K; K offset ~N(0,5)")


def long_context(N: int, causal: bool) -> Workload:
    return Workload(f"long_b1h16n{N}d128{'_causal' if causal else ''}", 1, 16, N, 128, BF16, causal, seed=5,
                    k_offset_std=4.0, t_noise_scale=0.5,
                    note="long context; N(0,1)+0.5*t(3) on Q,K; K offset ~N(0,4)")


LONG = [long_context(n, c) for n in (8192, 16384, 32768) for c in (False, True)]

# Language-model inference against a key/value cache with grouped-query heads
# (32 query heads sharing 8 K/V heads): one decoding step (one new token per
# sequence) and one 512-token chunk of a chunked prefill (causal, aligned at
# the last key); value structure of the LLM prefill family.
DECODE = Workload("llm_decode_b16hq32hkv8_nk8192d128", 16, 32, 1, 128, BF16, False, seed=6, k_offset_std=4.0,
                  outlier_channels=4, outlier_scale=20.0, Hkv=8, Nk=8192,
                  note="decoding step: 1 query per sequence, 8192 cached keys, 4 query heads per K/V head")
CHUNK = Workload("llm_chunk_b1hq32hkv8_nq512nk8192d128_causal", 1, 32, 512, 128, BF16, True, seed=7,
                 k_offset_std=4.0, outlier_channels=4, outlier_scale=20.0, Hkv=8, Nk=8192,
                 note="chunked prefill: the last 512 tokens of an 8192-token context")
CROSS = [DECODE, CHUNK]
ALL = [TINY, LLM, DIT, VIDEO] + LONG + CROSS
BY_NAME = {w.name: w for w in ALL}
# The configuration the headline throughput is quoted on: N = 16k, D = 128.
HEADLINE = long_context(16384, False)


def round_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round fp32 values to the 16-bit dtype (RNE) and return the raw bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if dtype == F16:
        return x.astype(np.float16).view(np.uint16)
    if dtype == BF16:
        u = x.view(np.uint32).astype(np.uint64)
        r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
        return r.astype(np.uint16)
    raise ValueError(dtype)


def bits_to_f32(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == F16:
        return bits.view(np.float16).astype(np.float32)
    return (bits.astype(np.uint32) << 16).view(np.float32)


def generate(w: Workload, heads: slice | None = None):
    """Return (q_bits, k_bits, v_bits) as uint16 arrays of shape [B,H,N,D]
    (K and V [B,Hkv,Nk,D] for a cross-attention or grouped-query workload).

    ``heads`` optionally restricts the output to a slice of the flattened B*H
    head index (the draw for every head is still the same as in the full
    tensor, because each head has its own sub-stream)."""
    if not w.self_attention:
        if heads is not None:
            raise ValueError("head slices are for self-attention workloads")
        return _generate_cross(w)
    B, H, N, D = w.B, w.H, w.N, w.D
    root = np.random.default_rng(w.seed)
    # shared outlier channel indices (same for every head)
    out_idx = root.choice(D, w.outlier_channels, replace=False) if w.outlier_channels else np.zeros(0, np.int64)
    hsel = range(B * H) if heads is None else range(B * H)[heads]
    seeds = root.integers(0, 2**63 - 1, size=B * H)
    qs, ks, vs = [], [], []
    for bh in hsel:
        rng = np.random.default_rng(int(seeds[bh]))
        q = rng.standard_normal((N, D), dtype=np.float32)
        k = rng.standard_normal((N, D), dtype=np.float32)
        v = rng.standard_normal((N, D), dtype=np.float32)
        if w.t_noise_scale:
            q += (w.t_noise_scale * rng.standard_t(3, (N, D))).astype(np.float32)
            k += (w.t_noise_scale * rng.standard_t(3, (N, D))).astype(np.float32)
        if w.outlier_channels:
            q[:, out_idx] *= np.float32(w.outlier_scale)
            if w.outliers_in_k:
                k[:, out_idx] *= np.float32(w.outlier_scale)
        if w.k_offset_std:
            k += (w.k_offset_std * rng.standard_normal(D)).astype(np.float32)[None, :]
        if w.v_offset_std:
            v += (w.v_offset_std * rng.standard_normal(D)).astype(np.float32)[None, :]
        qs.append(round_to_bits(q, w.dtype))
        ks.append(round_to_bits(k, w.dtype))
        vs.append(round_to_bits(v, w.dtype))
    nh = len(qs)
    shape = (B, H, N, D) if heads is None else (nh, 1, N, D)
    return (np.stack(qs).reshape(shape), np.stack(ks).reshape(shape), np.stack(vs).reshape(shape))


def custom(B, H, N, D, dtype=BF16, causal=False, seed=0, **kw) -> Workload:
    return Workload(f"custom_b{B}h{H}n{N}d{D}", B, H, N, D, dtype, causal, seed, **kw)


def _generate_cross(w: Workload):
    """Queries and keys/values with their own head counts and lengths: one
    sub-stream per (batch, query head) for Q, then one per (batch, K/V head)
    for K and V; distributions as in the self-attention draw."""
    B, Hq, Hk, Nq, Nk, D = w.B, w.H, w.hkv, w.N, w.nk, w.D
    root = np.random.default_rng(w.seed)
    out_idx = root.choice(D, w.outlier_channels, replace=False) if w.outlier_channels else np.zeros(0, np.int64)
    seeds = root.integers(0, 2**63 - 1, size=B * Hq + B * Hk)
    qs, ks, vs = [], [], []
    for bh in range(B * Hq):
        rng = np.random.default_rng(int(seeds[bh]))
        q = rng.standard_normal((Nq, D), dtype=np.float32)
        if w.t_noise_scale:
            q += (w.t_noise_scale * rng.standard_t(3, (Nq, D))).astype(np.float32)
        if w.outlier_channels:
            q[:, out_idx] *= np.float32(w.outlier_scale)
        qs.append(round_to_bits(q, w.dtype))
    for bh in range(B * Hk):
        rng = np.random.default_rng(int(seeds[B * Hq + bh]))
        k = rng.standard_normal((Nk, D), dtype=np.float32)
        v = rng.standard_normal((Nk, D), dtype=np.float32)
        if w.t_noise_scale:
            k += (w.t_noise_scale * rng.standard_t(3, (Nk, D))).astype(np.float32)
        if w.outlier_channels and w.outliers_in_k:
            k[:, out_idx] *= np.float32(w.outlier_scale)
        if w.k_offset_std:
            k += (w.k_offset_std * rng.standard_normal(D)).astype(np.float32)[None, :]
        if w.v_offset_std:
            v += (w.v_offset_std * rng.standard_normal(D)).astype(np.float32)[None, :]
        ks.append(round_to_bits(k, w.dtype))
        vs.append(round_to_bits(v, w.dtype))
    return (np.stack(qs).reshape(B, Hq, Nq, D), np.stack(ks).reshape(B, Hk, Nk, D),
            np.stack(vs).reshape(B, Hk, Nk, D))


@dataclass(frozen=True)
class PackedWorkload:
    """A packed variable-length batch: independent sequences of the given
    lengths in token-major [T, H, D] tensors, each drawn like ``base`` (its
    H, D, dtype, causal flag and distributions; ``base.N`` is ignored) with
    seed base.seed + sequence index."""
    name: str
    lengths: tuple
    base: Workload

    @property
    def ops(self) -> float:
        o = sum(4.0 * self.base.H * n * n * self.base.D for n in self.lengths)
        return o / 2 if self.base.causal else o


def generate_packed(pw: PackedWorkload):
    """(q, k, v) token-major [T, H, D] 16-bit patterns and cu_seqlens int32 [nseq + 1]."""
    H, D = pw.base.H, pw.base.D
    T = int(sum(pw.lengths))
    out = [np.zeros((T, H, D), np.uint16) for _ in range(3)]
    off = 0
    for s, n in enumerate(pw.lengths):
        if n:
            parts = generate(pw.base.with_(B=1, N=int(n), seed=pw.base.seed + s))
            for dst, src in zip(out, parts):
                dst[off:off + n] = np.transpose(src[0], (1, 0, 2))
        off += n
    cu = np.concatenate([[0], np.cumsum(pw.lengths)]).astype(np.int32)
    return out[0], out[1], out[2], cu


# An LLM-serving-style packed prefill batch: eight prompts of mixed length
# drawn like the LLM prefill workload (causal, H=32, D=128).
PACKED_LLM = PackedWorkload("packed_llm_8seq_t17115_h32d128_causal",
                            (4096, 1024, 3072, 512, 2048, 777, 4096, 1490), LLM)
PACKED = [PACKED_LLM]
