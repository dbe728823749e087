"""Helpers for the GPU parity tests: device placement, workspace readback and
conversion of the library's packed layouts to the oracle's canonical arrays.

Layout decoding follows include/sage.h; nothing here computes a step of the
attention method.
"""
from __future__ import annotations

import numpy as np

from fp8_attention_transformer_amd import sage
from fp8_attention_transformer_amd import workloads as wl


def torch_mod():
    import torch
    return torch


def to_device(bits: np.ndarray, dtype: str):
    torch = torch_mod()
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    t = t.view(torch.float16 if dtype == wl.F16 else torch.bfloat16)
    return t.cuda()


def in_code(dtype: str) -> int:
    return sage.F16 if dtype == wl.F16 else sage.BF16


def vperm_keys() -> np.ndarray:
    """Key held by each position p of a 128-key block of the FP8 V layout."""
    p = np.arange(128)
    s = p % 32
    return 64 * (p // 64) + 32 * (s // 16) + 8 * ((s % 16) // 4) + 4 * ((p % 64) // 32) + s % 4


FP6_MAG = np.array([0, 8, 16, 20, 24, 26, 28, 30], np.uint8)   # e2m3 patterns of 0..7


def fp6_lane_bytes(D: int) -> int:
    return 48 if D == 128 else 32


def fp6_row_bytes(D: int) -> int:
    return 2 * fp6_lane_bytes(D)


def _fp6_value(v: np.ndarray) -> np.ndarray:
    """FP6 e2m3 bit patterns -> float values."""
    v = v.astype(np.int64)
    e, m = (v >> 3) & 3, v & 7
    mag = np.where(e == 0, m / 8.0, 2.0 ** (e - 1) * (1.0 + m / 8.0))
    return np.where(v & 32, -mag, mag)


def fp6_tiles_to_codes(raw: np.ndarray, D: int, strict: bool = True) -> np.ndarray:
    """[BH, NP * row_bytes] FP6 tile layout (include/sage.h) -> int8 codes [BH, NP, D]."""
    LS = fp6_lane_bytes(D)
    BH = raw.shape[0]
    ch = raw.reshape(BH, -1, 64, LS).copy()          # [BH, tile, chunk, bytes]
    if D == 64:                                       # undo the swapped halves
        sw = ((np.arange(64) >> 3) & 1).astype(bool)
        ch[:, :, sw] = np.concatenate([ch[:, :, sw, 16:], ch[:, :, sw, :16]], axis=-1)
    groups = ch[..., :24 * (D // 64)].reshape(BH, ch.shape[1], 64, D // 64, 24)
    bits = np.unpackbits(groups, axis=-1, bitorder="little").reshape(groups.shape[:-1] + (32, 6))
    fields = (bits.astype(np.int64) << np.arange(6)).sum(-1)          # [BH, tile, chunk, m, i]
    vals = _fp6_value(fields)
    if strict:
        assert np.all(vals == np.rint(vals)) and np.all(np.abs(vals) <= 7), "FP6 fields are not INT4 codes"
    vals = np.clip(np.rint(vals), -127, 127)
    T = ch.shape[1]
    out = np.empty((BH, T, 32, D), np.int8)
    for h in range(2):
        for m in range(D // 64):
            out[:, :, :, 64 * m + 32 * h: 64 * m + 32 * h + 32] = vals[:, :, 32 * h:32 * h + 32, m, :]
    return out.reshape(BH, T * 32, D)


def codes_to_fp6_tiles(codes: np.ndarray, D: int) -> np.ndarray:
    """Inverse of fp6_tiles_to_codes: int8 codes [BH, NP, D] -> [BH, NP * row_bytes] bytes."""
    BH, NP, _ = codes.shape
    LS = fp6_lane_bytes(D)
    c = codes.astype(np.int64).reshape(BH, NP // 32, 32, D)
    pat = FP6_MAG[np.abs(c)].astype(np.int64) | np.where(c < 0, 32, 0)
    ch = np.zeros((BH, NP // 32, 64, LS), np.uint8)
    for h in range(2):
        for m in range(D // 64):
            f = pat[:, :, :, 64 * m + 32 * h: 64 * m + 32 * h + 32]          # [BH, T, 32 rows, 32 fields]
            bits = ((f[..., None] >> np.arange(6)) & 1).astype(np.uint8).reshape(f.shape[:-1] + (192,))
            ch[:, :, 32 * h:32 * h + 32, 24 * m:24 * m + 24] = np.packbits(bits, axis=-1, bitorder="little")
    if D == 64:
        sw = ((np.arange(64) >> 3) & 1).astype(bool)
        ch[:, :, sw] = np.concatenate([ch[:, :, sw, 16:], ch[:, :, sw, :16]], axis=-1)
    return ch.reshape(BH, -1)


def unpack_codes(packed: np.ndarray, N: int, D: int, qk_bits: int = 4, strict: bool = True) -> np.ndarray:
    """Stored code rows -> int8 codes [BH, N, D] (INT4: FP6 tiles; INT8: one byte per channel).
    strict: every FP6 field must be an INT4 code (off where parts of a workspace are never written)."""
    if qk_bits == 8:
        return packed.reshape(packed.shape[0], -1, D).view(np.int8)[:, :N].copy()
    return fp6_tiles_to_codes(packed, D, strict)[:, :N]


def unpermute_v(vcodes: np.ndarray, BH: int, NQB: int, D: int, N: int) -> np.ndarray:
    """[BH, NQB, D, 128] permuted FP8 bytes -> [BH, N, D]."""
    v = vcodes.reshape(BH, NQB, D, 128)
    keys = vperm_keys()
    out = np.empty((BH, NQB, 128, D), np.uint8)
    out[:, :, keys, :] = np.transpose(v, (0, 1, 3, 2))
    return out.reshape(BH, NQB * 128, D)[:, :N]


class Readback:
    """The prepass arrays of a workspace, copied to host in canonical form.
    Query-side arrays use (H, N), key/value-side arrays (Hkv, Nk)."""

    def __init__(self, ws: sage.Workspace, qk_bits: int = 4, strict: bool = True):
        torch = torch_mod()
        B, H, N, D = ws.B, ws.H, ws.N, ws.D
        Hk, Nk = ws.Hkv or H, ws.Nk or N
        BH, BHk = B * H, B * Hk
        NP, NPk = (N + 127) // 128 * 128, (Nk + 127) // 128 * 128
        NQB, NQBk = NP // 128, NPk // 128
        qb = ws.bufs()
        host = ws.tensor.cpu().numpy()
        base = ws.tensor.data_ptr()

        def arr(ptr, nbytes, dtype, shape):
            off = ptr - base
            return host[off:off + nbytes].view(dtype).reshape(shape)

        self.N, self.NP, self.NQB, self.D, self.BH = N, NP, NQB, D, BH
        self.Nk, self.NPk, self.NQBk, self.BHk = Nk, NPk, NQBk, BHk
        self.qk_bits = qk_bits
        rowb = fp6_row_bytes(D) if qk_bits == 4 else D
        self.q_codes_raw = arr(qb.q_codes, BH * NP * rowb, np.uint8, (BH, NP * rowb))
        self.k_codes_raw = arr(qb.k_codes, BHk * NPk * rowb, np.uint8, (BHk, NPk * rowb))
        self.q_codes_all = unpack_codes(self.q_codes_raw, NP, D, qk_bits, strict)   # padded rows included
        self.k_codes_all = unpack_codes(self.k_codes_raw, NPk, D, qk_bits, strict)
        self.q_codes = self.q_codes_all[:, :N]
        self.k_codes = self.k_codes_all[:, :Nk]
        self.q_scale_p = arr(qb.q_scale, BH * NP * 4, np.float32, (BH, NP))
        self.k_scale_p = arr(qb.k_scale, BHk * NPk // 16 * 4, np.float32, (BHk, NPk // 16))
        self.q_mean = arr(qb.q_mean, BH * NQB * D * 4, np.float32, (BH, NQB, D))
        self.k_mean = arr(qb.k_mean, BHk * D * 4, np.float32, (BHk, D))
        self.v_codes_raw = arr(qb.v_codes, BHk * NPk * D, np.uint8, (BHk, NQBk, D, 128))
        self.v_codes = unpermute_v(self.v_codes_raw, BHk, NQBk, D, Nk)
        self.v_scale = arr(qb.v_scale, BHk * D * 4, np.float32, (BHk, D))
        self.v_mean = arr(qb.v_mean, BHk * D * 4, np.float32, (BHk, D))
        self.delta_s_p = arr(qb.delta_s, BH * NQB * NPk * 4, np.float32, (BH, NQB, NPk))
        G = 2 * ((Nk + 31) // 32)
        self.q_scale = self.q_scale_p[:, :N]
        self.k_scale = self.k_scale_p[:, :G]
        self.delta_s = self.delta_s_p[:, :, :Nk]
        torch.cuda.synchronize()


def run_quant_smooth(q_bits, k_bits, v_bits, dtype: str, qk_bits: int = 4, smooth_v: bool = False):
    """Prepass into a poisoned workspace: the self-attention entry point when
    Q and K/V share heads and length, the cross-geometry one otherwise."""
    torch = torch_mod()
    B, H, N, D = q_bits.shape
    Hk, Nk = k_bits.shape[1], k_bits.shape[2]
    q, k, v = (to_device(a, dtype) for a in (q_bits, k_bits, v_bits))
    ws = sage.alloc_workspace(B, H, N, D, Hkv=Hk, Nk=Nk)
    ws.tensor.fill_(0xA5)  # poison: every array element the prepass owns must be written
    sh = torch.cuda.current_stream().cuda_stream
    if Hk == H and Nk == N:
        sage.quant_smooth(q.data_ptr(), k.data_ptr(), v.data_ptr(), in_code(dtype), B, H, N, D, ws.bufs(), sh,
                          qk_bits=qk_bits, smooth_v=smooth_v)
    else:
        sage.quant_smooth_cross(q.data_ptr(), k.data_ptr(), v.data_ptr(), in_code(dtype), B, H, Hk, N, Nk, D,
                                ws.bufs(), sh, qk_bits=qk_bits, smooth_v=smooth_v)
    torch.cuda.synchronize()
    return ws


def run_attn(q_bits, k_bits, v_bits, dtype: str, causal: bool, sm_scale: float, out_dtype=None, qk_bits: int = 4,
             smooth_v: bool = False):
    torch = torch_mod()
    B, H, N, D = q_bits.shape
    Hk, Nk = k_bits.shape[1], k_bits.shape[2]
    q, k, v = (to_device(a, dtype) for a in (q_bits, k_bits, v_bits))
    ws = sage.alloc_workspace(B, H, N, D, Hkv=Hk, Nk=Nk)
    out = sage.attn(q, k, v, causal=causal, sm_scale=sm_scale, out_dtype=out_dtype or torch.float32, workspace=ws,
                    qk_bits=qk_bits, smooth_v=smooth_v)
    torch.cuda.synchronize()
    return out, ws


def cos_sim(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))


# The output bar: max-abs 2e-3 against the oracle's mirror of the method.
O_TOL = 2e-3
# Relative window around FP8 rounding midpoints inside which the mirror marks
# a P~ element as one whose code the GPU's exp2 or compensation rounding could
# flip; reported for diagnosis only, it widens no bar.
EPS_TIE = 2.0 ** -14


def output_rounding(O_ref, out_dtype: str) -> np.ndarray:
    """Half a unit in the last place of a 16-bit output format at the size of
    |O| (plus the bar): the rounding of the fp32 result to the output dtype."""
    if out_dtype == "f32":
        return np.zeros(O_ref.shape)
    mant = 7 if out_dtype == "bf16" else 10
    mag = np.maximum(np.abs(O_ref.astype(np.float64)) + O_TOL, 2.0 ** -24)
    return np.exp2(np.floor(np.log2(mag)) - mant - 1)


def compare_o(O_gpu, O_ref, label: str, out_dtype: str = "f32", slack=None):
    """Element-wise |O_gpu - O_ref| <= 2e-3, plus (16-bit outputs only) the
    output rounding.  NaN fails.  Prints the largest error and, if the mirror's
    midpoint slack is given, how many rows hold a P~ element near an FP8
    midpoint (diagnostic)."""
    g = np.asarray(O_gpu, np.float64)
    r = np.asarray(O_ref, np.float64)
    err = np.abs(g - r)
    allowed = O_TOL + output_rounding(r, out_dtype)
    bad_el = ~(err <= allowed)
    bad = np.nonzero(bad_el.reshape(bad_el.shape[0], -1).any(1))[0]
    extra = ""
    if slack is not None:
        extra = f" rows_near_fp8_midpoint={int(np.sum(np.asarray(slack) > 0))}"
    print(f"[{label}] rows={r.shape[0]} maxerr={err.max():.3e} out={out_dtype}{extra}")
    assert bad.size == 0, (label, bad[:5], err.reshape(err.shape[0], -1).max(1)[bad[:5]])
    return float(err.max())


def sample_rows(N: int, heads: int, rng, per_head: int = 4, pair_blocks: bool = True) -> np.ndarray:
    """Query rows of every head (flattened head*N + i): the first and last rows,
    the first block's edge, the start and last row of the tail block, the
    middle, one row in query block p and one in its causal pair partner
    NQB-1-p (p varies with the head), and per_head random rows."""
    nqb = (N + 127) // 128
    rows = []
    for hh in range(heads):
        pick = {0, 1, 127, 128, N // 2, N - 1, (nqb - 1) * 128}
        if pair_blocks and nqb > 1:
            p = hh % nqb
            pick.add(p * 128 + int(rng.integers(0, 128)))
            pick.add((nqb - 1 - p) * 128 + int(rng.integers(0, 128)))
        pick.update(rng.integers(0, N, per_head).tolist())
        rows.extend(hh * N + np.array(sorted(i for i in pick if 0 <= i < N)))
    return np.array(rows, np.int64)
