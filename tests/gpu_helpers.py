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


def unpack_codes(packed: np.ndarray, N: int, qk_bits: int = 4) -> np.ndarray:
    """[BH, NP, D*qk_bits/8] code rows -> int8 codes [BH, N, D] (INT4: packed pairs; INT8: one byte each)."""
    if qk_bits == 8:
        return packed.view(np.int8)[:, :N].copy()
    v = packed.view(np.int8).astype(np.int16)[:, :N]
    even = (v & 15) - 8
    odd = v >> 4
    out = np.empty(v.shape[:-1] + (v.shape[-1] * 2,), np.int8)
    out[..., 0::2] = even
    out[..., 1::2] = odd
    return out


def unpermute_v(vcodes: np.ndarray, BH: int, NQB: int, D: int, N: int) -> np.ndarray:
    """[BH, NQB, D, 128] permuted FP8 bytes -> [BH, N, D]."""
    v = vcodes.reshape(BH, NQB, D, 128)
    keys = vperm_keys()
    out = np.empty((BH, NQB, 128, D), np.uint8)
    out[:, :, keys, :] = np.transpose(v, (0, 1, 3, 2))
    return out.reshape(BH, NQB * 128, D)[:, :N]


class Readback:
    """The prepass arrays of a workspace, copied to host in canonical form."""

    def __init__(self, ws: sage.Workspace, qk_bits: int = 4):
        torch = torch_mod()
        B, H, N, D = ws.B, ws.H, ws.N, ws.D
        BH = B * H
        NP = (N + 127) // 128 * 128
        NQB = NP // 128
        qb = ws.bufs()
        host = ws.tensor.cpu().numpy()
        base = ws.tensor.data_ptr()

        def arr(ptr, nbytes, dtype, shape):
            off = ptr - base
            return host[off:off + nbytes].view(dtype).reshape(shape)

        self.N, self.NP, self.NQB, self.D, self.BH = N, NP, NQB, D, BH
        self.qk_bits = qk_bits
        krow = D * qk_bits // 8
        self.q_codes_packed = arr(qb.q_codes, BH * NP * krow, np.uint8, (BH, NP, krow))
        self.k_codes_packed = arr(qb.k_codes, BH * NP * krow, np.uint8, (BH, NP, krow))
        self.zero_code_byte = 8 if qk_bits == 4 else 0
        self.q_codes = unpack_codes(self.q_codes_packed, N, qk_bits)
        self.k_codes = unpack_codes(self.k_codes_packed, N, qk_bits)
        self.q_scale_p = arr(qb.q_scale, BH * NP * 4, np.float32, (BH, NP))
        self.k_scale_p = arr(qb.k_scale, BH * NP // 16 * 4, np.float32, (BH, NP // 16))
        self.q_mean = arr(qb.q_mean, BH * NQB * D * 4, np.float32, (BH, NQB, D))
        self.k_mean = arr(qb.k_mean, BH * D * 4, np.float32, (BH, D))
        self.v_codes_raw = arr(qb.v_codes, BH * NP * D, np.uint8, (BH, NQB, D, 128))
        self.v_codes = unpermute_v(self.v_codes_raw, BH, NQB, D, N)
        self.v_scale = arr(qb.v_scale, BH * D * 4, np.float32, (BH, D))
        self.delta_s_p = arr(qb.delta_s, BH * NQB * NP * 4, np.float32, (BH, NQB, NP))
        G = 2 * ((N + 31) // 32)
        self.q_scale = self.q_scale_p[:, :N]
        self.k_scale = self.k_scale_p[:, :G]
        self.delta_s = self.delta_s_p[:, :, :N]
        torch.cuda.synchronize()


def run_quant_smooth(q_bits, k_bits, v_bits, dtype: str, qk_bits: int = 4):
    torch = torch_mod()
    B, H, N, D = q_bits.shape
    q, k, v = (to_device(a, dtype) for a in (q_bits, k_bits, v_bits))
    ws = sage.alloc_workspace(B, H, N, D)
    ws.tensor.fill_(0xA5)  # poison: every array element the prepass owns must be written
    sage.quant_smooth(q.data_ptr(), k.data_ptr(), v.data_ptr(), in_code(dtype), B, H, N, D, ws.bufs(),
                      torch.cuda.current_stream().cuda_stream, qk_bits=qk_bits)
    torch.cuda.synchronize()
    return ws


def run_attn(q_bits, k_bits, v_bits, dtype: str, causal: bool, sm_scale: float, out_dtype=None, qk_bits: int = 4):
    torch = torch_mod()
    B, H, N, D = q_bits.shape
    q, k, v = (to_device(a, dtype) for a in (q_bits, k_bits, v_bits))
    ws = sage.alloc_workspace(B, H, N, D)
    out = sage.attn(q, k, v, causal=causal, sm_scale=sm_scale, out_dtype=out_dtype or torch.float32, workspace=ws,
                    qk_bits=qk_bits)
    torch.cuda.synchronize()
    return out, ws


def cos_sim(a, b) -> float:
    a = np.asarray(a, np.float64).ravel()
    b = np.asarray(b, np.float64).ravel()
    return float(a @ b / (np.linalg.norm(a) * np.linalg.norm(b)))
