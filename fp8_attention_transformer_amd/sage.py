"""ctypes binding of libsage (include/sage.h): argument marshalling only.

Every step of the attention runs in the HIP kernels of libsage.so; torch is
used here only to allocate device memory and to name the current stream.  The
functions carry the C names without the ``sage_`` prefix.  There is no CPU
fallback: if the library is missing, loading raises.
"""
from __future__ import annotations

import ctypes
import math
import os
from dataclasses import dataclass

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libsage.so")

OK, ERR_INVALID, ERR_UNSUPPORTED, ERR_WORKSPACE, ERR_HIP = 0, -1, -2, -3, -4
F16, BF16, F32 = 0, 1, 2

EXPORTED = [
    "sage_contract_version", "sage_status_string", "sage_workspace_bytes", "sage_quant_bufs_from_workspace",
    "sage_quant_smooth", "sage_attn_fwd", "sage_attn_quantized", "sage_qk_int32_debug", "sage_fp8_encode_debug",
    "sage_quant_smooth_varlen", "sage_attn_fwd_varlen", "sage_attn_quantized_varlen",
    "sage_workspace_bytes_cross", "sage_quant_bufs_from_workspace_cross", "sage_quant_smooth_cross",
    "sage_attn_fwd_cross", "sage_attn_quantized_cross",
    "sage_decode_split_keys", "sage_decode_workspace_bytes", "sage_attn_decode",
    "sage_split_keys", "sage_split_workspace_bytes", "sage_attn_fwd_split", "sage_attn_fwd_static",
    "sage_quant_smooth_adaptive", "sage_quant_smooth_adaptive_cross", "sage_fp8_mfma_debug",
]
ADAPTIVE = 0   # qk_bits value of the adaptive width (INT4 or INT8 per key/value head)
STATIC_SCRATCH_BYTES = 128 << 20   # SAGE_STATIC_SCRATCH_BYTES


class QuantBufs(ctypes.Structure):
    """Mirror of sage_quant_bufs (device pointers)."""
    _fields_ = [(name, ctypes.c_void_p) for name in (
        "q_codes", "k_codes", "q_scale", "k_scale", "q_mean", "k_mean", "v_codes", "v_scale", "delta_s",
        "k_part", "v_part", "v_mean", "m2_part", "adapt_stat", "head_bits")]


class SageError(RuntimeError):
    def __init__(self, status: int, where: str):
        super().__init__(f"{where}: {status_string(status)}")
        self.status = status


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() or "
                               "python fp8_attention_transformer_amd/build.py")
        L = ctypes.CDLL(LIB_PATH)
        P, i32, sz, f32 = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
        L.sage_contract_version.restype = i32
        L.sage_status_string.argtypes = [i32]
        L.sage_status_string.restype = ctypes.c_char_p
        L.sage_workspace_bytes.argtypes = [i32, i32, i32, i32]
        L.sage_workspace_bytes.restype = sz
        L.sage_quant_bufs_from_workspace.argtypes = [P, sz, i32, i32, i32, i32, ctypes.POINTER(QuantBufs)]
        L.sage_quant_bufs_from_workspace.restype = i32
        L.sage_quant_smooth.argtypes = [P, P, P, i32, i32, i32, i32, i32, i32, i32, ctypes.POINTER(QuantBufs), P]
        L.sage_quant_smooth.restype = i32
        L.sage_attn_fwd.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, f32, i32, i32, i32, i32, P, sz, P]
        L.sage_attn_fwd.restype = i32
        L.sage_attn_quantized.argtypes = [ctypes.POINTER(QuantBufs), P, i32, i32, i32, i32, i32, f32, i32, i32, P]
        L.sage_attn_quantized.restype = i32
        L.sage_qk_int32_debug.argtypes = [ctypes.POINTER(QuantBufs), i32, i32, i32, i32, i32, i32, i32, i32, i32,
                                          i32, P, P]
        L.sage_qk_int32_debug.restype = i32
        L.sage_fp8_encode_debug.argtypes = [P, P, sz, P]
        L.sage_fp8_encode_debug.restype = i32
        L.sage_fp8_mfma_debug.argtypes = [P, P, P, P, P]
        L.sage_fp8_mfma_debug.restype = i32
        L.sage_quant_smooth_varlen.argtypes = [P, P, P, i32, P, i32, i32, i32, i32, i32, i32, i32,
                                               ctypes.POINTER(QuantBufs), P]
        L.sage_quant_smooth_varlen.restype = i32
        L.sage_attn_fwd_varlen.argtypes = [P, P, P, P, P, i32, i32, i32, i32, i32, i32, f32, i32, i32, i32, i32, P,
                                           sz, P]
        L.sage_attn_fwd_varlen.restype = i32
        L.sage_attn_quantized_varlen.argtypes = [ctypes.POINTER(QuantBufs), P, P, i32, i32, i32, i32, i32, i32, f32,
                                                 i32, i32, P]
        L.sage_attn_quantized_varlen.restype = i32
        L.sage_workspace_bytes_cross.argtypes = [i32] * 6
        L.sage_workspace_bytes_cross.restype = sz
        L.sage_quant_bufs_from_workspace_cross.argtypes = [P, sz] + [i32] * 6 + [ctypes.POINTER(QuantBufs)]
        L.sage_quant_bufs_from_workspace_cross.restype = i32
        L.sage_quant_smooth_cross.argtypes = [P, P, P] + [i32] * 9 + [ctypes.POINTER(QuantBufs), P]
        L.sage_quant_smooth_cross.restype = i32
        L.sage_attn_fwd_cross.argtypes = [P, P, P, P] + [i32] * 7 + [f32, i32, i32, i32, i32, P, sz, P]
        L.sage_attn_fwd_cross.restype = i32
        L.sage_attn_quantized_cross.argtypes = [ctypes.POINTER(QuantBufs), P] + [i32] * 7 + [f32, i32, i32, P]
        L.sage_attn_quantized_cross.restype = i32
        L.sage_decode_split_keys.argtypes = [i32] * 5
        L.sage_decode_split_keys.restype = i32
        L.sage_decode_workspace_bytes.argtypes = [i32] * 6
        L.sage_decode_workspace_bytes.restype = sz
        L.sage_attn_decode.argtypes = [P, P, P, P] + [i32] * 5 + [f32, i32, i32, i32, i32, P, sz, P]
        L.sage_attn_decode.restype = i32
        L.sage_split_keys.argtypes = [i32] * 6
        L.sage_split_keys.restype = i32
        L.sage_split_workspace_bytes.argtypes = [i32] * 7
        L.sage_split_workspace_bytes.restype = sz
        L.sage_attn_fwd_split.argtypes = [P, P, P, P] + [i32] * 7 + [f32, i32, i32, i32, i32, i32, P, sz, P]
        L.sage_attn_fwd_split.restype = i32
        L.sage_attn_fwd_static.argtypes = [P, P, P, P, i32, i32, i32, i32, i32, f32, i32, i32, i32, i32, P]
        L.sage_attn_fwd_static.restype = i32
        L.sage_quant_smooth_adaptive.argtypes = [P, P, P, i32, i32, i32, i32, i32, f32, i32,
                                                 ctypes.POINTER(QuantBufs), P]
        L.sage_quant_smooth_adaptive.restype = i32
        L.sage_quant_smooth_adaptive_cross.argtypes = [P, P, P] + [i32] * 7 + [f32, i32, ctypes.POINTER(QuantBufs), P]
        L.sage_quant_smooth_adaptive_cross.restype = i32
        _lib = L
    return _lib


def _check(status: int, where: str):
    if status != OK:
        raise SageError(status, where)


def status_string(status: int) -> str:
    return lib().sage_status_string(status).decode()


def contract_version() -> int:
    return lib().sage_contract_version()


def workspace_bytes(B: int, H: int, N: int, D: int) -> int:
    return lib().sage_workspace_bytes(B, H, N, D)


def quant_bufs_from_workspace(ws_ptr: int, nbytes: int, B: int, H: int, N: int, D: int) -> QuantBufs:
    qb = QuantBufs()
    _check(lib().sage_quant_bufs_from_workspace(ws_ptr, nbytes, B, H, N, D, ctypes.byref(qb)),
           "sage_quant_bufs_from_workspace")
    return qb


def quant_smooth(q_ptr: int, k_ptr: int, v_ptr: int, in_dtype: int, B: int, H: int, N: int, D: int,
                 bufs: QuantBufs, stream: int = 0, qk_bits: int = 4, smooth_v: bool = False) -> None:
    _check(lib().sage_quant_smooth(q_ptr, k_ptr, v_ptr, in_dtype, B, H, N, D, qk_bits, int(bool(smooth_v)),
                                   ctypes.byref(bufs), stream), "sage_quant_smooth")


def quant_smooth_adaptive(q_ptr: int, k_ptr: int, v_ptr: int, in_dtype: int, B: int, H: int, N: int, D: int,
                          sm_scale: float, bufs: QuantBufs, stream: int = 0, smooth_v: bool = False) -> None:
    _check(lib().sage_quant_smooth_adaptive(q_ptr, k_ptr, v_ptr, in_dtype, B, H, N, D, float(sm_scale),
                                            int(bool(smooth_v)), ctypes.byref(bufs), stream),
           "sage_quant_smooth_adaptive")


def quant_smooth_adaptive_cross(q_ptr: int, k_ptr: int, v_ptr: int, in_dtype: int, B: int, Hq: int, Hkv: int,
                                Nq: int, Nk: int, D: int, sm_scale: float, bufs: QuantBufs, stream: int = 0,
                                smooth_v: bool = False) -> None:
    _check(lib().sage_quant_smooth_adaptive_cross(q_ptr, k_ptr, v_ptr, in_dtype, B, Hq, Hkv, Nq, Nk, D,
                                                  float(sm_scale), int(bool(smooth_v)), ctypes.byref(bufs), stream),
           "sage_quant_smooth_adaptive_cross")


def attn_fwd(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, B: int, H: int, N: int, D: int, causal: bool,
             sm_scale: float, in_dtype: int, out_dtype: int, ws_ptr: int, ws_bytes: int, stream: int = 0,
             qk_bits: int = 4, smooth_v: bool = False) -> None:
    _check(lib().sage_attn_fwd(q_ptr, k_ptr, v_ptr, o_ptr, B, H, N, D, int(bool(causal)), float(sm_scale), qk_bits,
                               int(bool(smooth_v)), in_dtype, out_dtype, ws_ptr, ws_bytes, stream), "sage_attn_fwd")


def attn_fwd_static(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, B: int, H: int, N: int, D: int, causal: bool,
                    sm_scale: float, in_dtype: int, out_dtype: int, stream: int = 0, qk_bits: int = 4,
                    smooth_v: bool = False) -> None:
    """sage_attn_fwd_static: the forward with the library's fixed device scratch
    array as its workspace (nothing is allocated)."""
    _check(lib().sage_attn_fwd_static(q_ptr, k_ptr, v_ptr, o_ptr, B, H, N, D, int(bool(causal)), float(sm_scale),
                                      qk_bits, int(bool(smooth_v)), in_dtype, out_dtype, stream),
           "sage_attn_fwd_static")


def attn_quantized(bufs: QuantBufs, o_ptr: int, B: int, H: int, N: int, D: int, causal: bool, sm_scale: float,
                   out_dtype: int, stream: int = 0, qk_bits: int = 4) -> None:
    _check(lib().sage_attn_quantized(ctypes.byref(bufs), o_ptr, B, H, N, D, int(bool(causal)), float(sm_scale),
                                     qk_bits, out_dtype, stream), "sage_attn_quantized")


def qk_int32_debug(bufs: QuantBufs, B: int, H: int, N: int, D: int, bh: int, q0: int, k0: int, nq: int, nk: int,
                   out_ptr: int, stream: int = 0, qk_bits: int = 4) -> None:
    _check(lib().sage_qk_int32_debug(ctypes.byref(bufs), B, H, N, D, qk_bits, bh, q0, k0, nq, nk, out_ptr, stream),
           "sage_qk_int32_debug")


def fp8_encode_debug(in_ptr: int, out_ptr: int, n: int, stream: int = 0) -> None:
    _check(lib().sage_fp8_encode_debug(in_ptr, out_ptr, n, stream), "sage_fp8_encode_debug")


def fp8_mfma_debug(a_ptr: int, b_ptr: int, c_ptr: int, d_ptr: int, stream: int = 0) -> None:
    """d = a*b + c on the FP8 matrix core: a uint8 [32][64], b uint8 [64][32]
    (e4m3 codes), c and d fp32 [32][32], device pointers."""
    _check(lib().sage_fp8_mfma_debug(a_ptr, b_ptr, c_ptr, d_ptr, stream), "sage_fp8_mfma_debug")


def quant_smooth_varlen(q_ptr: int, k_ptr: int, v_ptr: int, in_dtype: int, cu_ptr: int, nseq: int, max_seqlen: int,
                        total: int, H: int, D: int, bufs: QuantBufs, stream: int = 0, qk_bits: int = 4,
                        smooth_v: bool = False) -> None:
    _check(lib().sage_quant_smooth_varlen(q_ptr, k_ptr, v_ptr, in_dtype, cu_ptr, nseq, max_seqlen, total, H, D,
                                          qk_bits, int(bool(smooth_v)), ctypes.byref(bufs), stream),
           "sage_quant_smooth_varlen")


def attn_quantized_varlen(bufs: QuantBufs, o_ptr: int, cu_ptr: int, nseq: int, max_seqlen: int, total: int, H: int,
                          D: int, causal: bool, sm_scale: float, out_dtype: int, stream: int = 0,
                          qk_bits: int = 4) -> None:
    _check(lib().sage_attn_quantized_varlen(ctypes.byref(bufs), o_ptr, cu_ptr, nseq, max_seqlen, total, H, D,
                                            int(bool(causal)), float(sm_scale), qk_bits, out_dtype, stream),
           "sage_attn_quantized_varlen")


def attn_fwd_varlen(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, cu_ptr: int, nseq: int, max_seqlen: int,
                    total: int, H: int, D: int, causal: bool, sm_scale: float, in_dtype: int, out_dtype: int,
                    ws_ptr: int, ws_bytes: int, stream: int = 0, qk_bits: int = 4, smooth_v: bool = False) -> None:
    _check(lib().sage_attn_fwd_varlen(q_ptr, k_ptr, v_ptr, o_ptr, cu_ptr, nseq, max_seqlen, total, H, D,
                                      int(bool(causal)), float(sm_scale), qk_bits, int(bool(smooth_v)), in_dtype,
                                      out_dtype, ws_ptr, ws_bytes, stream), "sage_attn_fwd_varlen")


def workspace_bytes_cross(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, D: int) -> int:
    return lib().sage_workspace_bytes_cross(B, Hq, Hkv, Nq, Nk, D)


def quant_bufs_from_workspace_cross(ws_ptr: int, nbytes: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int,
                                    D: int) -> QuantBufs:
    qb = QuantBufs()
    _check(lib().sage_quant_bufs_from_workspace_cross(ws_ptr, nbytes, B, Hq, Hkv, Nq, Nk, D, ctypes.byref(qb)),
           "sage_quant_bufs_from_workspace_cross")
    return qb


def quant_smooth_cross(q_ptr: int, k_ptr: int, v_ptr: int, in_dtype: int, B: int, Hq: int, Hkv: int, Nq: int,
                       Nk: int, D: int, bufs: QuantBufs, stream: int = 0, qk_bits: int = 4,
                       smooth_v: bool = False) -> None:
    _check(lib().sage_quant_smooth_cross(q_ptr, k_ptr, v_ptr, in_dtype, B, Hq, Hkv, Nq, Nk, D, qk_bits,
                                         int(bool(smooth_v)), ctypes.byref(bufs), stream), "sage_quant_smooth_cross")


def attn_fwd_cross(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int,
                   D: int, causal: bool, sm_scale: float, in_dtype: int, out_dtype: int, ws_ptr: int, ws_bytes: int,
                   stream: int = 0, qk_bits: int = 4, smooth_v: bool = False) -> None:
    _check(lib().sage_attn_fwd_cross(q_ptr, k_ptr, v_ptr, o_ptr, B, Hq, Hkv, Nq, Nk, D, int(bool(causal)),
                                     float(sm_scale), qk_bits, int(bool(smooth_v)), in_dtype, out_dtype, ws_ptr,
                                     ws_bytes, stream), "sage_attn_fwd_cross")


def attn_quantized_cross(bufs: QuantBufs, o_ptr: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int, D: int,
                         causal: bool, sm_scale: float, out_dtype: int, stream: int = 0, qk_bits: int = 4) -> None:
    _check(lib().sage_attn_quantized_cross(ctypes.byref(bufs), o_ptr, B, Hq, Hkv, Nq, Nk, D, int(bool(causal)),
                                           float(sm_scale), qk_bits, out_dtype, stream), "sage_attn_quantized_cross")


def decode_split_keys(B: int, Hq: int, Hkv: int, Nk: int, D: int) -> int:
    return lib().sage_decode_split_keys(B, Hq, Hkv, Nk, D)


def decode_workspace_bytes(B: int, Hq: int, Hkv: int, Nk: int, D: int, split_keys: int = 0) -> int:
    return lib().sage_decode_workspace_bytes(B, Hq, Hkv, Nk, D, split_keys)


def attn_decode_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, B: int, Hq: int, Hkv: int, Nk: int, D: int,
                    sm_scale: float, in_dtype: int, out_dtype: int, ws_ptr: int, ws_bytes: int, stream: int = 0,
                    smooth_v: bool = False, split_keys: int = 0) -> None:
    _check(lib().sage_attn_decode(q_ptr, k_ptr, v_ptr, o_ptr, B, Hq, Hkv, Nk, D, float(sm_scale), int(bool(smooth_v)),
                                  split_keys, in_dtype, out_dtype, ws_ptr, ws_bytes, stream), "sage_attn_decode")


def split_keys(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, D: int) -> int:
    return lib().sage_split_keys(B, Hq, Hkv, Nq, Nk, D)


def split_workspace_bytes(B: int, Hq: int, Hkv: int, Nq: int, Nk: int, D: int, split_keys: int = 0) -> int:
    return lib().sage_split_workspace_bytes(B, Hq, Hkv, Nq, Nk, D, split_keys)


def attn_fwd_split(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, B: int, Hq: int, Hkv: int, Nq: int, Nk: int,
                   D: int, causal: bool, sm_scale: float, in_dtype: int, out_dtype: int, ws_ptr: int, ws_bytes: int,
                   stream: int = 0, qk_bits: int = 4, smooth_v: bool = False, split_keys: int = 0) -> None:
    _check(lib().sage_attn_fwd_split(q_ptr, k_ptr, v_ptr, o_ptr, B, Hq, Hkv, Nq, Nk, D, int(bool(causal)),
                                     float(sm_scale), qk_bits, int(bool(smooth_v)), split_keys, in_dtype, out_dtype,
                                     ws_ptr, ws_bytes, stream), "sage_attn_fwd_split")


# ---------------------------------------------------------------- torch glue --
# Device memory and the stream handle come from torch; nothing is computed here.

def _torch_dtype_code(t) -> int:
    import torch
    return {torch.float16: F16, torch.bfloat16: BF16, torch.float32: F32}[t]


@dataclass
class Workspace:
    tensor: object      # torch.uint8 device tensor
    B: int
    H: int              # query heads
    N: int              # query tokens
    D: int
    Hkv: int = 0        # key/value heads (0: H)
    Nk: int = 0         # key/value tokens (0: N)

    @property
    def ptr(self) -> int:
        return self.tensor.data_ptr()

    @property
    def nbytes(self) -> int:
        return self.tensor.numel()

    def bufs(self) -> QuantBufs:
        return quant_bufs_from_workspace_cross(self.ptr, self.nbytes, self.B, self.H, self.Hkv or self.H, self.N,
                                               self.Nk or self.N, self.D)


def alloc_workspace(B: int, H: int, N: int, D: int, device="cuda", Hkv: int = 0, Nk: int = 0) -> Workspace:
    import torch
    n = workspace_bytes_cross(B, H, Hkv or H, N, Nk or N, D)
    if n == 0:
        raise SageError(ERR_INVALID, "sage_workspace_bytes_cross")
    return Workspace(torch.empty(n, dtype=torch.uint8, device=device), B, H, N, D, Hkv or H, Nk or N)


def _stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def attn(q, k, v, causal: bool = False, sm_scale: float | None = None, out_dtype=None, workspace: Workspace = None,
         out=None, qk_bits: int = 4, smooth_v: bool = False):
    """Drop-in attention: q [B, Hq, Nq, D], k and v [B, Hkv, Nk, D] fp16/bf16
    device tensors (Hq a multiple of Hkv; Hq == Hkv and Nq == Nk for plain
    self-attention).  qk_bits 4: INT4 Q/K codes, 8: INT8, 0 (ADAPTIVE): INT4 or
    INT8 per key/value head as the adaptive-width rule picks (the choice is in
    the workspace, see head_bits); smooth_v: subtract the V channel means
    before FP8; a causal mask is aligned at the last key."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, Nq, D] and k, v one [B, Hkv, Nk, D] shape")
    B, H, N, D = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("q, k, v must share B and D")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, N, D), dtype=out_dtype, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(B, H, N, D, q.device, Hkv=Hk, Nk=Nk)
    args = (causal, sm_scale, _torch_dtype_code(q.dtype), _torch_dtype_code(out.dtype), workspace.ptr,
            workspace.nbytes, _stream_handle(q.device), qk_bits, smooth_v)
    if Hk == H and Nk == N:
        attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, N, D, *args)
    else:
        attn_fwd_cross(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, Hk, N, Nk, D, *args)
    return out


def attn_varlen(q, k, v, cu_seqlens, max_seqlen: int, causal: bool = False, sm_scale: float | None = None,
                out_dtype=None, workspace: Workspace = None, out=None, qk_bits: int = 4, smooth_v: bool = False):
    """Packed variable-length attention: q, k, v token-major [T, H, D] fp16/bf16
    device tensors, cu_seqlens an int32 device tensor [nseq + 1] of sequence
    offsets (the form of the varlen entry point named in the code record)."""
    import torch
    if q.shape != k.shape or q.shape != v.shape or q.dim() != 3:
        raise ValueError("q, k, v must share one [T, H, D] shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    for t in (q, k, v, cu_seqlens):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v and cu_seqlens must be contiguous device tensors")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or cu_seqlens.numel() < 2:
        raise ValueError("cu_seqlens must be int32 [nseq + 1]")
    T, H, D = q.shape
    nseq = cu_seqlens.numel() - 1
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((T, H, D), dtype=out_dtype, device=q.device)
    if workspace is None:
        workspace = alloc_workspace(nseq, H, max_seqlen, D, q.device)
    attn_fwd_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), cu_seqlens.data_ptr(), nseq, max_seqlen,
                    T, H, D, causal, sm_scale, _torch_dtype_code(q.dtype), _torch_dtype_code(out.dtype),
                    workspace.ptr, workspace.nbytes, _stream_handle(q.device), qk_bits, smooth_v)
    return out


def attn_decode(q, k, v, sm_scale: float | None = None, out_dtype=None, workspace=None, out=None,
                smooth_v: bool = False, split_keys: int = 0):
    """One decoding step: q [B, Hq, 1, D], k and v [B, Hkv, Nk, D] fp16/bf16
    device tensors (Hq a multiple of Hkv).  Returns [B, Hq, 1, D].  split_keys:
    keys per range of the split-key schedule (a multiple of 128; 0 = the
    library's choice, decode_split_keys)."""
    import torch
    if q.dim() != 4 or q.shape[2] != 1 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, 1, D] and k, v one [B, Hkv, Nk, D] shape")
    B, H, _, D = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("q, k, v must share B and D")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, 1, D), dtype=out_dtype, device=q.device)
    if workspace is None:
        n = decode_workspace_bytes(B, H, Hk, Nk, D, split_keys)
        if n == 0:
            raise SageError(ERR_INVALID, "sage_decode_workspace_bytes")
        workspace = torch.empty(n, dtype=torch.uint8, device=q.device)
    attn_decode_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, Hk, Nk, D, sm_scale,
                    _torch_dtype_code(q.dtype), _torch_dtype_code(out.dtype), workspace.data_ptr(),
                    workspace.numel(), _stream_handle(q.device), smooth_v, split_keys)
    return out


def attn_split(q, k, v, causal: bool = False, sm_scale: float | None = None, out_dtype=None, out=None,
               qk_bits: int = 4, smooth_v: bool = False, split_keys: int = 0, workspace=None):
    """attn() with split key ranges (sage_attn_fwd_split): q [B, Hq, Nq, D],
    k and v [B, Hkv, Nk, D].  Returns (out, workspace tensor); the workspace
    starts with the prepass buffers of the cross geometry."""
    import torch
    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape:
        raise ValueError("q must be [B, Hq, Nq, D] and k, v one [B, Hkv, Nk, D] shape")
    B, H, N, D = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    if k.shape[0] != B or k.shape[3] != D:
        raise ValueError("q, k, v must share B and D")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.float16, torch.bfloat16):
        raise ValueError("q, k, v must all be float16 or all bfloat16")
    for t in (q, k, v):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous device tensors")
    if sm_scale is None:
        sm_scale = 1.0 / math.sqrt(D)
    out_dtype = out_dtype or q.dtype
    if out is None:
        out = torch.empty((B, H, N, D), dtype=out_dtype, device=q.device)
    if workspace is None:
        nbytes = split_workspace_bytes(B, H, Hk, N, Nk, D, split_keys)
        if nbytes == 0:
            raise SageError(ERR_INVALID, "sage_split_workspace_bytes")
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    attn_fwd_split(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), B, H, Hk, N, Nk, D, causal, sm_scale,
                   _torch_dtype_code(q.dtype), _torch_dtype_code(out.dtype), workspace.data_ptr(), workspace.numel(),
                   _stream_handle(q.device), qk_bits, smooth_v, split_keys)
    return out, workspace


def head_bits(workspace: Workspace):
    """The code width chosen for each key/value head by the last adaptive
    prepass into this workspace: int32 [B, Hkv] on the device (4 or 8)."""
    import torch
    qb = workspace.bufs()
    n = workspace.B * (workspace.Hkv or workspace.H)
    off = qb.head_bits - workspace.ptr
    return workspace.tensor[off:off + 4 * n].view(torch.int32).view(workspace.B, workspace.Hkv or workspace.H)


def adapt_stats(workspace: Workspace):
    """The adaptive-width statistics of the last adaptive prepass: fp32
    [B, Hkv, 6] = A_Q, E_Q, A_K, E_K, EV, V2 per key/value head."""
    import torch
    qb = workspace.bufs()
    hk = workspace.Hkv or workspace.H
    n = workspace.B * hk * 8
    off = qb.adapt_stat - workspace.ptr
    return workspace.tensor[off:off + 4 * n].view(torch.float32).view(workspace.B, hk, 8)[:, :, :6]
