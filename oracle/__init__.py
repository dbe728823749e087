"""CPU oracle for the SageAttention2 forward pass -- test infrastructure only.

This package is the reference that the GPU path is checked against.  It may be
imported only by ``tests/``, by ``__graft_entry__.smoke()`` and by the CPU
baseline leg of ``bench.py``.  The product package never imports it.

The arithmetic lives in ``sage_oracle.cpp`` (plain C++17, scalar loops, built
with ``-O2 -ffp-contract=off``); this module only builds it and marshals numpy
arrays through ctypes.  Which passage of the SageAttention2 pages each step
follows, and the readings taken where the pages are silent, are listed in the
header of ``sage_oracle.cpp``.

Pins (the tests under ``tests/test_oracle_*.py`` tie each function to
something other than itself):
  * e4m3 codec            -- exhaustive comparison with torch.float8_e4m3fn.
  * quant_smooth          -- hand-derived example (tests/golden), closed-form
                             means, quantizer properties, power-of-two scaling.
  * qk_int32              -- numpy int64 matrix product; closed forms.
  * attn_exact            -- direct fp64 brute force (numpy); the three
                             invariants (K mean shift, Q compensation, rows of
                             P sum to one).
  * attn_mirror           -- equals attn_exact over the same quantized operands
                             when P~ is not quantized (online softmax identity);
                             special cases Q = 0, causal row 0, one dominant key.
  * general geometry      -- (tests/test_oracle_geometry.py) cross-attention,
                             decoding and grouped-query heads against a numpy
                             fp64 brute force with the bottom-right causal mask;
                             grouped heads equal repeated K/V heads bit for bit;
                             a single query is its own block mean.
Parity unpinned: the cosine similarity against FP32 attention is a property of
the method on the synthetic inputs; the pages print no accuracy figure for it.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from dataclasses import dataclass

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sage_oracle.cpp")
_LIB = os.path.join(_HERE, "libsage_oracle.so")

BQ_MEAN = 128
BK = 128

MIRROR_QUANT_P = 1
EXACT_SMOOTH_K = 1
EXACT_SMOOTH_Q = 2
EXACT_QUANT_QK = 4
EXACT_QUANT_V = 8
EXACT_SMOOTH_V = 16

DT_F16 = 0
DT_BF16 = 1


def build(force: bool = True) -> str:
    """Compile the oracle shared library in-tree with g++."""
    if force or not os.path.exists(_LIB):
        cmd = ["g++", "-std=c++17", "-O2", "-ffp-contract=off", "-Wall", "-shared", "-fPIC",
               "-pthread", "-o", _LIB + ".tmp", _SRC]
        subprocess.run(cmd, check=True)
        os.replace(_LIB + ".tmp", _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build(force=False)
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        i32, i64, f32, f64 = ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_double
        L.oracle_contract_version.restype = i32
        L.oracle_e4m3_encode.argtypes = [P, P, i64]
        L.oracle_e4m3_decode.argtypes = [P, P, i64]
        L.oracle_decode_input.argtypes = [P, i32, P, i64]
        L.oracle_quant_smooth.argtypes = [P, P, P] + [i32] * 9 + [P] * 11 + [i32]
        L.oracle_adaptive_bits.argtypes = [P, P, P] + [i32] * 7 + [f32, P, P, i32]
        L.oracle_adaptive_bits.restype = i32
        L.oracle_quant_smooth.restype = i32
        L.oracle_qk_int32.argtypes = [P, P, i32, i32, i32, i32, i32, P]
        L.oracle_qk_int32.restype = i32
        L.oracle_attn_mirror.argtypes = [P] * 8 + [i32] * 7 + [f32, i32, i32, P, i64, f32, P, P, P, i32]
        L.oracle_attn_mirror.restype = i32
        L.oracle_attn_exact.argtypes = [P, P, P, i32] + [P] * 8 + [i32] * 7 + [f64, i32, P, i64, P, P, i32]
        L.oracle_attn_exact.restype = i32
        _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _threads(n):
    return n if n else (os.cpu_count() or 1)


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode(_ptr(x), _ptr(out), x.size)
    return out


def e4m3_decode(b: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(b, dtype=np.uint8)
    out = np.empty(b.shape, dtype=np.float32)
    lib().oracle_e4m3_decode(_ptr(b), _ptr(out), b.size)
    return out


def decode_input(bits: np.ndarray, dtype: int) -> np.ndarray:
    bits = np.ascontiguousarray(bits, dtype=np.uint16)
    out = np.empty(bits.shape, dtype=np.float32)
    lib().oracle_decode_input(_ptr(bits), dtype, _ptr(out), bits.size)
    return out


@dataclass
class Quant:
    """Canonical (unpacked, unpadded) prepass outputs.  Queries have Hq heads
    and Nq tokens, keys/values Hkv heads and Nk tokens (Hq a multiple of Hkv);
    for self-attention Hq == Hkv == H and Nq == Nk == N."""
    q_codes: np.ndarray   # int8  [B,Hq,Nq,D]
    q_scale: np.ndarray   # fp32  [B,Hq,Nq]
    k_codes: np.ndarray   # int8  [B,Hkv,Nk,D]
    k_scale: np.ndarray   # fp32  [B,Hkv,2*ceil(Nk/32)]
    q_mean: np.ndarray    # fp32  [B,Hq,ceil(Nq/128),D]
    k_mean: np.ndarray    # fp32  [B,Hkv,D]
    v_codes: np.ndarray   # uint8 [B,Hkv,Nk,D]
    v_scale: np.ndarray   # fp32  [B,Hkv,D]
    delta_s: np.ndarray   # fp32  [B,Hq,ceil(Nq/128),Nk]
    v_mean: np.ndarray = None   # fp32 [B,Hkv,D]: V channel means (zeros without V smoothing)


def adaptive_bits(q_bits, k_bits, v_bits, dtype: int, sm_scale: float, nthreads: int = 0):
    """The adaptive code width of every key/value head (the rule in the header
    of sage_oracle.cpp).  Returns (head_bits int32 [B,Hkv] of 4 or 8,
    stats fp32 [B,Hkv,6] = A_Q, E_Q, A_K, E_K, EV, V2)."""
    B, Hq, Nq, D = q_bits.shape
    _, Hk, Nk, _ = k_bits.shape
    qb_, kb_, vb_ = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q_bits, k_bits, v_bits))
    bits = np.empty((B, Hk), np.int32)
    stats = np.empty((B, Hk, 6), np.float32)
    rc = lib().oracle_adaptive_bits(_ptr(qb_), _ptr(kb_), _ptr(vb_), dtype, B, Hq, Hk, Nq, Nk, D, float(sm_scale),
                                    _ptr(bits), _ptr(stats), _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle_adaptive_bits rejected its arguments")
    return bits, stats


def quant_smooth(q_bits, k_bits, v_bits, dtype: int, nthreads: int = 0, with_delta_s: bool = True,
                 qk_bits: int = 4, smooth_v: bool = False, head_bits=None, sm_scale: float | None = None) -> Quant:
    """Run the prepass; with_delta_s=False skips the (quadratic) compensation
    term and leaves ``delta_s`` as None.  qk_bits selects INT4 (4) or INT8 (8)
    codes for Q and K, or 0: the width of each key/value head (and its query
    heads) from head_bits [B,Hkv], or, if head_bits is None, from
    adaptive_bits(..., sm_scale); smooth_v subtracts the per-channel V mean
    before FP8.  q_bits is [B,Hq,Nq,D]; k_bits and v_bits are [B,Hkv,Nk,D]."""
    B, Hq, Nq, D = q_bits.shape
    _, Hk, Nk, _ = k_bits.shape
    if k_bits.shape != v_bits.shape or k_bits.shape[0] != B or k_bits.shape[3] != D:
        raise ValueError("K and V must be [B, Hkv, Nk, D] with Q's B and D")
    nqb = (Nq + BQ_MEAN - 1) // BQ_MEAN
    G = 2 * ((Nk + 31) // 32)
    qb_, kb_, vb_ = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q_bits, k_bits, v_bits))
    hb = None
    if qk_bits == 0:
        if head_bits is None:
            if sm_scale is None:
                raise ValueError("qk_bits 0 needs head_bits or sm_scale")
            head_bits, _ = adaptive_bits(q_bits, k_bits, v_bits, dtype, sm_scale, nthreads)
        hb = np.ascontiguousarray(head_bits, dtype=np.int32).reshape(B, Hk)
    out = Quant(
        q_codes=np.empty((B, Hq, Nq, D), np.int8), q_scale=np.empty((B, Hq, Nq), np.float32),
        k_codes=np.empty((B, Hk, Nk, D), np.int8), k_scale=np.empty((B, Hk, G), np.float32),
        q_mean=np.empty((B, Hq, nqb, D), np.float32), k_mean=np.empty((B, Hk, D), np.float32),
        v_codes=np.empty((B, Hk, Nk, D), np.uint8), v_scale=np.empty((B, Hk, D), np.float32),
        delta_s=np.empty((B, Hq, nqb, Nk), np.float32) if with_delta_s else None,
        v_mean=np.empty((B, Hk, D), np.float32))
    rc = lib().oracle_quant_smooth(_ptr(qb_), _ptr(kb_), _ptr(vb_), dtype, B, Hq, Hk, Nq, Nk, D, qk_bits,
                                   int(bool(smooth_v)), _ptr(hb),
                                   _ptr(out.q_codes), _ptr(out.q_scale), _ptr(out.k_codes), _ptr(out.k_scale),
                                   _ptr(out.q_mean), _ptr(out.k_mean), _ptr(out.v_codes), _ptr(out.v_scale),
                                   _ptr(out.v_mean), _ptr(out.delta_s), _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle_quant_smooth rejected its arguments")
    return out


def qk_int32(q_codes_head, k_codes_head, q0, k0, nq, nk) -> np.ndarray:
    qc = np.ascontiguousarray(q_codes_head, dtype=np.int8)
    kc = np.ascontiguousarray(k_codes_head, dtype=np.int8)
    D = qc.shape[-1]
    out = np.empty((nq, nk), np.int32)
    rc = lib().oracle_qk_int32(_ptr(qc), _ptr(kc), D, q0, k0, nq, nk, _ptr(out))
    if rc != 0:
        raise ValueError("oracle_qk_int32 rejected its arguments")
    return out


def attn_mirror(qz: Quant, causal: bool, sm_scale: float, rows=None, quant_p: bool = True,
                eps: float = 0.0, nthreads: int = 0, kv_split: int = 0):
    """Returns (O [nrows, D] fp32, slack [nrows] fp32, lse [nrows, 2] fp32).
    rows index the flattened [B, Hq, Nq] query grid.  kv_split > 0 (a multiple
    of 128): keys in ranges of kv_split, each with its own online softmax,
    merged at the end (the split-key schedule)."""
    B, H, N, D = qz.q_codes.shape
    Hk, Nk = qz.k_codes.shape[1], qz.k_codes.shape[2]
    if rows is None:
        nrows = B * H * N
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    O = np.empty((nrows, D), np.float32)
    slack = np.empty(nrows, np.float32)
    lse = np.empty((nrows, 2), np.float32)
    rc = lib().oracle_attn_mirror(_ptr(qz.q_codes), _ptr(qz.q_scale), _ptr(qz.k_codes), _ptr(qz.k_scale),
                                  _ptr(qz.v_codes), _ptr(qz.v_scale), _ptr(qz.v_mean), _ptr(qz.delta_s),
                                  B, H, Hk, N, Nk, D, int(causal), float(sm_scale),
                                  MIRROR_QUANT_P if quant_p else 0, int(kv_split), _ptr(rows_arr), nrows,
                                  float(eps),
                                  _ptr(O), _ptr(slack), _ptr(lse), _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_mirror rejected its arguments")
    return O, slack, lse


def attn_exact(q_bits, k_bits, v_bits, dtype: int, causal: bool, sm_scale: float, flags: int,
               qz: Quant | None = None, rows=None, nthreads: int = 0):
    """Returns (O [nrows, D] fp64, row sums of P [nrows] fp64).  q_bits is
    [B,Hq,Nq,D], k_bits and v_bits [B,Hkv,Nk,D]; rows index [B, Hq, Nq]."""
    B, H, N, D = q_bits.shape
    Hk, Nk = k_bits.shape[1], k_bits.shape[2]
    qb_, kb_, vb_ = (np.ascontiguousarray(a, dtype=np.uint16) for a in (q_bits, k_bits, v_bits))
    if rows is None:
        nrows = B * H * N
        rows_arr = None
    else:
        rows_arr = np.ascontiguousarray(rows, dtype=np.int64)
        nrows = rows_arr.size
    O = np.empty((nrows, D), np.float64)
    psum = np.empty(nrows, np.float64)
    z = qz if qz is not None else Quant(*([None] * 9))
    rc = lib().oracle_attn_exact(_ptr(qb_), _ptr(kb_), _ptr(vb_), dtype,
                                 _ptr(z.q_codes), _ptr(z.q_scale), _ptr(z.k_codes), _ptr(z.k_scale),
                                 _ptr(z.v_codes), _ptr(z.v_scale), _ptr(z.v_mean), _ptr(z.delta_s),
                                 B, H, Hk, N, Nk, D, int(causal), float(sm_scale), flags, _ptr(rows_arr), nrows,
                                 _ptr(O), _ptr(psum), _threads(nthreads))
    if rc != 0:
        raise ValueError("oracle_attn_exact rejected its arguments")
    return O, psum
