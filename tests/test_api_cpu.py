"""C-ABI checks that need no GPU: the library loads, exports every entry point
declared in include/sage.h, and validates arguments synchronously (every error
path below returns before anything touches a device)."""
import ctypes
import math
import os
import re

import numpy as np

import pytest

from fp8_attention_transformer_amd import sage

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
FAKE = 0x10000000  # never dereferenced: validation fails first
NF = len(sage.QuantBufs._fields_)   # arrays of a buffer set


def _declared():
    src = open(os.path.join(ROOT, "include", "sage.h")).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(sage_[a-z0-9_]+)\s*\(", src)))


def test_exports_every_declared_symbol():
    names = _declared()
    assert len(names) >= 8
    L = sage.lib()
    for n in names:
        assert hasattr(L, n), n
    assert sorted(sage.EXPORTED) == names


def test_contract_and_status_strings():
    assert sage.contract_version() == 2
    for st in (sage.OK, sage.ERR_INVALID, sage.ERR_UNSUPPORTED, sage.ERR_WORKSPACE, sage.ERR_HIP):
        assert sage.status_string(st).startswith("SAGE_")


@pytest.mark.parametrize("shape", [(0, 1, 10, 64), (1, 0, 10, 64), (1, 1, 0, 64), (1, 1, 10, 96), (1, 1, 10, 32),
                                   (1, 1, 1 << 25, 64), (1, 1, (1 << 23) + 1, 64), (1, 1, 400000, 128)])
def test_workspace_bytes_invalid(shape):
    assert sage.workspace_bytes(*shape) == 0


def test_workspace_bytes_limits():
    """The largest accepted shapes: DeltaS rows of a head below 2^30 fp32
    (N = 360000 self-attention), keys up to 2^23 against few queries."""
    assert sage.workspace_bytes(1, 1, 360000, 128) > 0
    L = sage.lib()
    assert L.sage_workspace_bytes_cross(1, 1, 1, 128, 1 << 23, 128) > 0
    assert L.sage_workspace_bytes_cross(1, 1, 1, 128, (1 << 23) + 1, 128) == 0


def _sizes(B, H, N, D):
    NP = (N + 127) // 128 * 128
    NQB = NP // 128
    BH = B * H
    return [BH * NP * D, BH * NP * D, BH * NP * 4, BH * NP // 16 * 4, BH * NQB * D * 4, BH * D * 4,
            BH * NP * D, BH * D * 4, BH * NQB * NP * 4, BH * NQB * 2 * D * 4, BH * NQB * 2 * D * 4, BH * D * 4,
            BH * NQB * 2 * D * 4, (BH * 8 + BH * NQB * 2 + BH * NQB) * 4, BH * 4]


@pytest.mark.parametrize("shape", [(1, 2, 256, 64), (4, 32, 4096, 128), (2, 48, 17776, 64), (1, 1, 1, 128)])
def test_workspace_carving(shape):
    nbytes = sage.workspace_bytes(*shape)
    sizes = _sizes(*shape)
    assert nbytes >= sum(sizes)
    base = 1 << 40
    qb = sage.quant_bufs_from_workspace(base, nbytes, *shape)
    ptrs = [getattr(qb, f) for f, _ in sage.QuantBufs._fields_]
    for p, s in zip(ptrs, sizes):
        assert p % 256 == 0 and base <= p and p + s <= base + nbytes
    spans = sorted(zip(ptrs, sizes))
    for (p0, s0), (p1, _) in zip(spans, spans[1:]):
        assert p0 + s0 <= p1
    with pytest.raises(sage.SageError) as e:
        sage.quant_bufs_from_workspace(base, nbytes - 1, *shape)
    assert e.value.status == sage.ERR_WORKSPACE
    with pytest.raises(sage.SageError) as e:
        sage.quant_bufs_from_workspace(0, nbytes, *shape)
    assert e.value.status == sage.ERR_INVALID


def _attn(**kw):
    a = dict(q=FAKE, k=FAKE + (1 << 30), v=FAKE + (2 << 30), o=FAKE + (3 << 30), B=1, H=2, N=256, D=64, causal=0,
             sm_scale=0.125, qk_bits=4, smooth_v=0, in_dtype=sage.F16, out_dtype=sage.F32, ws=FAKE + (4 << 30),
             ws_bytes=None)
    a.update(kw)
    if a["ws_bytes"] is None:
        a["ws_bytes"] = sage.workspace_bytes(a["B"], a["H"], a["N"], a["D"])
    return sage.lib().sage_attn_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["H"], a["N"], a["D"], a["causal"],
                                    a["sm_scale"], a["qk_bits"], a["smooth_v"], a["in_dtype"], a["out_dtype"], a["ws"],
                                    a["ws_bytes"], None)


@pytest.mark.parametrize("kw,expect", [
    (dict(q=None), sage.ERR_INVALID), (dict(k=None), sage.ERR_INVALID), (dict(v=None), sage.ERR_INVALID),
    (dict(o=None), sage.ERR_INVALID), (dict(ws=None), sage.ERR_INVALID), (dict(D=96), sage.ERR_INVALID),
    (dict(N=0), sage.ERR_INVALID), (dict(B=-1), sage.ERR_INVALID), (dict(sm_scale=0.0), sage.ERR_INVALID),
    (dict(sm_scale=-1.0), sage.ERR_INVALID), (dict(sm_scale=math.nan), sage.ERR_INVALID),
    (dict(sm_scale=math.inf), sage.ERR_INVALID), (dict(in_dtype=sage.F32), sage.ERR_INVALID),
    (dict(in_dtype=7), sage.ERR_INVALID), (dict(out_dtype=5), sage.ERR_INVALID),
    (dict(ws_bytes=100), sage.ERR_WORKSPACE), (dict(o=FAKE + 64), sage.ERR_INVALID),
    (dict(o=FAKE + (4 << 30) + 4096), sage.ERR_INVALID), (dict(qk_bits=-1), sage.ERR_INVALID),
    (dict(qk_bits=2), sage.ERR_INVALID), (dict(qk_bits=6), sage.ERR_INVALID), (dict(qk_bits=16), sage.ERR_INVALID),
    (dict(smooth_v=2), sage.ERR_INVALID), (dict(smooth_v=-1), sage.ERR_INVALID),
    # inputs and workspace start on a 16-byte boundary (read in 16-byte pieces)
    (dict(q=FAKE + 2), sage.ERR_INVALID), (dict(k=FAKE + (1 << 30) + 8), sage.ERR_INVALID),
    (dict(v=FAKE + (2 << 30) + 4), sage.ERR_INVALID), (dict(ws=FAKE + (4 << 30) + 8), sage.ERR_INVALID),
])
def test_attn_fwd_validation(kw, expect):
    assert _attn(**kw) == expect


def test_quant_smooth_and_debug_validation():
    L = sage.lib()
    qb = sage.QuantBufs(*([FAKE] * NF))
    assert L.sage_quant_smooth(None, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 4, 0, ctypes.byref(qb), None) == sage.ERR_INVALID
    assert L.sage_quant_smooth(FAKE, FAKE, FAKE, sage.F32, 1, 1, 10, 64, 4, 0, ctypes.byref(qb), None) == sage.ERR_INVALID
    bad = sage.QuantBufs(*([FAKE] * (NF - 1) + [0]))
    assert L.sage_quant_smooth(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 4, 0, ctypes.byref(bad), None) == sage.ERR_INVALID
    for i in range(NF):   # every array of the buffer set on a 16-byte boundary
        off = [FAKE] * NF
        off[i] = FAKE + 4
        mis = sage.QuantBufs(*off)
        assert L.sage_quant_smooth(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 4, 0, ctypes.byref(mis),
                                   None) == sage.ERR_INVALID, i
    assert L.sage_quant_smooth(FAKE + 2, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 4, 0, ctypes.byref(qb),
                               None) == sage.ERR_INVALID
    assert L.sage_quant_smooth(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 4, 0, None, None) == sage.ERR_INVALID
    dbg = L.sage_qk_int32_debug
    assert dbg(ctypes.byref(qb), 1, 1, 100, 64, 4, 0, 0, 0, 101, 4, FAKE, None) == sage.ERR_INVALID
    assert dbg(ctypes.byref(qb), 1, 1, 100, 64, 4, 1, 0, 0, 4, 4, FAKE, None) == sage.ERR_INVALID
    assert dbg(ctypes.byref(qb), 1, 1, 100, 64, 4, 0, 99, 0, 2, 4, FAKE, None) == sage.ERR_INVALID
    assert dbg(ctypes.byref(qb), 1, 1, 100, 64, 4, 0, 0, -1, 2, 4, FAKE, None) == sage.ERR_INVALID
    assert dbg(ctypes.byref(qb), 1, 1, 100, 64, 4, 0, 0, 0, 0, 4, FAKE, None) == sage.ERR_INVALID
    assert dbg(ctypes.byref(qb), 1, 1, 100, 64, 4, 0, 0, 0, 4, 4, None, None) == sage.ERR_INVALID
    assert dbg(ctypes.byref(qb), 1, 1, 100, 64, 7, 0, 0, 0, 4, 4, FAKE, None) == sage.ERR_INVALID
    assert L.sage_quant_smooth(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 3, 0, ctypes.byref(qb), None) == sage.ERR_INVALID
    assert L.sage_attn_quantized(ctypes.byref(qb), FAKE, 1, 1, 10, 64, 0, 0.125, 5, sage.F32, None) == sage.ERR_INVALID
    assert L.sage_quant_smooth(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 4, 2, ctypes.byref(qb), None) == sage.ERR_INVALID
    assert L.sage_attn_quantized(ctypes.byref(qb), FAKE, 1, 1, 10, 64, 0, 0.0, 8, sage.F32, None) == sage.ERR_INVALID
    assert L.sage_fp8_encode_debug(None, FAKE, 10, None) == sage.ERR_INVALID
    assert L.sage_fp8_encode_debug(FAKE, FAKE, 0, None) == sage.ERR_INVALID
    for i in range(4):   # every pointer of the FP8 product debug call
        ptrs = [FAKE] * 4
        ptrs[i] = None
        assert L.sage_fp8_mfma_debug(*ptrs, None) == sage.ERR_INVALID, i


def test_product_package_does_not_import_the_oracle():
    pkg = os.path.join(ROOT, "fp8_attention_transformer_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", src, re.M), f
                assert "sage_oracle" not in src, f


def test_fp6_tile_layout_helpers():
    """The test-side decoder of the FP6 code layout (include/sage.h), pinned by
    bytes worked out by hand and by a round trip."""
    import sys
    sys.path.insert(0, os.path.join(ROOT, "tests"))
    import gpu_helpers as gh
    # D = 128, row 0: channel 0 = +1 (e2m3 0b001000), channel 1 = -7 (0b111110):
    # byte 0 = 8 | (62 << 6) & 255 = 136, byte 1 = 62 >> 2 = 15; channel 32
    # (half 1) = +3 (0b010100) lands in chunk 32 at byte 0; channel 64 (group
    # 1, half 0) = -1 (0b101000) at byte 24 of chunk 0.
    codes = np.zeros((1, 32, 128), np.int8)
    codes[0, 0, 0], codes[0, 0, 1], codes[0, 0, 32], codes[0, 0, 64] = 1, -7, 3, -1
    raw = gh.codes_to_fp6_tiles(codes, 128)
    assert raw.shape == (1, 32 * 96)
    assert raw[0, 0] == 136 and raw[0, 1] == 15 and raw[0, 32 * 48] == 20 and raw[0, 24] == 40
    assert np.count_nonzero(raw) == 4
    # D = 64, row 9 (chunk 9, halves swapped): channel 0 = +2 (0b010000) at byte 16
    codes = np.zeros((1, 32, 64), np.int8)
    codes[0, 9, 0] = 2
    raw = gh.codes_to_fp6_tiles(codes, 64)
    assert raw[0, 9 * 32 + 16] == 16 and np.count_nonzero(raw) == 1
    rng = np.random.default_rng(3)
    for D in (64, 128):
        c = rng.integers(-7, 8, (2, 96, D)).astype(np.int8)
        assert np.array_equal(gh.fp6_tiles_to_codes(gh.codes_to_fp6_tiles(c, D), D), c)


def test_varlen_validation():
    L = sage.lib()
    qb = sage.QuantBufs(*([FAKE] * NF))
    qs = L.sage_quant_smooth_varlen
    ok_args = (FAKE, FAKE, FAKE, sage.BF16, FAKE, 3, 256, 500, 2, 64, 4, 0, ctypes.byref(qb), None)
    for i, bad in [(4, None), (5, 0), (6, 0), (7, 0), (9, 96), (10, 5), (11, 2), (3, sage.F32)]:
        args = list(ok_args)
        args[i] = bad
        assert qs(*args) == sage.ERR_INVALID, (i, bad)
    fwd = L.sage_attn_fwd_varlen
    ws_bytes = sage.workspace_bytes(3, 2, 256, 64)
    base = [FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE, 3, 256, 500, 2, 64, 0, 0.125, 4, 0,
            sage.BF16, sage.F32, FAKE + (4 << 30), ws_bytes, None]
    for i, bad, expect in [(4, None, sage.ERR_INVALID), (11, 0.0, sage.ERR_INVALID), (17, 100, sage.ERR_WORKSPACE),
                           (3, FAKE + 16, sage.ERR_INVALID), (5, -1, sage.ERR_INVALID), (13, 3, sage.ERR_INVALID)]:
        args = list(base)
        args[i] = bad
        assert fwd(*args) == expect, (i, bad)


def _sizes_cross(B, Hq, Hk, Nq, Nk, D):
    NPq, NPk = (Nq + 127) // 128 * 128, (Nk + 127) // 128 * 128
    NQB, NKB = NPq // 128, NPk // 128
    BHq, BHk = B * Hq, B * Hk
    part = BHk * NKB * 2 * D * 4
    return [BHq * NPq * D, BHk * NPk * D, BHq * NPq * 4, BHk * NPk // 16 * 4, BHq * NQB * D * 4, BHk * D * 4,
            BHk * NPk * D, BHk * D * 4, BHq * NQB * NPk * 4, max(part, BHq * NQB * 2 * D * 2),
            max(part, BHq * NQB * D * 2), BHk * D * 4, part, (BHk * 8 + BHq * NQB * 2 + BHk * NKB) * 4, BHk * 4]


@pytest.mark.parametrize("shape", [(1, 4, 2, 1, 8192, 128), (16, 32, 8, 1, 4096, 128), (2, 6, 3, 1000, 77, 64),
                                   (1, 2, 2, 300, 300, 64)])
def test_workspace_carving_cross(shape):
    nbytes = sage.workspace_bytes_cross(*shape)
    sizes = _sizes_cross(*shape)
    assert nbytes >= sum(sizes)
    base = 1 << 40
    qb = sage.quant_bufs_from_workspace_cross(base, nbytes, *shape)
    ptrs = [getattr(qb, f) for f, _ in sage.QuantBufs._fields_]
    for p, s in zip(ptrs, sizes):
        assert p % 256 == 0 and base <= p and p + s <= base + nbytes
    spans = sorted(zip(ptrs, sizes))
    for (p0, s0), (p1, _) in zip(spans, spans[1:]):
        assert p0 + s0 <= p1
    B, Hq, Hk, Nq, Nk, D = shape
    if Hq == Hk and Nq == Nk:   # self-attention: the dense layout, byte for byte
        assert nbytes == sage.workspace_bytes(B, Hq, Nq, D)
        dense = sage.quant_bufs_from_workspace(base, nbytes, B, Hq, Nq, D)
        assert [getattr(dense, f) for f, _ in sage.QuantBufs._fields_] == ptrs


def test_cross_validation():
    L = sage.lib()
    ws = sage.workspace_bytes_cross
    assert ws(1, 4, 3, 10, 10, 64) == 0          # Hq not a multiple of Hkv
    assert ws(1, 4, 0, 10, 10, 64) == 0
    assert ws(1, 4, 2, 10, 0, 64) == 0
    assert ws(1, 4, 2, 0, 10, 64) == 0
    assert ws(1, 4, 2, 10, 1 << 25, 64) == 0
    assert ws(1, 4, 2, 10, 10, 96) == 0
    assert ws(1, 4, 2, 1, 10, 64) > 0
    qb = sage.QuantBufs(*([FAKE] * NF))
    qs = L.sage_quant_smooth_cross
    ok = (FAKE, FAKE, FAKE, sage.BF16, 1, 4, 2, 1, 300, 64, 4, 0, ctypes.byref(qb), None)
    for i, bad in [(0, None), (3, sage.F32), (5, 3), (6, 3), (7, 0), (8, 0), (9, 96), (10, 5), (11, 2)]:
        args = list(ok)
        args[i] = bad
        assert qs(*args) == sage.ERR_INVALID, (i, bad)
    fwd = L.sage_attn_fwd_cross
    wsb = ws(1, 4, 2, 100, 300, 64)
    base = [FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), 1, 4, 2, 100, 300, 64, 1, 0.125, 4, 0,
            sage.BF16, sage.F32, FAKE + (4 << 30), wsb, None]
    for i, bad, expect in [(7, 301, sage.ERR_INVALID),       # causal with more queries than keys
                           (5, 5, sage.ERR_INVALID), (11, 0.0, sage.ERR_INVALID), (17, 100, sage.ERR_WORKSPACE),
                           (3, FAKE + 16, sage.ERR_INVALID), (12, 3, sage.ERR_INVALID), (13, 2, sage.ERR_INVALID)]:
        args = list(base)
        args[i] = bad
        assert fwd(*args) == expect, (i, bad)
    aq = L.sage_attn_quantized_cross
    assert aq(ctypes.byref(qb), FAKE, 1, 4, 2, 301, 300, 64, 1, 0.125, 4, sage.F32, None) == sage.ERR_INVALID
    assert aq(ctypes.byref(qb), FAKE, 1, 4, 3, 10, 300, 64, 0, 0.125, 4, sage.F32, None) == sage.ERR_INVALID
    assert aq(None, FAKE, 1, 4, 2, 10, 300, 64, 0, 0.125, 4, sage.F32, None) == sage.ERR_INVALID


def test_decode_validation():
    L = sage.lib()
    assert sage.decode_split_keys(16, 32, 8, 8192, 128) == 4096   # 256 workgroups: one per compute unit
    assert sage.decode_split_keys(1, 4, 3, 100, 64) == 0
    assert sage.decode_split_keys(1, 4, 2, 1, 64) == 128
    assert sage.decode_workspace_bytes(1, 4, 2, 1000, 128, 100) == 0
    assert sage.decode_workspace_bytes(1, 4, 2, 1000, 128, -128) == 0
    assert sage.decode_workspace_bytes(1, 4, 2, 1000, 128, 256) > 0
    # more ranges need more partial-output space
    assert sage.decode_workspace_bytes(1, 4, 2, 1000, 128, 128) > sage.decode_workspace_bytes(1, 4, 2, 1000, 128, 1024)
    wsb = sage.decode_workspace_bytes(1, 4, 2, 1000, 128, 0)
    base = [FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), 1, 4, 2, 1000, 128, 0.125, 0, 0, sage.BF16,
            sage.F32, FAKE + (4 << 30), wsb, None]
    for i, bad, expect in [(0, None, sage.ERR_INVALID), (6, 3, sage.ERR_INVALID), (7, 0, sage.ERR_INVALID),
                           (8, 96, sage.ERR_INVALID), (9, 0.0, sage.ERR_INVALID), (10, 2, sage.ERR_INVALID),
                           (11, 100, sage.ERR_INVALID), (12, sage.F32, sage.ERR_INVALID), (15, 64, sage.ERR_WORKSPACE),
                           (3, FAKE + 16, sage.ERR_INVALID), (14, None, sage.ERR_INVALID),
                           (0, FAKE + 2, sage.ERR_INVALID), (2, FAKE + (2 << 30) + 8, sage.ERR_INVALID),
                           (14, FAKE + (4 << 30) + 4, sage.ERR_INVALID)]:
        args = list(base)
        args[i] = bad
        assert L.sage_attn_decode(*args) == expect, (i, bad)


def test_split_validation():
    L = sage.lib()
    assert sage.split_keys(1, 32, 8, 512, 8192, 128) == 2048   # 512 workgroups: two per compute unit
    assert sage.split_keys(1, 4, 3, 10, 10, 64) == 0
    assert sage.split_workspace_bytes(1, 4, 2, 100, 1000, 128, 100) == 0
    ws_one = sage.split_workspace_bytes(1, 4, 2, 100, 1000, 128, 1024)
    assert ws_one > sage.workspace_bytes_cross(1, 4, 2, 100, 1000, 128)
    assert sage.split_workspace_bytes(1, 4, 2, 100, 1000, 128, 128) > ws_one
    wsb = sage.split_workspace_bytes(1, 4, 2, 100, 1000, 128, 0)
    base = [FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), 1, 4, 2, 100, 1000, 128, 1, 0.125, 4, 0, 0,
            sage.BF16, sage.F32, FAKE + (4 << 30), wsb, None]
    for i, bad, expect in [(7, 1001, sage.ERR_INVALID), (5, 5, sage.ERR_INVALID), (11, 0.0, sage.ERR_INVALID),
                           (14, 100, sage.ERR_INVALID), (14, -128, sage.ERR_INVALID), (12, 3, sage.ERR_INVALID),
                           (18, 100, sage.ERR_WORKSPACE), (3, FAKE + 16, sage.ERR_INVALID)]:
        args = list(base)
        args[i] = bad
        assert L.sage_attn_fwd_split(*args) == expect, (i, bad)


def test_static_entry_rejects_before_any_device_call():
    """sage_attn_fwd_static: a shape whose workspace exceeds the fixed scratch
    array returns SAGE_ERR_WORKSPACE, an invalid shape SAGE_ERR_INVALID, both
    before anything touches a device."""
    L = sage.lib()
    big = (1, 16, 16384, 128)
    assert sage.workspace_bytes(*big) > sage.STATIC_SCRATCH_BYTES
    assert sage.workspace_bytes(1, 16, 8192, 128) <= sage.STATIC_SCRATCH_BYTES
    args = lambda shape: (FAKE, FAKE, FAKE, FAKE + (1 << 30)) + shape + (0, 0.1, 4, 0, sage.BF16, sage.BF16, None)
    assert L.sage_attn_fwd_static(*args(big)) == sage.ERR_WORKSPACE
    assert L.sage_attn_fwd_static(*args((1, 1, 10, 96))) == sage.ERR_INVALID


def test_adaptive_width_validation():
    """qk_bits 0 (adaptive width): the prepass entry points that take 4 or 8
    reject it, the adaptive prepass needs a positive finite sm_scale, packed
    sequences reject it; all before any device call."""
    L = sage.lib()
    qb = sage.QuantBufs(*([FAKE] * NF))
    assert L.sage_quant_smooth(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 0, 0, ctypes.byref(qb),
                               None) == sage.ERR_INVALID
    assert L.sage_quant_smooth_cross(FAKE, FAKE, FAKE, sage.BF16, 1, 4, 2, 10, 300, 64, 0, 0, ctypes.byref(qb),
                                     None) == sage.ERR_INVALID
    qa = L.sage_quant_smooth_adaptive
    for sm in (0.0, -1.0, math.nan, math.inf):
        assert qa(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, sm, 0, ctypes.byref(qb), None) == sage.ERR_INVALID
    assert qa(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 96, 0.1, 0, ctypes.byref(qb), None) == sage.ERR_INVALID
    assert qa(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 0.1, 2, ctypes.byref(qb), None) == sage.ERR_INVALID
    assert qa(FAKE, FAKE, FAKE, sage.BF16, 1, 1, 10, 64, 0.1, 0, None, None) == sage.ERR_INVALID
    qac = L.sage_quant_smooth_adaptive_cross
    assert qac(FAKE, FAKE, FAKE, sage.BF16, 1, 4, 3, 10, 300, 64, 0.1, 0, ctypes.byref(qb), None) == sage.ERR_INVALID
    assert L.sage_quant_smooth_varlen(FAKE, FAKE, FAKE, sage.BF16, FAKE, 3, 256, 500, 2, 64, 0, 0, ctypes.byref(qb),
                                      None) == sage.ERR_INVALID
    ws_bytes = sage.workspace_bytes(3, 2, 256, 64)
    assert L.sage_attn_fwd_varlen(FAKE, FAKE + (1 << 30), FAKE + (2 << 30), FAKE + (3 << 30), FAKE, 3, 256, 500, 2,
                                  64, 0, 0.125, 0, 0, sage.BF16, sage.F32, FAKE + (4 << 30), ws_bytes,
                                  None) == sage.ERR_INVALID
    # the dense forward accepts 0 as far as argument checks go: a bad sm_scale is still caught first
    assert _attn(qk_bits=0, sm_scale=0.0) == sage.ERR_INVALID
    assert _attn(qk_bits=0, ws_bytes=100) == sage.ERR_WORKSPACE


def test_bench_counter_record_matches_source():
    """The committed traffic/counter record of the fused kernel is keyed to the
    current kernel source (bench.py reports it only then), and its fields are
    consistent: HBM bytes from the FETCH/WRITE counts and their copy factors,
    fractions within [0, 1]."""
    import json
    import bench
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["source_hash"] == bench.kernel_source_hash()
    cal = t["copy_calibration"]
    want = int(t["fetch_kib_counted"] * 1024 * cal["fetch_factor"] + t["write_kib_counted"] * 1024 * cal["write_factor"])
    assert t["bytes_per_launch"] == want
    assert bench.measured_traffic(t["workload"]) == want
    c = bench.measured_counters(t["workload"])
    assert c is not None
    for k in ("l2_hit_rate", "valu_busy_frac", "mfma_busy_frac", "mfma_overlapped_with_valu_frac", "wave_wait_frac"):
        assert 0.0 <= c[k] <= 1.0, k
    assert bench.measured_counters("no_such_workload") is None
