"""GPU parity of the separate query / key-value geometry: decoding against a
key/value cache, chunked prefill and cross-attention (Nq != Nk), grouped-query
and multi-query heads (Hq = g * Hkv), causal masks aligned at the last key.

Bar: prepass codes, scales, means and FP8 V bit-exact against the oracle; the
compensation term within the fp32-chain bound of its bf16x3 evaluation; O
within max-abs 2e-3 of the oracle's mirror mode (element-wise, fp32 output).
"""
from __future__ import annotations

import numpy as np
import pytest

from fp8_attention_transformer_amd import workloads as wl

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
EPS_TIE = 2.0 ** -14

CASES = [
    # (B, Hq, Hkv, Nq, Nk, D, causal, qk_bits, smooth_v)
    (1, 4, 2, 1, 1000, 128, False, 4, False),      # decode, grouped heads
    (2, 8, 2, 1, 777, 64, True, 8, False),         # decode, causal (the one query sees every key)
    (1, 2, 2, 200, 1030, 128, True, 4, True),      # chunked prefill, bottom-right causal
    (1, 6, 3, 300, 77, 64, False, 4, False),       # cross-attention, more queries than keys
    (2, 4, 1, 257, 257, 128, True, 8, True),       # multi-query, square
    (1, 2, 1, 129, 4096, 128, True, 4, False),     # short chunk at the end of a long cache
    (1, 4, 4, 33, 300, 64, False, 8, True),        # plain heads, cross lengths
    # long non-causal key ranges with an even number of query blocks run two
    # query blocks per workgroup (three-deep K/V staging); ragged keys, ragged
    # queries, grouped heads
    (1, 4, 2, 256, 12900, 128, False, 4, False),
    (1, 2, 2, 250, 12500, 128, False, 8, True),
    (1, 2, 1, 256, 100, 128, False, 4, False),     # two query blocks, one (ragged) key block
]


def _id(c):
    B, Hq, Hk, Nq, Nk, D, causal, bits, sv = c
    return f"b{B}hq{Hq}hkv{Hk}nq{Nq}nk{Nk}d{D}{'_c' if causal else ''}_int{bits}{'_sv' if sv else ''}"


def _workload(c, seed):
    B, Hq, Hk, Nq, Nk, D, causal, bits, sv = c
    return wl.custom(B, Hq, Nq, D, Hkv=Hk, Nk=Nk, causal=causal, seed=seed, k_offset_std=3.0, v_offset_std=1.5,
                     outlier_channels=2, outlier_scale=8.0)


def _check_prepass(rb, z, k_bits, oracle_lib):
    B, Hq, Nq, D = z.q_codes.shape
    Hk, Nk = z.k_codes.shape[1], z.k_codes.shape[2]
    fq = lambda a: a.reshape((B * Hq,) + a.shape[2:])
    fk = lambda a: a.reshape((B * Hk,) + a.shape[2:])
    assert np.array_equal(rb.q_codes, fq(z.q_codes)), "q codes"
    assert np.array_equal(rb.q_scale, fq(z.q_scale)), "q scales"
    assert np.array_equal(rb.q_mean, fq(z.q_mean)), "q means"
    assert np.array_equal(rb.k_codes, fk(z.k_codes)), "k codes"
    assert np.array_equal(rb.k_scale, fk(z.k_scale)), "k scales"
    assert np.array_equal(rb.k_mean, fk(z.k_mean)), "k means"
    assert np.array_equal(rb.v_codes, fk(z.v_codes)), "v codes"
    assert np.array_equal(rb.v_scale, fk(z.v_scale)), "v scales"
    assert np.array_equal(rb.v_mean, fk(z.v_mean)), "v means"
    # padding: zero codes and scales past Nq / Nk, zero V bytes past Nk
    import gpu_helpers as gh
    keys = np.arange(rb.NQBk)[:, None] * 128 + gh.vperm_keys()[None, :]
    pad = keys >= Nk
    if pad.any():
        assert np.all(rb.v_codes_raw.transpose(0, 1, 3, 2)[:, pad] == 0), "padding V bytes"
    assert np.all(rb.q_scale_p[:, Nq:] == 0) and np.all(rb.q_codes_all[:, Nq:] == 0)
    assert np.all(rb.k_codes_all[:, Nk:] == 0)
    # compensation term: within (6D + 8) 2^-24 sum_c |qmean_c gamma(K)_jc|
    g = Hq // Hk
    K = oracle_lib.decode_input(k_bits, 1).reshape(B, Hk, Nk, D)
    gK = np.abs((K - z.k_mean[:, :, None, :]).astype(np.float32)).astype(np.float64)
    gK = np.repeat(gK, g, axis=1).reshape(B * Hq, Nk, D)
    qm = np.abs(z.q_mean.reshape(B * Hq, -1, D)).astype(np.float64)
    bound = (6 * D + 8) * 2.0 ** -24 * np.einsum("bqc,bjc->bqj", qm, gK)
    err = np.abs(rb.delta_s.astype(np.float64) - z.delta_s.reshape(B * Hq, -1, Nk))
    assert np.all(err <= bound + 1e-30), "compensation term"
    assert np.all(rb.delta_s_p[:, :, Nk:] == 0)


def _compare_o(O_gpu, O_ref, slack, label):
    import gpu_helpers as gh
    gh.compare_o(O_gpu, O_ref, label, slack=slack)


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_cross_parity(oracle_lib, case):
    import gpu_helpers as gh
    B, Hq, Hk, Nq, Nk, D, causal, bits, sv = case
    w = _workload(case, seed=Nq * 7 + Nk)
    q, k, v = wl.generate(w)
    z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16, qk_bits=bits, smooth_v=sv)
    # prepass alone into a poisoned workspace
    rb = gh.Readback(gh.run_quant_smooth(q, k, v, w.dtype, qk_bits=bits, smooth_v=sv), qk_bits=bits)
    _check_prepass(rb, z, k, oracle_lib)
    # the whole call
    O_ref, slack, _ = oracle_lib.attn_mirror(z, causal, w.scale, eps=EPS_TIE)
    out, ws = gh.run_attn(q, k, v, w.dtype, causal, w.scale, qk_bits=bits, smooth_v=sv)
    O_gpu = out.cpu().numpy().reshape(-1, D)
    _compare_o(O_gpu, O_ref, slack, _id(case))
    O_fp, _ = oracle_lib.attn_exact(q, k, v, 1, causal, w.scale, 0)
    c_gpu, c_orc = gh.cos_sim(O_gpu, O_fp), gh.cos_sim(O_ref, O_fp)
    print(f"[{_id(case)}] cos_sim gpu={c_gpu:.6f} oracle={c_orc:.6f}")
    assert abs(c_gpu - c_orc) < 1e-4


def test_grouped_heads_equal_repeated_kv_heads_gpu(oracle_lib):
    """Grouped-query output equals, bit for bit, the output of plain heads on
    K/V repeated along the head axis (same kernels, same arithmetic per head)."""
    import gpu_helpers as gh
    B, Hq, Hk, Nq, Nk, D = 2, 6, 2, 150, 400, 128
    w = wl.custom(B, Hq, Nq, D, Hkv=Hk, Nk=Nk, causal=True, seed=77, k_offset_std=3.0)
    q, k, v = wl.generate(w)
    kr, vr = np.repeat(k, Hq // Hk, axis=1), np.repeat(v, Hq // Hk, axis=1)
    for bits in (4, 8):
        a, _ = gh.run_attn(q, k, v, w.dtype, True, w.scale, qk_bits=bits, smooth_v=True)
        b, _ = gh.run_attn(q, kr, vr, w.dtype, True, w.scale, qk_bits=bits, smooth_v=True)
        assert np.array_equal(a.cpu().numpy(), b.cpu().numpy()), bits


def test_cross_entry_with_self_geometry_equals_dense(oracle_lib):
    import torch
    import gpu_helpers as gh
    from fp8_attention_transformer_amd import sage
    B, H, N, D = 1, 3, 300, 64
    w = wl.custom(B, H, N, D, causal=True, seed=78, k_offset_std=3.0)
    q, k, v = wl.generate(w)
    dense, _ = gh.run_attn(q, k, v, w.dtype, True, w.scale)
    qd, kd, vd = (gh.to_device(a, w.dtype) for a in (q, k, v))
    ws = sage.alloc_workspace(B, H, N, D)
    out = torch.empty((B, H, N, D), dtype=torch.float32, device="cuda")
    sage.attn_fwd_cross(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), out.data_ptr(), B, H, H, N, N, D, True, w.scale,
                        sage.BF16, sage.F32, ws.ptr, ws.nbytes, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(out, dense)


def test_cross_split_calls_equal_fwd(oracle_lib):
    """sage_quant_smooth_cross + sage_attn_quantized_cross give sage_attn_fwd_cross's output exactly."""
    import torch
    import gpu_helpers as gh
    from fp8_attention_transformer_amd import sage
    B, Hq, Hk, Nq, Nk, D = 2, 4, 2, 70, 333, 128
    w = wl.custom(B, Hq, Nq, D, Hkv=Hk, Nk=Nk, causal=True, seed=79, k_offset_std=3.0)
    q, k, v = wl.generate(w)
    ref, _ = gh.run_attn(q, k, v, w.dtype, True, w.scale)
    qd, kd, vd = (gh.to_device(a, w.dtype) for a in (q, k, v))
    ws = sage.alloc_workspace(B, Hq, Nq, D, Hkv=Hk, Nk=Nk)
    bufs = ws.bufs()
    out = torch.empty((B, Hq, Nq, D), dtype=torch.float32, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    sage.quant_smooth_cross(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), sage.BF16, B, Hq, Hk, Nq, Nk, D, bufs, sh)
    sage.attn_quantized_cross(bufs, out.data_ptr(), B, Hq, Hk, Nq, Nk, D, True, w.scale, sage.F32, sh)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)


@pytest.mark.parametrize("bits", [4, 8])
def test_chunk_full_size(oracle_lib, bits):
    """The benchmark's chunked-prefill workload (512 queries against 8192 cached
    keys, 32 query heads on 8 K/V heads, causal) through the cross-geometry
    entry points: every head's prepass bit-exact; O on rows of every query
    head."""
    import gpu_helpers as gh
    w = wl.CHUNK
    q, k, v = wl.generate(w)
    out, ws = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, qk_bits=bits)
    rb = gh.Readback(ws, qk_bits=bits)
    z_all = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16, with_delta_s=False, qk_bits=bits)
    fq = lambda a: a.reshape((w.B * w.H,) + a.shape[2:])
    fk = lambda a: a.reshape((w.B * w.hkv,) + a.shape[2:])
    for name in ("q_codes", "q_scale", "q_mean"):
        assert np.array_equal(getattr(rb, name), fq(getattr(z_all, name))), name
    for name in ("k_codes", "k_scale", "k_mean", "v_codes", "v_scale", "v_mean"):
        assert np.array_equal(getattr(rb, name), fk(getattr(z_all, name))), name
    del z_all
    O_gpu = out.cpu().numpy().reshape(w.B * w.H * w.N, w.D)
    z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16, qk_bits=bits)
    rows = gh.sample_rows(w.N, w.B * w.H, np.random.default_rng(7))
    O_ref, slack, _ = oracle_lib.attn_mirror(z, True, w.scale, rows=rows, eps=EPS_TIE)
    _compare_o(O_gpu[rows], O_ref, slack, f"{w.name}/int{bits}/all_heads")
    O_fp, _ = oracle_lib.attn_exact(q, k, v, 1, True, w.scale, 0, rows=rows)
    c_gpu, c_orc = gh.cos_sim(O_gpu[rows], O_fp), gh.cos_sim(O_ref, O_fp)
    print(f"[{w.name}/int{bits}] cos_sim gpu={c_gpu:.5f} oracle={c_orc:.5f}")
    assert abs(c_gpu - c_orc) < 1e-3
