"""GPU parity of the adaptive code width (qk_bits 0) against the CPU oracle.

The technical-report summary page (Key Contribution 3) names an adaptive
quantization that keeps end-to-end metrics; the rule taken here (oracle
header, include/sage.h) picks INT4 or INT8 per key/value head from the
predicted INT4 logit noise.  Bit-exact: the chosen widths, the six statistics
of every head, codes, scales and means of every head at its width.  O within
max-abs 2e-3 of the oracle's mirror on every row (small cases) or on rows of
every head (full size), and cosine similarity >= 0.99 against FP32 attention
on all five workloads (the accuracy the rule is for).
"""
from __future__ import annotations

import numpy as np
import pytest

from fp8_attention_transformer_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _sdt(w):
    return 0 if w.dtype == wl.F16 else 1


def _scaled_heads(q_bits, dtype, factor, heads):
    """q with the given flattened heads multiplied by factor (re-rounded):
    low-temperature heads, which the rule gives INT4."""
    B, H, N, D = q_bits.shape
    x = wl.bits_to_f32(q_bits, dtype).reshape(B * H, N, D).copy()
    x[list(heads)] *= np.float32(factor)
    return wl.round_to_bits(x.reshape(B, H, N, D), dtype)


def _run(q, k, v, dtype, causal, sm_scale, out_dtype=None):
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    B, H, N, D = q.shape
    Hk, Nk = k.shape[1], k.shape[2]
    ws = sage.alloc_workspace(B, H, N, D, Hkv=Hk, Nk=Nk)
    ws.tensor.fill_(0xA5)   # every element the prepass owns must be written
    qd, kd, vd = (gh.to_device(a, dtype) for a in (q, k, v))
    out = sage.attn(qd, kd, vd, causal=causal, sm_scale=sm_scale, out_dtype=out_dtype or torch.float32, workspace=ws,
                    qk_bits=sage.ADAPTIVE)
    torch.cuda.synchronize()
    bits = sage.head_bits(ws).cpu().numpy()
    stats = sage.adapt_stats(ws).cpu().numpy()
    return out, ws, bits, stats


def _check(oracle_lib, w, q, k, v, ws, bits, stats):
    """Widths and statistics bit-exact; codes, scales, means of every head at its width."""
    import gpu_helpers as gh
    ob, ost = oracle_lib.adaptive_bits(q, k, v, _sdt(w), w.scale)
    print(f"[{w.name}] widths gpu={np.bincount(bits.ravel(), minlength=9)[[4, 8]]} "
          f"oracle={np.bincount(ob.ravel(), minlength=9)[[4, 8]]}")
    assert np.array_equal(bits, ob), "head widths"
    assert np.array_equal(stats, ost), "width statistics"
    z = oracle_lib.quant_smooth(q, k, v, _sdt(w), qk_bits=0, head_bits=ob)
    rb = gh.Readback(ws, qk_bits=8)
    B, H = q.shape[:2]
    Hk = k.shape[1]
    zq = lambda a: a.reshape((a.shape[0] * a.shape[1],) + a.shape[2:])
    assert np.array_equal(rb.q_codes, zq(z.q_codes)), "q codes"
    assert np.array_equal(rb.k_codes, zq(z.k_codes)), "k codes"
    assert np.array_equal(rb.q_scale, zq(z.q_scale)), "q scales"
    assert np.array_equal(rb.k_scale, zq(z.k_scale)), "k scales"
    assert np.array_equal(rb.q_mean, zq(z.q_mean)), "q means"
    assert np.array_equal(rb.k_mean, zq(z.k_mean)), "k means"
    assert np.array_equal(rb.v_codes, zq(z.v_codes)), "v codes"
    assert np.array_equal(rb.v_scale, zq(z.v_scale)), "v scales"
    # the codes of an INT4 head stay in [-7, 7]
    g = H // Hk
    for bh in range(B * H):
        if ob.reshape(-1)[(bh // H) * Hk + (bh % H) // g] == 4:
            assert np.abs(rb.q_codes[bh].astype(np.int32)).max() <= 7
    return z


SMALL = [
    wl.custom(1, 2, 300, 128, seed=201, k_offset_std=4.0, v_offset_std=1.0),
    wl.custom(1, 3, 1000, 64, causal=True, seed=202, outlier_channels=8, outlier_scale=15.0, outliers_in_k=True,
              k_offset_std=5.0),
    wl.custom(2, 2, 129, 64, dtype=wl.F16, seed=203, k_offset_std=2.0),
    wl.custom(1, 1, 17, 128, causal=True, seed=204),
]


@pytest.mark.parametrize("w", SMALL, ids=lambda w: w.name)
@pytest.mark.parametrize("mixed", [False, True])
def test_adaptive_small_every_row(oracle_lib, w, mixed):
    import gpu_helpers as gh
    q, k, v = wl.generate(w)
    if mixed:   # every other head at a quarter of its temperature: INT4 there
        q = _scaled_heads(q, w.dtype, 0.25, range(0, w.B * w.H, 2))
    out, ws, bits, stats = _run(q, k, v, w.dtype, w.causal, w.scale)
    z = _check(oracle_lib, w, q, k, v, ws, bits, stats)
    O_ref, _, _ = oracle_lib.attn_mirror(z, w.causal, w.scale)
    gh.compare_o(out.cpu().numpy().reshape(-1, w.D), O_ref, f"{w.name}/adaptive/mixed={mixed}")


def test_adaptive_mixed_widths_in_one_launch(oracle_lib):
    """Six heads, three of them low-temperature: both widths in one launch,
    bf16 output."""
    import torch
    import gpu_helpers as gh
    w = wl.custom(1, 6, 1500, 128, causal=True, seed=205, k_offset_std=4.0, outlier_channels=4, outlier_scale=6.0)
    q, k, v = wl.generate(w)
    q = _scaled_heads(q, w.dtype, 0.2, [0, 2, 5])
    out, ws, bits, stats = _run(q, k, v, w.dtype, w.causal, w.scale, out_dtype=torch.bfloat16)
    assert set(bits.ravel().tolist()) == {4, 8}, bits
    z = _check(oracle_lib, w, q, k, v, ws, bits, stats)
    O_ref, _, _ = oracle_lib.attn_mirror(z, w.causal, w.scale)
    gh.compare_o(out.float().cpu().numpy().reshape(-1, w.D), O_ref, "mixed/bf16", out_dtype="bf16")


def test_adaptive_grouped_heads_and_split(oracle_lib):
    """Grouped-query cross geometry (one width per K/V head, statistics pooled
    over its query heads) through the fused path and the split-key path."""
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    B, Hq, Hk, Nq, Nk, D = 1, 8, 2, 300, 700, 128
    rng = np.random.default_rng(206)
    Q = rng.standard_normal((B, Hq, Nq, D)).astype(np.float32)
    K = rng.standard_normal((B, Hk, Nk, D)).astype(np.float32) + 4 * rng.standard_normal(D).astype(np.float32)
    V = rng.standard_normal((B, Hk, Nk, D)).astype(np.float32)
    Q[:, :4] *= 0.2   # the query heads of K/V head 0: INT4 for that group
    q, k, v = (wl.round_to_bits(a, "bf16") for a in (Q, K, V))
    w = wl.custom(B, Hq, Nq, D, causal=True, seed=206)   # name, dtype and scale
    out, ws, bits, stats = _run(q, k, v, wl.BF16, True, w.scale)
    assert bits.tolist() == [[4, 8]], bits
    z = _check(oracle_lib, w, q, k, v, ws, bits, stats)
    O_ref, _, _ = oracle_lib.attn_mirror(z, True, w.scale)
    gh.compare_o(out.cpu().numpy().reshape(-1, D), O_ref, "gqa/adaptive")
    qd, kd, vd = (gh.to_device(a, wl.BF16) for a in (q, k, v))
    o2, _ = sage.attn_split(qd, kd, vd, causal=True, sm_scale=w.scale, out_dtype=torch.float32,
                            qk_bits=sage.ADAPTIVE, split_keys=256)
    torch.cuda.synchronize()
    O_ref2, _, _ = oracle_lib.attn_mirror(z, True, w.scale, kv_split=256)
    gh.compare_o(o2.cpu().numpy().reshape(-1, D), O_ref2, "gqa/adaptive/split")


FULL = [wl.TINY, wl.LLM, wl.DIT, wl.VIDEO, wl.long_context(8192, True), wl.HEADLINE]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_adaptive_full_size(oracle_lib, w):
    """Every head: widths, statistics, codes and scales bit-exact; O on rows of
    every head; cosine similarity against FP32 attention >= 0.99."""
    import gpu_helpers as gh
    q, k, v = wl.generate(w)
    BH = w.B * w.H
    out, ws, bits, stats = _run(q, k, v, w.dtype, w.causal, w.scale)
    z = _check(oracle_lib, w, q, k, v, ws, bits, stats)
    O_gpu = out.cpu().numpy().reshape(BH * w.N, w.D)
    del out
    rng = np.random.default_rng(w.seed)
    rows = gh.sample_rows(w.N, BH, rng)
    O_ref, _, _ = oracle_lib.attn_mirror(z, w.causal, w.scale, rows=rows)
    gh.compare_o(O_gpu[rows], O_ref, f"{w.name}/adaptive/all_heads")
    sub = rows[np.isin(rows // w.N, sorted({0, BH // 2, BH - 1}))]
    O_fp, _ = oracle_lib.attn_exact(q, k, v, _sdt(w), w.causal, w.scale, 0, rows=sub)
    c = gh.cos_sim(O_gpu[sub], O_fp)
    print(f"[{w.name}/adaptive] cos_sim vs fp32 = {c:.5f}")
    assert c >= 0.99
