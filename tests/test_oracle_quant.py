"""Pins for the oracle's prepass: smoothing statistics, INT4 and FP8 quantizers,
fragment-group structure of the K scales, and the compensation term.

Method (SageAttention2 abstract, arXiv 2411.10958 page): Q and K are quantized
to INT4 at a fine, hardware-friendly granularity, P~ and V to FP8, and Q is
smoothed to make INT4 QK^T accurate; the title names outlier smoothing, read
here as smoothing K as well.  Nothing below re-runs the oracle's formulas; each
check is a hand-derived value, a closed form or a property the rules imply.
"""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

from fp8_attention_transformer_amd import workloads as wl

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "quant_hand_example.json")


def _bits(x, dtype="bf16"):
    return wl.round_to_bits(np.asarray(x, np.float32), dtype)


def _build_from_golden(g):
    B, H, N, D = g["shape"]
    arrs = {}
    for name in ("q", "k", "v"):
        a = np.zeros((B, H, N, D), np.float32)
        for ch, vals in g["inputs"][name].items():
            a[0, 0, :, int(ch)] = vals
        arrs[name] = _bits(a)
    return arrs["q"], arrs["k"], arrs["v"]


def test_hand_example(oracle_lib):
    g = json.load(open(GOLDEN))
    e = g["expected"]
    q, k, v = _build_from_golden(g)
    z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16)
    D = g["shape"][3]

    def full(d):
        out = np.zeros(D, np.float32)
        for ch, val in d.items():
            out[int(ch)] = val
        return out

    assert np.array_equal(z.q_mean[0, 0, 0], full(e["q_mean_block0"]))
    assert np.array_equal(z.k_mean[0, 0], full(e["k_mean"]))
    assert np.array_equal(z.q_scale[0, 0], np.array(e["q_scale"], np.float32))
    assert np.array_equal(z.k_scale[0, 0], np.array(e["k_scale"], np.float32))
    for name, arr in (("q_codes", z.q_codes), ("k_codes", z.k_codes)):
        exp = np.zeros((4, D), np.int8)
        for ch, vals in e[name].items():
            exp[:, int(ch)] = vals
        assert np.array_equal(arr[0, 0], exp), name
    vs = np.zeros(D, np.float32)
    for ch, frac in e["v_scale"].items():
        vs[int(ch)] = np.float32(float(Fraction(frac)))
    assert np.array_equal(z.v_scale[0, 0], vs)
    vc = np.zeros((4, D), np.uint8)
    for ch, vals in e["v_codes"].items():
        vc[:, int(ch)] = vals
    assert np.array_equal(z.v_codes[0, 0], vc)
    assert np.array_equal(z.delta_s[0, 0, 0], np.array(e["delta_s_block0"], np.float32))
    acc = oracle_lib.qk_int32(z.q_codes[0, 0], z.k_codes[0, 0], 0, 0, 4, 4)
    assert np.array_equal(acc, np.array(e["qk_int32"], np.int32))


def _random_inputs(N, D, seed, dtype="bf16", B=1, H=2, **kw):
    w = wl.custom(B, H, N, D, dtype=dtype, seed=seed, **kw)
    return wl.generate(w)


@pytest.mark.parametrize("N,D", [(1, 64), (17, 64), (100, 128), (129, 64), (300, 128)])
@pytest.mark.parametrize("qk_bits", [4, 8])
def test_quantizer_properties(oracle_lib, N, D, qk_bits):
    qmax = 7 if qk_bits == 4 else 127
    q, k, v = _random_inputs(N, D, seed=N + D, k_offset_std=3.0, outlier_channels=2, outlier_scale=10.0)
    z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16, qk_bits=qk_bits)
    Q = oracle_lib.decode_input(q, 1)
    K = oracle_lib.decode_input(k, 1)
    V = oracle_lib.decode_input(v, 1)
    for codes in (z.q_codes, z.k_codes):
        assert codes.min() >= -qmax and codes.max() <= qmax
    # smoothed values rebuilt from the reported means (fp32 subtraction)
    qb = np.arange(N) // 128
    gQ = Q - z.q_mean[:, :, qb, :]
    gK = K - z.k_mean[:, :, None, :]
    # Q: reconstruction error at most half a step, and the largest |value| maps to +-7
    dq = z.q_scale[..., None]
    assert np.all(np.abs(gQ - z.q_codes * dq) <= dq * 0.5 * (1 + 2 ** -20) + 1e-30)
    tok_has_max = (np.abs(z.q_codes) == qmax).any(-1) | (z.q_scale == 0)
    assert tok_has_max.all()
    assert np.array_equal(z.q_scale, np.abs(gQ).max(-1) / np.float32(qmax))
    # K: per fragment group
    j = np.arange(N)
    grp = 2 * (j // 32) + ((j % 32) // 4) % 2
    dk = z.k_scale[:, :, grp][..., None]
    assert np.all(np.abs(gK - z.k_codes * dk) <= dk * 0.5 * (1 + 2 ** -20) + 1e-30)
    # V: the decoded FP8 value is within half an e4m3 step (relative 2^-4) or the subnormal step
    vhat = oracle_lib.e4m3_decode(z.v_codes) * z.v_scale[:, :, None, :]
    err = np.abs(vhat - V)
    assert np.all(err <= np.abs(V) * 2.0 ** -4 * 1.0001 + z.v_scale[:, :, None, :] * 2.0 ** -10 * 1.0001)
    assert np.array_equal(z.v_scale, np.abs(V).max(2) / np.float32(448))


def test_group_structure_by_perturbation(oracle_lib):
    """A single outlier key raises exactly the scale of its documented group."""
    N, D = 96, 64
    q, k, v = _random_inputs(N, D, seed=11, H=1)
    base = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16).k_scale[0, 0]
    for jj in list(range(0, 32)) + [37, 45, 66, 95]:
        k2 = k.copy()
        k2[0, 0, jj, 5] = _bits(np.float32(4000.0)).item()
        ks = oracle_lib.quant_smooth(q, k2, v, oracle_lib.DT_BF16).k_scale[0, 0]
        o = jj % 32
        g = 2 * (jj // 32) + (o // 4) % 2
        assert ks[g] > 100 * base[g], (jj, g)
        # other groups change only through the (tiny) shift of the channel mean
        others = np.delete(np.arange(ks.size), g)
        assert np.all(np.abs(ks[others] - base[others]) <= 0.2 * base[others] + 4000.0 / N / 7 * 1.01)


@pytest.mark.parametrize("N", [128, 256, 100, 300])
def test_means_closed_form(oracle_lib, N):
    """Integer-valued inputs: all sums are exact in fp32, so each mean is the
    correctly rounded quotient of an exact integer sum by the count."""
    rng = np.random.default_rng(N)
    D = 64
    Qi = rng.integers(-8, 9, (1, 1, N, D)).astype(np.float32)
    Ki = rng.integers(-8, 9, (1, 1, N, D)).astype(np.float32)
    z = oracle_lib.quant_smooth(_bits(Qi), _bits(Ki), _bits(Ki), oracle_lib.DT_BF16)
    ksum = Ki[0, 0].astype(np.int64).sum(0)
    assert np.array_equal(z.k_mean[0, 0], ksum.astype(np.float32) / np.float32(N))
    for qb in range((N + 127) // 128):
        rows = Qi[0, 0, qb * 128:(qb + 1) * 128].astype(np.int64)
        assert np.array_equal(z.q_mean[0, 0, qb], rows.sum(0).astype(np.float32) / np.float32(rows.shape[0]))


def test_sign_symmetry_and_power_of_two_scaling(oracle_lib):
    N, D = 200, 128
    q, k, v = _random_inputs(N, D, seed=3, k_offset_std=2.0)
    z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16)
    # negation: flip the sign bits of all inputs
    zn = oracle_lib.quant_smooth(q ^ 0x8000, k ^ 0x8000, v ^ 0x8000, oracle_lib.DT_BF16)
    assert np.array_equal(zn.q_codes, -z.q_codes) and np.array_equal(zn.k_codes, -z.k_codes)
    assert np.array_equal(zn.q_scale, z.q_scale) and np.array_equal(zn.k_scale, z.k_scale)
    assert np.array_equal(zn.q_mean, -z.q_mean) and np.array_equal(zn.k_mean, -z.k_mean)
    assert np.array_equal(zn.v_codes ^ 0x80, z.v_codes) or np.array_equal(
        zn.v_codes[z.v_codes != 0] ^ 0x80, z.v_codes[z.v_codes != 0])
    assert np.array_equal(zn.delta_s, z.delta_s)
    # scaling by 4 (exponent +2 in bf16, exact): codes unchanged, scales and means x4, DeltaS x16
    s = lambda a: a + np.uint16(2 << 7) * (a & 0x7FFF != 0)
    z4 = oracle_lib.quant_smooth(s(q), s(k), s(v), oracle_lib.DT_BF16)
    assert np.array_equal(z4.q_codes, z.q_codes) and np.array_equal(z4.k_codes, z.k_codes)
    assert np.array_equal(z4.q_scale, 4 * z.q_scale) and np.array_equal(z4.k_scale, 4 * z.k_scale)
    assert np.array_equal(z4.q_mean, 4 * z.q_mean) and np.array_equal(z4.k_mean, 4 * z.k_mean)
    assert np.array_equal(z4.v_codes, z.v_codes) and np.array_equal(z4.v_scale, 4 * z.v_scale)
    assert np.array_equal(z4.delta_s, 16 * z.delta_s)


def test_delta_s_definition_bound(oracle_lib):
    """DeltaS is qmean . gamma(K), rounded once: compare with an exact rational
    evaluation on a few entries."""
    N, D = 260, 64
    q, k, v = _random_inputs(N, D, seed=5, H=1, k_offset_std=4.0)
    z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16)
    K = oracle_lib.decode_input(k, 1)[0, 0]
    gK = K - z.k_mean[0, 0][None, :]
    rng = np.random.default_rng(0)
    for _ in range(20):
        qb = int(rng.integers(0, z.delta_s.shape[2]))
        j = int(rng.integers(0, N))
        exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(z.q_mean[0, 0, qb], gK[j]))
        assert z.delta_s[0, 0, qb, j] == np.float32(float(exact))


def test_zero_inputs(oracle_lib):
    z0 = np.zeros((1, 1, 40, 64), np.uint16)
    z = oracle_lib.quant_smooth(z0, z0, z0, oracle_lib.DT_BF16)
    for a in (z.q_codes, z.k_codes, z.v_codes, z.q_scale, z.k_scale, z.v_scale, z.delta_s, z.q_mean, z.k_mean):
        assert not np.any(a)


@pytest.mark.parametrize("N", [128, 300])
def test_v_smoothing_mean_and_codes(oracle_lib, N):
    """V smoothing (technical-report summary, Key Contribution 2): integer V
    gives an exact closed-form channel mean; the FP8 codes are those of
    V - mean with scale amax|V - mean| / 448; without smoothing the mean
    output is zero and the codes are unchanged from the plain prepass."""
    rng = np.random.default_rng(N + 1)
    D = 64
    Qi = rng.integers(-8, 9, (1, 1, N, D)).astype(np.float32)
    Vi = rng.integers(-8, 9, (1, 1, N, D)).astype(np.float32) + rng.integers(-20, 21, (1, 1, 1, D))
    q, v = _bits(Qi), _bits(Vi)
    z0 = oracle_lib.quant_smooth(q, q, v, oracle_lib.DT_BF16)
    z1 = oracle_lib.quant_smooth(q, q, v, oracle_lib.DT_BF16, smooth_v=True)
    assert not np.any(z0.v_mean)
    vsum = Vi[0, 0].astype(np.int64).sum(0)
    vbar = vsum.astype(np.float32) / np.float32(N)
    assert np.array_equal(z1.v_mean[0, 0], vbar)
    gV = (Vi[0, 0] - vbar).astype(np.float32)
    dv = (np.abs(gV).max(0) / np.float32(448)).astype(np.float32)
    assert np.array_equal(z1.v_scale[0, 0], dv)
    ref = oracle_lib.e4m3_encode((gV / dv).astype(np.float32))
    assert np.array_equal(z1.v_codes[0, 0], ref)
    # everything else of the prepass is untouched by V smoothing
    for f in ("q_codes", "q_scale", "k_codes", "k_scale", "q_mean", "k_mean", "delta_s"):
        assert np.array_equal(getattr(z0, f), getattr(z1, f)), f
