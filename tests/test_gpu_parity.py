"""GPU parity: libsage (HIP, gfx950) against the CPU oracle, through the C ABI.

Both code widths of Q and K (qk_bits 4: INT4, 8: INT8) are covered.
Bit-exact: Q/K codes, all scales, means, FP8 V codes, int32 QK^T (also at its
closed-form extremes).  Toleranced: the compensation term (fp32 vs the oracle's
fp64 accumulation, bound derived from the fp32 chain) and O: max-abs 2e-3
element-wise for fp32 outputs, plus half an output ulp for 16-bit outputs (the
output rounding only).  Small cases cover every row; the full-size workloads
run in the same launch configuration as the benchmark and are compared on
rows of every head (first, last, block edges, tail block, a causal pair of
query blocks and random rows).
"""
from __future__ import annotations

import numpy as np
import pytest

from fp8_attention_transformer_amd import workloads as wl

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
EPS_TIE = 2.0 ** -14   # midpoint window of the mirror's diagnostic slack (no effect on the bar)

SMALL = [
    wl.TINY,
    wl.custom(1, 1, 1, 64, seed=101),
    wl.custom(1, 2, 17, 64, causal=True, seed=102, k_offset_std=3.0),
    wl.custom(1, 1, 100, 128, causal=True, seed=103, k_offset_std=4.0, outlier_channels=4, outlier_scale=20.0),
    wl.custom(2, 1, 129, 64, dtype=wl.F16, seed=104, k_offset_std=2.0),
    wl.custom(1, 2, 300, 128, seed=105, k_offset_std=4.0, v_offset_std=1.0),
    wl.custom(1, 1, 640, 128, causal=True, seed=106, t_noise_scale=0.5, k_offset_std=4.0),
    wl.custom(1, 3, 1000, 64, causal=True, seed=107, outlier_channels=8, outlier_scale=15.0, outliers_in_k=True,
              k_offset_std=5.0),
    # D = 128, non-causal, two query blocks (one 8-wave workgroup per pair): a
    # two-block key range with ragged queries and keys
    wl.custom(1, 2, 200, 128, seed=108, k_offset_std=3.0, v_offset_std=1.0),
]
FULL = [wl.LLM, wl.DIT, wl.VIDEO] + wl.LONG
FULL_CASES = [(w, 4) for w in FULL] + [(w, 8) for w in (wl.LLM, wl.VIDEO, wl.HEADLINE)]
BITS = [4, 8]


def _id(w):
    return w.name + ("_c" if w.causal else "")


def _sdt(w):
    return 0 if w.dtype == wl.F16 else 1


def _check_prepass(rb, z):
    """rb: GPU readback; z: oracle Quant for the same heads."""
    B, H, N, D = z.q_codes.shape
    zq = lambda a: a.reshape((B * H,) + a.shape[2:])
    assert np.array_equal(rb.q_codes, zq(z.q_codes)), "q codes"
    assert np.array_equal(rb.k_codes, zq(z.k_codes)), "k codes"
    assert np.array_equal(rb.q_scale, zq(z.q_scale)), "q scales"
    assert np.array_equal(rb.k_scale, zq(z.k_scale)), "k scales"
    assert np.array_equal(rb.q_mean, zq(z.q_mean)), "q means"
    assert np.array_equal(rb.k_mean, zq(z.k_mean)), "k means"
    assert np.array_equal(rb.v_scale, zq(z.v_scale)), "v scales"
    assert np.array_equal(rb.v_codes, zq(z.v_codes)), "v codes"
    assert np.array_equal(rb.v_mean, zq(z.v_mean)), "v means"
    # padding rows: zero codes and zero scales; padding keys of V are zero bytes
    keys = (np.arange(rb.NQB)[:, None] * 128 + gh_vperm(D)[None, :])            # [NQB, 128] key of each position
    pad = keys >= N
    if pad.any():
        assert np.all(rb.v_codes_raw.transpose(0, 1, 3, 2)[:, pad] == 0), "padding V bytes"
    assert np.all(rb.q_scale_p[:, N:] == 0)
    assert np.all(rb.q_codes_all[:, N:] == 0) and np.all(rb.k_codes_all[:, N:] == 0)
    if rb.qk_bits == 4:
        # every stored byte is the layout's encoding of the codes (pad bytes zero)
        import gpu_helpers as gh
        assert np.array_equal(rb.q_codes_raw, gh.codes_to_fp6_tiles(rb.q_codes_all, D)), "q FP6 layout"
        assert np.array_equal(rb.k_codes_raw, gh.codes_to_fp6_tiles(rb.k_codes_all, D)), "k FP6 layout"


def _ds_bound(oracle_lib, z, k_bits, dtype_code):
    """Error bound of the GPU compensation term, per entry:
    (6*D + 8) * 2^-24 * sum_c |qmean_c * gamma(K)_jc|.
    The GPU splits each fp32 operand into three bf16 pieces (residual at most
    2^-24 relative) and accumulates the six products x_a*y_b with a+b <= 4 in
    fp32: the dropped products and residuals cost at most ~5 * 2^-24 per term,
    and fp32 accumulation of 6*D products in any order at most 6*D * 2^-24."""
    B, H, N, D = z.q_codes.shape
    K = oracle_lib.decode_input(k_bits, dtype_code).reshape(B * H, N, D)
    gK = np.abs((K - z.k_mean.reshape(B * H, 1, D)).astype(np.float32)).astype(np.float64)
    qm = np.abs(z.q_mean.reshape(B * H, -1, D)).astype(np.float64)
    return (6 * D + 8) * 2.0 ** -24 * np.einsum("bqc,bjc->bqj", qm, gK)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("w", SMALL, ids=_id)
def test_prepass_bitexact_small(oracle_lib, w, bits):
    import gpu_helpers as gh
    q, k, v = wl.generate(w)
    z = oracle_lib.quant_smooth(q, k, v, _sdt(w), qk_bits=bits)
    rb = gh.Readback(gh.run_quant_smooth(q, k, v, w.dtype, qk_bits=bits), qk_bits=bits)
    _check_prepass(rb, z)
    # compensation term within the fp32-chain bound
    err = np.abs(rb.delta_s.astype(np.float64) - z.delta_s.reshape(w.B * w.H, -1, w.N))
    assert np.all(err <= _ds_bound(oracle_lib, z, k, _sdt(w)) + 1e-30)
    # padded key columns are zero
    assert np.all(rb.delta_s_p[:, :, w.N:] == 0)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("w", SMALL, ids=_id)
def test_qk_int32_bitexact_small(oracle_lib, w, bits):
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    q, k, v = wl.generate(w)
    z = oracle_lib.quant_smooth(q, k, v, _sdt(w), with_delta_s=False, qk_bits=bits)
    ws = gh.run_quant_smooth(q, k, v, w.dtype, qk_bits=bits)
    N = w.N
    for bh in range(w.B * w.H):
        out = torch.empty((N, N), dtype=torch.int32, device="cuda")
        sage.qk_int32_debug(ws.bufs(), w.B, w.H, N, w.D, bh, 0, 0, N, N, out.data_ptr(), qk_bits=bits)
        qc = z.q_codes.reshape(-1, N, w.D)[bh]
        kc = z.k_codes.reshape(-1, N, w.D)[bh]
        ref = oracle_lib.qk_int32(qc, kc, 0, 0, N, N)
        assert np.array_equal(out.cpu().numpy(), ref)
    # an interior window with ragged edges
    if N >= 40:
        out = torch.empty((N - 7 - 3, N - 11 - 2), dtype=torch.int32, device="cuda")
        sage.qk_int32_debug(ws.bufs(), w.B, w.H, N, w.D, 0, 7, 11, N - 10, N - 13, out.data_ptr(), qk_bits=bits)
        ref = oracle_lib.qk_int32(z.q_codes.reshape(-1, N, w.D)[0], z.k_codes.reshape(-1, N, w.D)[0], 7, 11,
                                  N - 10, N - 13)
        assert np.array_equal(out.cpu().numpy(), ref)


def gh_vperm(D):
    import gpu_helpers as gh
    return gh.vperm_keys()


def _compare_o(O_gpu, O_ref, slack, label, out_dtype="f32"):
    import gpu_helpers as gh
    return gh.compare_o(O_gpu, O_ref, label, out_dtype, slack)


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("w", SMALL, ids=_id)
def test_attention_parity_small(oracle_lib, w, bits):
    import gpu_helpers as gh
    q, k, v = wl.generate(w)
    z = oracle_lib.quant_smooth(q, k, v, _sdt(w), qk_bits=bits)
    O_ref, slack, _ = oracle_lib.attn_mirror(z, w.causal, w.scale, eps=EPS_TIE)
    out, ws = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, qk_bits=bits)
    O_gpu = out.cpu().numpy().reshape(-1, w.D)
    _compare_o(O_gpu, O_ref, slack, f"{w.name}/int{bits}")
    # the workspace of the attention call holds the same prepass
    rb = gh.Readback(ws, qk_bits=bits)
    _check_prepass(rb, z)
    # cos-sim against FP32 attention equals the method's own (oracle) value
    O_fp, _ = oracle_lib.attn_exact(q, k, v, _sdt(w), w.causal, w.scale, 0)
    c_gpu, c_orc = gh.cos_sim(O_gpu, O_fp), gh.cos_sim(O_ref, O_fp)
    print(f"[{w.name}/int{bits}] cos_sim gpu={c_gpu:.5f} oracle={c_orc:.5f}")
    assert abs(c_gpu - c_orc) < 1e-4


@pytest.mark.parametrize("w", SMALL[:4], ids=_id)
def test_low_precision_outputs(oracle_lib, w):
    """bf16 / fp16 outputs: the bar plus the output's own rounding (half an
    ulp at |O|), nothing else."""
    import torch
    import gpu_helpers as gh
    q, k, v = wl.generate(w)
    z = oracle_lib.quant_smooth(q, k, v, _sdt(w))
    O_ref, slack, _ = oracle_lib.attn_mirror(z, w.causal, w.scale, eps=EPS_TIE)
    for dt, name in ((torch.bfloat16, "bf16"), (torch.float16, "f16")):
        out, _ = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, out_dtype=dt)
        O_gpu = out.float().cpu().numpy().reshape(-1, w.D)
        _compare_o(O_gpu, O_ref, slack, f"{w.name}-{name}", out_dtype=name)


@pytest.mark.parametrize("bits", BITS)
def test_determinism(oracle_lib, bits):
    import gpu_helpers as gh
    w = SMALL[6]
    q, k, v = wl.generate(w)
    a, _ = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, qk_bits=bits)
    b, _ = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, qk_bits=bits)
    assert np.array_equal(a.cpu().numpy(), b.cpu().numpy())


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("causal", [False, True])
def test_result_independent_of_grid(oracle_lib, bits, causal):
    """A head's output does not depend on the rest of the launch: heads run
    inside a batch of six (other workgroup numbering, XCD placement and, for
    causal calls with few query blocks, pairing) equal the same heads run
    alone, bit for bit."""
    import gpu_helpers as gh
    w = wl.custom(2, 3, 1100, 128, causal=causal, seed=151, k_offset_std=3.0, t_noise_scale=0.5)
    q, k, v = wl.generate(w)
    full, _ = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, qk_bits=bits)
    full = full.cpu().numpy()
    for b_, h_ in ((0, 0), (1, 2), (0, 1)):
        one = lambda a: np.ascontiguousarray(a[b_:b_ + 1, h_:h_ + 1])
        alone, _ = gh.run_attn(one(q), one(k), one(v), w.dtype, w.causal, w.scale, qk_bits=bits)
        assert np.array_equal(alone.cpu().numpy()[0, 0], full[b_, h_]), (b_, h_)


def test_fp8_conversion_matches_oracle(oracle_lib):
    """The device e4m3 conversion used for V and P~ equals the oracle codec on a
    dense sweep of [0, 464] (every 3rd fp32 bit pattern plus neighbourhoods of
    every midpoint) and on negatives."""
    import torch
    from fp8_attention_transformer_amd import sage
    hi = int(np.array([464.0], np.float32).view(np.uint32)[0])
    mids = []
    grid = oracle_lib.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    for a, b in zip(grid[:-1], grid[1:]):
        m = np.float32((np.float64(a) + np.float64(b)) / 2)
        mb = int(np.array([m], np.float32).view(np.uint32)[0])
        mids.append(np.arange(mb - 64, mb + 65, dtype=np.uint32))
    parts = [np.concatenate(mids)]
    chunk = 1 << 25
    for start in range(0, hi + 1, chunk * 3):
        parts_bits = np.arange(start, min(start + chunk * 3, hi + 1), 3, dtype=np.uint32)
        x = parts_bits.view(np.float32)
        for sgn in (1.0, -1.0) if start == 0 else (1.0,):
            xs = (x * np.float32(sgn)).astype(np.float32)
            dev_in = torch.from_numpy(xs).cuda()
            dev_out = torch.empty(xs.size, dtype=torch.uint8, device="cuda")
            sage.fp8_encode_debug(dev_in.data_ptr(), dev_out.data_ptr(), xs.size)
            got = dev_out.cpu().numpy()
            ref = oracle_lib.e4m3_encode(xs)
            bad = np.nonzero(got != ref)[0]
            assert bad.size == 0, (xs[bad[:5]], got[bad[:5]], ref[bad[:5]])
    x = parts[0].view(np.float32)
    dev_in = torch.from_numpy(x).cuda()
    dev_out = torch.empty(x.size, dtype=torch.uint8, device="cuda")
    sage.fp8_encode_debug(dev_in.data_ptr(), dev_out.data_ptr(), x.size)
    assert np.array_equal(dev_out.cpu().numpy(), oracle_lib.e4m3_encode(x))


@pytest.mark.parametrize("w,bits", FULL_CASES, ids=lambda c: c.name if hasattr(c, "name") else f"int{c}")
def test_full_size_parity(oracle_lib, w, bits):
    """The benchmark's workload and launch: all heads on the GPU; codes and
    scales of every head bit-exact; O compared on rows of every head (first,
    last, block edges, tail block, a causal pair of query blocks, random
    rows); the compensation term and int32 tiles on the first and last head."""
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    q, k, v = wl.generate(w)
    BH = w.B * w.H
    out, ws = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, qk_bits=bits)
    rb = gh.Readback(ws, qk_bits=bits)
    z_all = oracle_lib.quant_smooth(q, k, v, _sdt(w), qk_bits=bits)
    _check_prepass(rb, z_all)
    O_gpu_all = out.cpu().numpy().reshape(BH * w.N, w.D)
    del out
    rng = np.random.default_rng(w.seed)
    rows = gh.sample_rows(w.N, BH, rng)
    O_ref, slack, _ = oracle_lib.attn_mirror(z_all, w.causal, w.scale, rows=rows, eps=EPS_TIE)
    _compare_o(O_gpu_all[rows], O_ref, slack, f"{w.name}/int{bits}/all_heads")
    heads_seen = np.unique(rows // w.N)
    assert heads_seen.size == BH
    # cos-sim against FP32 attention on the rows of a few heads equals the method's own
    sub = rows[np.isin(rows // w.N, [0, BH // 2, BH - 1])]
    O_fp, _ = oracle_lib.attn_exact(q, k, v, _sdt(w), w.causal, w.scale, 0, rows=sub)
    c_gpu = gh.cos_sim(O_gpu_all[sub], O_fp)
    c_orc = gh.cos_sim(O_ref[np.isin(rows, sub)], O_fp)
    print(f"[{w.name}/int{bits}] cos_sim gpu={c_gpu:.5f} oracle={c_orc:.5f}")
    assert abs(c_gpu - c_orc) < 1e-3
    for bh in (0, BH - 1):
        qs, kk, vs = (a.reshape(BH, 1, w.N, w.D)[bh:bh + 1] for a in (q, k, v))
        # compensation term within the fp32-chain bound
        zh = oracle_lib.quant_smooth(qs, kk, vs, _sdt(w), qk_bits=bits)
        err = np.abs(rb.delta_s[bh].astype(np.float64) - zh.delta_s[0, 0])
        assert np.all(err <= _ds_bound(oracle_lib, zh, kk, _sdt(w))[0] + 1e-30)
        # int32 tiles: first, last, tail and random windows
        wins = [(0, 0), (w.N - 64, w.N - 64), (0, w.N - 64)] + [tuple(rng.integers(0, w.N - 64, 2)) for _ in range(4)]
        for q0, k0 in wins:
            o32 = torch.empty((64, 64), dtype=torch.int32, device="cuda")
            sage.qk_int32_debug(ws.bufs(), w.B, w.H, w.N, w.D, bh, int(q0), int(k0), 64, 64, o32.data_ptr(),
                                qk_bits=bits)
            ref = oracle_lib.qk_int32(zh.q_codes[0, 0], zh.k_codes[0, 0], int(q0), int(k0), 64, 64)
            assert np.array_equal(o32.cpu().numpy(), ref)


def _closed_form_inputs(N, D, pattern, qk_bits, seed=0):
    """bf16 Q and K whose codes are known in closed form: every token is +-a on
    all channels (sign per token, block means zero by pairing tokens), so the
    per-token and per-group amax is a and every code is +-qmax.  pattern:
    'same' (K like Q), 'neg' (K = -Q sign pattern), 'alt' (K alternates sign
    across channels)."""
    rng = np.random.default_rng(seed)
    assert N % 2 == 0
    sq = rng.choice([-1.0, 1.0], N // 2)
    sq = np.concatenate([sq, -sq])[rng.permutation(N)].astype(np.float32)   # zero mean per 128 block? checked below
    Q = np.repeat((1.5 * sq)[:, None], D, 1)
    if pattern == "same":
        K = np.ones((N, D), np.float32) * 0.75
    elif pattern == "neg":
        K = -np.ones((N, D), np.float32) * 0.75
    else:
        K = np.tile(np.array([0.75, -0.75], np.float32), (N, D // 2))
    K = K * np.concatenate([np.ones(N // 2), -np.ones(N // 2)])[:, None].astype(np.float32)
    V = rng.standard_normal((N, D)).astype(np.float32)
    return Q[None, None], K[None, None], V[None, None]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("D", [64, 128])
def test_qk_closed_forms(oracle_lib, bits, D):
    """int32 QK^T at its extremes through the prepass and the kernel's tile
    routine: codes +-qmax on every channel give +-qmax^2*D exactly (49*D for
    INT4, 16129*D for INT8), and a sign pattern alternating across channels
    gives 0."""
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    qmax = 7 if bits == 4 else 127
    N = 256
    for pattern in ("same", "neg", "alt"):
        Q, K, V = _closed_form_inputs(N, D, pattern, bits, seed=D + bits)
        bf = lambda x: wl.round_to_bits(x, "bf16")
        q, k, v = bf(Q), bf(K), bf(V)
        z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16, with_delta_s=False, qk_bits=bits)
        # the construction really gives +-qmax codes (smoothing removes nothing from Q: its block means are
        # not forced to zero, so only the per-token sign pattern of Q - mean is checked through the codes)
        ws = gh.run_quant_smooth(q, k, v, wl.BF16, qk_bits=bits)
        rb = gh.Readback(ws, qk_bits=bits)
        assert np.array_equal(rb.q_codes[0], z.q_codes[0, 0]) and np.array_equal(rb.k_codes[0], z.k_codes[0, 0])
        kc = z.k_codes[0, 0].astype(np.int64)
        assert np.all(np.abs(kc) == qmax), "K codes are +-qmax"
        out = torch.empty((N, N), dtype=torch.int32, device="cuda")
        sage.qk_int32_debug(ws.bufs(), 1, 1, N, D, 0, 0, 0, N, N, out.data_ptr(), qk_bits=bits)
        got = out.cpu().numpy().astype(np.int64)
        qc = z.q_codes[0, 0].astype(np.int64)
        full_q = np.all(np.abs(qc) == qmax, axis=1)            # tokens whose codes are all +-qmax
        assert full_q.sum() >= N // 4
        sq = np.sign(qc[:, 0])
        sk = np.sign(kc[:, 0])
        if pattern == "alt":
            expect = np.zeros((N, N), np.int64)
        else:
            expect = np.outer(sq, sk) * qmax * qmax * D
        assert np.array_equal(got[full_q], expect[full_q]), pattern
        assert np.array_equal(got, qc @ kc.T)


@pytest.mark.parametrize("bits", BITS)
def test_subnormal_scale_codes_clamped(oracle_lib, bits):
    """Codes are clamp(rint(x / delta), -qmax, qmax) even when delta = amax/qmax
    rounds down among the fp32 subnormals.  One K channel holds m tokens of
    the smallest bf16 subnormal (2^-133) among 40000 zeros, so its mean is
    RN(m * 2^-133 / 40000) = 10 * 2^-149 (INT4, m = 6) or 190 * 2^-149 (INT8,
    m = 116); a 16-key group of zeros then has amax = that mean and delta =
    2^-149, and x / delta reaches -10 (-190) before the clamp."""
    import gpu_helpers as gh
    N, D = 40000, 64
    m, units = (6, 10) if bits == 4 else (116, 190)
    rng = np.random.default_rng(17)
    k = np.zeros((1, 1, N, D), np.uint16)
    k[0, 0, :m, 5] = 0x0001                                      # bf16 2^-133
    q = wl.round_to_bits(rng.standard_normal((1, 1, N, D)).astype(np.float32), "bf16")
    v = wl.round_to_bits(rng.standard_normal((1, 1, N, D)).astype(np.float32), "bf16")
    z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16, with_delta_s=False, qk_bits=bits)
    assert z.k_mean[0, 0, 5] == np.float32(units * 2.0 ** -149)
    # keys from 128 on are zeros: their groups' delta rounds to one subnormal unit
    assert np.all(z.k_scale[0, 0, 8:] == np.float32(2.0 ** -149))
    qmax = 7 if bits == 4 else 127
    assert np.all(z.k_codes[0, 0, 128:, 5] == -qmax), "the clamp decides these codes"
    rb = gh.Readback(gh.run_quant_smooth(q, k, v, wl.BF16, qk_bits=bits), qk_bits=bits)
    _check_prepass(rb, z)


SMOOTH_V_CASES = [SMALL[3], SMALL[4], SMALL[5], SMALL[7],
                  wl.custom(1, 2, 333, 128, seed=108, k_offset_std=3.0, v_offset_std=4.0)]


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("w", SMOOTH_V_CASES, ids=_id)
def test_smooth_v_parity_small(oracle_lib, w, bits):
    """V smoothing: prepass bit-exact (V means, scales of V - mean, FP8 codes)
    and O within the bar against the oracle's mirror with the mean added back."""
    import gpu_helpers as gh
    q, k, v = wl.generate(w)
    z = oracle_lib.quant_smooth(q, k, v, _sdt(w), qk_bits=bits, smooth_v=True)
    O_ref, slack, _ = oracle_lib.attn_mirror(z, w.causal, w.scale, eps=EPS_TIE)
    out, ws = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, qk_bits=bits, smooth_v=True)
    rb = gh.Readback(ws, qk_bits=bits)
    _check_prepass(rb, z)
    O_gpu = out.cpu().numpy().reshape(-1, w.D)
    _compare_o(O_gpu, O_ref, slack, f"{w.name}/int{bits}/smooth_v")
    O_fp, _ = oracle_lib.attn_exact(q, k, v, _sdt(w), w.causal, w.scale, 0)
    c_gpu, c_orc = gh.cos_sim(O_gpu, O_fp), gh.cos_sim(O_ref, O_fp)
    print(f"[{w.name}/int{bits}/smooth_v] cos_sim gpu={c_gpu:.5f} oracle={c_orc:.5f}")
    assert abs(c_gpu - c_orc) < 1e-4


def test_smooth_v_full_size_dit(oracle_lib):
    """The DiT workload (V carries a per-channel offset) with V smoothing, in
    the benchmark's launch: prepass of every head bit-exact, O on sampled rows
    of the first and last head."""
    import gpu_helpers as gh
    w = wl.DIT
    q, k, v = wl.generate(w)
    BH = w.B * w.H
    out, ws = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, smooth_v=True)
    rb = gh.Readback(ws)
    z_all = oracle_lib.quant_smooth(q, k, v, _sdt(w), with_delta_s=False, smooth_v=True)
    _check_prepass(rb, z_all)
    del z_all
    O_gpu_all = out.cpu().numpy().reshape(BH * w.N, w.D)
    z = oracle_lib.quant_smooth(q, k, v, _sdt(w), smooth_v=True)
    rows = gh.sample_rows(w.N, BH, np.random.default_rng(w.seed))
    O_ref, slack, _ = oracle_lib.attn_mirror(z, w.causal, w.scale, rows=rows, eps=EPS_TIE)
    _compare_o(O_gpu_all[rows], O_ref, slack, f"{w.name}/smooth_v/all_heads")


@pytest.mark.parametrize("bits", BITS)
@pytest.mark.parametrize("smooth_v", [False, True])
def test_signed_zeros_and_zero_channels(oracle_lib, bits, smooth_v):
    """Codes of signed zeros: V entries of -0 keep the sign of their FP8 code
    (0x80), a V channel of zeros only (scale 0) gives +0 codes, and Q/K zeros
    give code 0; every prepass array bit-exact against the oracle."""
    import gpu_helpers as gh
    w = wl.custom(2, 2, 300, 128, seed=131, k_offset_std=2.0, v_offset_std=0.0)
    q, k, v = (a.copy() for a in wl.generate(w))
    rng = np.random.default_rng(5)
    for a in (q, k, v):
        m = rng.random(a.shape) < 0.05
        a[m] = np.where(rng.random(m.sum()) < 0.5, 0x8000, 0x0000)       # bf16 -0 / +0
    v[0, 1, :, 7] = np.where(rng.random(w.N) < 0.5, 0x8000, 0x0000)      # an all-zero V channel
    k[1, 0, :, 3] = 0x8000                                                 # an all -0 K channel
    out, ws = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale, qk_bits=bits, smooth_v=smooth_v)
    rb = gh.Readback(ws, qk_bits=bits)
    z = oracle_lib.quant_smooth(q, k, v, _sdt(w), qk_bits=bits, smooth_v=smooth_v)
    _check_prepass(rb, z)
    if not smooth_v:
        assert (rb.v_codes == 0x80).any(), "the case holds -0 V codes"
    assert np.all(rb.v_codes[2 * 0 + 1, :, 7] == 0), "zero channel"
    O_ref, slack, _ = oracle_lib.attn_mirror(z, False, w.scale, eps=EPS_TIE)
    _compare_o(out.cpu().numpy().reshape(-1, w.D), O_ref, slack, f"signed_zeros/int{bits}/sv{int(smooth_v)}")


@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_unaligned_output_equals_aligned(out):
    """The epilogue stores four channels per instruction when the output is
    16-byte aligned and one element at a time otherwise: an output one
    element off alignment gets the same values, bit for bit."""
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    w = wl.custom(1, 2, 300, 128, causal=True, seed=141, k_offset_std=3.0)
    q, k, v = (gh.to_device(a, w.dtype) for a in wl.generate(w))
    odt, code = (torch.bfloat16, sage.BF16) if out == "bf16" else (torch.float32, sage.F32)
    n = w.B * w.H * w.N * w.D
    ws = sage.alloc_workspace(w.B, w.H, w.N, w.D).tensor
    base = torch.full((n + 8,), 7.0, dtype=odt, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    args = (w.B, w.H, w.N, w.D, w.causal, w.scale, sage.BF16, code, ws.data_ptr(), ws.numel(), sh)
    sage.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), base.data_ptr(), *args)
    aligned = base[:n].clone()
    base.fill_(7.0)
    sage.attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), base[1:].data_ptr(), *args)
    torch.cuda.synchronize()
    assert torch.equal(base[1:n + 1], aligned)
    assert base[0].item() == 7.0 and torch.all(base[n + 1:] == 7.0)   # nothing written outside
