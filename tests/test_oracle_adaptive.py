"""Pins for the oracle's adaptive code width (qk_bits 0).

The SageAttention2 technical-report summary page (Key Contribution 3) names an
adaptive quantization method that keeps end-to-end metrics, without defining
it; the 8-bit alternative is the SageAttention (v1) page's width.  The reading
(header of oracle/sage_oracle.cpp): per key/value head, predict the variance
INT4 codes add to the softmax logits,
    sigma^2 = sm^2/12 * (mean amax_q^2 / 49 * mean |gK|^2 + mean amax_k^2 / 49 * mean |gQ|^2),
weight it by rho = E|V - vbar|^2 / (E|V - vbar|^2 + |vbar|^2), and use INT4 iff
sigma^2 * rho <= 0.02 (predicted cosine loss at most 0.01).

Checks, none of which re-runs the oracle's arithmetic:
  * the six statistics equal their definitions evaluated by brute force on
    inputs where every fp32 step is exact (integer values, dyadic means);
  * the predicted sigma^2 matches the measured variance of the logit error of
    the INT4 codes the oracle produces (the 1/12 and 1/49 and both terms);
  * the predicted cosine loss matches the measured one on a plain Gaussian
    head, and bounds it on a head with a V offset;
  * hand-built heads: a low-temperature head picks INT4, an outlier head INT8;
    invariances (V scale, permutation of whole key blocks);
  * qk_bits 0 gives each head exactly the codes of its own width;
  * the purpose: in adaptive mode every workload reaches cosine similarity
    >= 0.99 against FP32 attention (sampled heads and rows).
"""
import numpy as np
import pytest

from fp8_attention_transformer_amd import workloads as wl


def _bits(x, dtype="bf16"):
    return wl.round_to_bits(np.asarray(x, np.float32), dtype)


def _group(j):
    return 2 * (j // 32) + ((j % 32) // 4) % 2


def _paired(rng, n, d, lo, hi):
    """[n, d] integers around zero whose every 128-row block sums to zero per
    channel (rows come in +x / -x pairs inside each block)."""
    half = rng.integers(lo, hi + 1, size=(n // 2, d)).astype(np.float32)
    out = np.empty((n, d), np.float32)
    for b0 in range(0, n, 128):
        h0 = b0 // 2
        blk = half[h0:h0 + 64]
        rows = np.concatenate([blk, -blk])
        out[b0:b0 + 128] = rows[rng.permutation(128)]
    return out


def _brute_stats(Q, K, V):
    """The six statistics from their definitions (fp64), one head, self-attention."""
    N, D = Q.shape
    A_Q = E_Q = 0.0
    for b0 in range(0, N, 128):
        blk = Q[b0:b0 + 128].astype(np.float64)
        g = blk - blk.mean(0)
        A_Q += float((np.abs(g).max(1) ** 2).sum())
        E_Q += float((g ** 2).sum())
    kb = K.astype(np.float64)
    gK = kb - kb.mean(0)
    gam = np.zeros(2 * ((N + 31) // 32))
    for j in range(N):
        gam[_group(j)] = max(gam[_group(j)], np.abs(gK[j]).max())
    A_K = float(sum(gam[_group(j)] ** 2 for j in range(N)))
    E_K = float((gK ** 2).sum())
    vb = V.astype(np.float64)
    vbar = vb.mean(0)
    EV = float(((vb - vbar) ** 2).sum())
    V2 = float(N * (vbar ** 2).sum())
    return np.array([A_Q, E_Q, A_K, E_K, EV, V2])


def test_statistics_equal_definitions_on_exact_inputs(oracle_lib):
    rng = np.random.default_rng(11)
    N, D = 256, 64
    off_k = rng.integers(-6, 7, size=D).astype(np.float32)
    off_v = rng.integers(-3, 4, size=D).astype(np.float32)
    Q = _paired(rng, N, D, -5, 5) + rng.integers(-4, 5, size=D).astype(np.float32)
    K = _paired(rng, N, D, -5, 5) + off_k
    V = _paired(rng, N, D, -4, 4) + off_v
    bits, st = oracle_lib.adaptive_bits(_bits(Q)[None, None], _bits(K)[None, None], _bits(V)[None, None],
                                        oracle_lib.DT_BF16, 0.125)
    exp = _brute_stats(Q, K, V)
    assert np.array_equal(st[0, 0].astype(np.float64), exp), (st[0, 0], exp)


def _int4_logit_error_var(oracle_lib, q, k, v, sm):
    """Measured variance of the INT4 logit error over all (query, key) pairs."""
    z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16, qk_bits=4)
    Q = wl.bits_to_f32(q, "bf16").astype(np.float64)[0, 0]
    K = wl.bits_to_f32(k, "bf16").astype(np.float64)[0, 0]
    exact = sm * (Q @ K.T)
    N = Q.shape[0]
    S = z.q_codes[0, 0].astype(np.float64) @ z.k_codes[0, 0].astype(np.float64).T
    groups = np.array([_group(j) for j in range(N)])
    dq = z.q_scale[0, 0].astype(np.float64)
    dk = z.k_scale[0, 0].astype(np.float64)[groups]
    qblk = np.arange(N) // 128
    deq = sm * (S * dq[:, None] * dk[None, :] + z.delta_s[0, 0].astype(np.float64)[qblk])
    # the constant (per query) part of K's mean cancels in softmax: compare row-centred errors
    err = deq - exact
    err -= err.mean(1, keepdims=True)
    return float(err.var())


@pytest.mark.parametrize("kind", ["gauss", "outlier_q", "heavy"])
def test_predicted_sigma_matches_measured_logit_noise(oracle_lib, kind):
    rng = np.random.default_rng({"gauss": 21, "outlier_q": 22, "heavy": 23}[kind])
    N, D, sm = 512, 64, 0.125
    Q = rng.standard_normal((N, D)).astype(np.float32)
    K = rng.standard_normal((N, D)).astype(np.float32) + 3.0 * rng.standard_normal(D).astype(np.float32)
    V = rng.standard_normal((N, D)).astype(np.float32)
    if kind == "outlier_q":
        Q[:, :3] *= 12.0
    if kind == "heavy":
        Q += 0.5 * rng.standard_t(3, (N, D)).astype(np.float32)
        K += 0.5 * rng.standard_t(3, (N, D)).astype(np.float32)
    q, k, v = (_bits(a)[None, None] for a in (Q, K, V))
    _, st = oracle_lib.adaptive_bits(q, k, v, oracle_lib.DT_BF16, sm)
    A_Q, E_Q, A_K, E_K = (float(x) for x in st[0, 0, :4])
    pred = sm * sm / 12.0 * (A_Q / 49.0 * E_K + A_K / 49.0 * E_Q) / (N * N)
    meas = _int4_logit_error_var(oracle_lib, q, k, v, sm)
    # the uniform-rounding model is an estimate: within 35% on these heads
    assert 0.65 * meas <= pred <= 1.35 * meas, (kind, pred, meas)


def test_predicted_cosine_loss(oracle_lib):
    """Gaussian head (no V offset): the predicted INT4 cosine loss sigma^2/2 *
    rho matches the loss the oracle measures against FP32 attention; with a V
    offset the prediction (attention on one key) is an upper bound."""
    w = wl.TINY
    q, k, v = wl.generate(w)
    qh, kh, vh = q[:, :1], k[:, :1], v[:, :1]
    _, st = oracle_lib.adaptive_bits(qh, kh, vh, oracle_lib.DT_F16, w.scale)
    A_Q, E_Q, A_K, E_K, EV, V2 = (float(x) for x in st[0, 0])
    N = w.N
    s2 = w.scale ** 2 / 12.0 * (A_Q / 49.0 * E_K + A_K / 49.0 * E_Q) / (N * N)
    pred_loss = s2 / 2 * EV / (EV + V2)
    z = oracle_lib.quant_smooth(qh, kh, vh, oracle_lib.DT_F16, qk_bits=4)
    O, _, _ = oracle_lib.attn_mirror(z, False, w.scale)
    Oe, _ = oracle_lib.attn_exact(qh, kh, vh, oracle_lib.DT_F16, False, w.scale, 0)
    a, b = O.astype(np.float64).ravel(), Oe.ravel()
    loss = 1.0 - a @ b / np.linalg.norm(a) / np.linalg.norm(b)
    assert 0.7 * loss <= pred_loss <= 1.3 * loss, (pred_loss, loss)
    # V with a large per-channel offset: measured loss far below the bound
    rng = np.random.default_rng(5)
    V = wl.bits_to_f32(vh, "f16")[0, 0] + 2.0 * rng.standard_normal(w.D).astype(np.float32)
    v2 = wl.round_to_bits(V, "f16")[None, None]
    _, st2 = oracle_lib.adaptive_bits(qh, kh, v2, oracle_lib.DT_F16, w.scale)
    EV2, V22 = float(st2[0, 0, 4]), float(st2[0, 0, 5])
    z2 = oracle_lib.quant_smooth(qh, kh, v2, oracle_lib.DT_F16, qk_bits=4)
    O2, _, _ = oracle_lib.attn_mirror(z2, False, w.scale)
    Oe2, _ = oracle_lib.attn_exact(qh, kh, v2, oracle_lib.DT_F16, False, w.scale, 0)
    a, b = O2.astype(np.float64).ravel(), Oe2.ravel()
    loss2 = 1.0 - a @ b / np.linalg.norm(a) / np.linalg.norm(b)
    assert loss2 <= s2 / 2 * EV2 / (EV2 + V22)


def test_hand_built_heads_pick_each_width(oracle_lib):
    """Head 0: low temperature (small Q), INT4 is accurate enough; head 1: the
    same keys with four query channels scaled x20, INT8."""
    rng = np.random.default_rng(31)
    N, D = 256, 128
    Q = rng.standard_normal((2, N, D)).astype(np.float32)
    K = rng.standard_normal((2, N, D)).astype(np.float32) + 4.0 * rng.standard_normal(D).astype(np.float32)
    V = rng.standard_normal((2, N, D)).astype(np.float32)
    Q[0] *= 0.25
    Q[1, :, :4] *= 20.0
    q, k, v = (_bits(a)[None] for a in (Q, K, V))
    bits, _ = oracle_lib.adaptive_bits(q, k, v, oracle_lib.DT_BF16, 1.0 / np.sqrt(D))
    assert bits.tolist() == [[4, 8]]
    # the choice is scale-free in V, and invariant to swapping whole 128-key blocks
    b2, _ = oracle_lib.adaptive_bits(q, k, _bits(4.0 * V)[None], oracle_lib.DT_BF16, 1.0 / np.sqrt(D))
    assert b2.tolist() == [[4, 8]]
    perm = np.concatenate([np.arange(128, 256), np.arange(0, 128)])
    b3, st3 = oracle_lib.adaptive_bits(q, k[:, :, perm], v[:, :, perm], oracle_lib.DT_BF16, 1.0 / np.sqrt(D))
    assert b3.tolist() == [[4, 8]]
    # a larger softmax scale moves head 0 across the threshold
    b4, _ = oracle_lib.adaptive_bits(q, k, v, oracle_lib.DT_BF16, 8.0 / np.sqrt(D))
    assert b4.tolist() == [[8, 8]]


def test_mixed_widths_give_each_head_its_own_codes(oracle_lib):
    rng = np.random.default_rng(41)
    B, H, N, D = 1, 3, 200, 64
    Q = rng.standard_normal((B, H, N, D)).astype(np.float32)
    K = rng.standard_normal((B, H, N, D)).astype(np.float32)
    V = rng.standard_normal((B, H, N, D)).astype(np.float32)
    q, k, v = (_bits(a) for a in (Q, K, V))
    hb = np.array([[4, 8, 4]], np.int32)
    z = oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16, qk_bits=0, head_bits=hb)
    for h, bits in enumerate(hb[0]):
        zh = oracle_lib.quant_smooth(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], oracle_lib.DT_BF16,
                                     qk_bits=int(bits))
        for name in ("q_codes", "q_scale", "k_codes", "k_scale", "v_codes", "delta_s"):
            assert np.array_equal(getattr(z, name)[:, h], getattr(zh, name)[:, 0]), (h, name)
    with pytest.raises(ValueError):
        oracle_lib.quant_smooth(q, k, v, oracle_lib.DT_BF16, qk_bits=0, head_bits=np.array([[4, 6, 4]]))


def test_grouped_heads_share_one_choice(oracle_lib):
    """Grouped-query heads: one width per key/value head; its statistics pool
    the query heads of the group (equal to one query head of twice the length
    built from the two, when the blocks line up)."""
    rng = np.random.default_rng(51)
    N, D = 256, 64
    Q = rng.standard_normal((1, 2, N, D)).astype(np.float32)
    K = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    V = rng.standard_normal((1, 1, N, D)).astype(np.float32)
    q, k, v = (_bits(a) for a in (Q, K, V))
    bits, st = oracle_lib.adaptive_bits(q, k, v, oracle_lib.DT_BF16, 0.125)
    assert bits.shape == (1, 1)
    _, s0 = oracle_lib.adaptive_bits(q[:, :1], k, v, oracle_lib.DT_BF16, 0.125)
    _, s1 = oracle_lib.adaptive_bits(q[:, 1:], k, v, oracle_lib.DT_BF16, 0.125)
    assert st[0, 0, 0] == np.float32(s0[0, 0, 0] + s1[0, 0, 0])
    assert st[0, 0, 1] == np.float32(s0[0, 0, 1] + s1[0, 0, 1])
    assert np.array_equal(st[0, 0, 2:], s0[0, 0, 2:])


# The purpose of the rule: cosine similarity >= 0.99 against FP32 attention
# in adaptive mode.  Two heads and 96 rows per workload (the full-size GPU
# tests check every head of the GPU path against this oracle).
ACC_CASES = [wl.TINY, wl.LLM, wl.DIT, wl.VIDEO, wl.long_context(8192, True)]


@pytest.mark.parametrize("w", ACC_CASES, ids=lambda w: w.name)
def test_adaptive_mode_reaches_cos_sim_099(oracle_lib, w):
    rng = np.random.default_rng(7)
    nh = w.B * w.H
    heads = sorted({0, nh - 1})
    dt = oracle_lib.DT_F16 if w.dtype == wl.F16 else oracle_lib.DT_BF16
    got, ref = [], []
    for hh in heads:
        q, k, v = wl.generate(w, heads=slice(hh, hh + 1))
        z = oracle_lib.quant_smooth(q, k, v, dt, qk_bits=0, sm_scale=w.scale)
        rows = np.sort(rng.choice(w.N, min(w.N, 96), replace=False))
        O, _, _ = oracle_lib.attn_mirror(z, w.causal, w.scale, rows=rows)
        Oe, _ = oracle_lib.attn_exact(q, k, v, dt, w.causal, w.scale, 0, rows=rows)
        got.append(O.astype(np.float64))
        ref.append(Oe)
    a, b = np.concatenate(got).ravel(), np.concatenate(ref).ravel()
    cos = a @ b / np.linalg.norm(a) / np.linalg.norm(b)
    assert cos >= 0.99, (w.name, cos)
