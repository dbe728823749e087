"""GPU parity of the packed variable-length entry points against the oracle.

A packed batch is nseq independent self-attention problems in token-major
[T, H, D] tensors with sequence offsets cu_seqlens.  The oracle has no
separate varlen mode: each sequence is checked against the dense oracle run on
that sequence alone ([1, H, N_s, D]), which is what the entry point promises.
Bit-exact: codes, scales, means, FP8 V per sequence; O within the same bar as
the dense tests (max-abs 2e-3, element-wise, fp32 output).
"""
from __future__ import annotations

import numpy as np
import pytest

from fp8_attention_transformer_amd import workloads as wl

pytestmark = pytest.mark.gpu

O_TOL = 2e-3
EPS_TIE = 2.0 ** -14

CASES = [
    # (lengths, H, D, causal, qk_bits, smooth_v)
    ([17, 128, 1, 300], 2, 64, False, 4, False),
    ([129, 0, 256, 40], 2, 128, True, 4, False),
    ([200, 77, 384], 3, 128, False, 8, False),
    ([1000, 5, 130], 1, 64, True, 8, True),
    ([333, 333], 2, 128, False, 4, True),
]


def _id(c):
    lens, H, D, causal, bits, sv = c
    return f"L{'-'.join(map(str, lens))}_h{H}d{D}{'_c' if causal else ''}_int{bits}{'_sv' if sv else ''}"


def _make(lens, H, D, seed):
    """Per-sequence inputs [1, H, N_s, D] (bf16 bits) and their token-major packing."""
    seqs = []
    for s, n in enumerate(lens):
        if n == 0:
            seqs.append(None)
            continue
        w = wl.custom(1, H, n, D, seed=seed + s, k_offset_std=3.0, v_offset_std=1.5, outlier_channels=2,
                      outlier_scale=8.0)
        seqs.append((w, wl.generate(w)))
    T = sum(lens)
    packed = []
    for i in range(3):
        arr = np.zeros((T, H, D), np.uint16)
        off = 0
        for n, sq in zip(lens, seqs):
            if n:
                arr[off:off + n] = np.transpose(sq[1][i][0], (1, 0, 2))
            off += n
        packed.append(arr)
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    return seqs, packed, cu


def _to_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).cuda()


@pytest.mark.parametrize("case", CASES, ids=_id)
def test_varlen_parity(oracle_lib, case):
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    lens, H, D, causal, bits, sv = case
    seqs, packed, cu = _make(lens, H, D, seed=500 + sum(lens))
    nseq, maxlen, T = len(lens), max(lens), int(cu[-1])
    q, k, v = (_to_dev(a) for a in packed)
    cu_d = torch.from_numpy(cu).cuda()
    scale = 1.0 / np.sqrt(D)
    ws = sage.alloc_workspace(nseq, H, maxlen, D)
    ws.tensor.fill_(0xA5)
    out = sage.attn_varlen(q, k, v, cu_d, maxlen, causal=causal, sm_scale=scale, out_dtype=torch.float32,
                           workspace=ws, qk_bits=bits, smooth_v=sv)
    torch.cuda.synchronize()
    O_all = out.cpu().numpy()                                  # [T, H, D]
    # dense geometry (nseq, H, maxlen, D); blocks past a sequence are never written
    rb = gh.Readback(ws, qk_bits=bits, strict=False)
    for s, n in enumerate(lens):
        if n == 0:
            continue
        w, (qs, ks_, vs) = seqs[s]
        z = oracle_lib.quant_smooth(qs, ks_, vs, 1, qk_bits=bits, smooth_v=sv)
        nqb, G = (n + 127) // 128, 2 * ((n + 31) // 32)
        for h in range(H):
            bh = s * H + h
            assert np.array_equal(rb.q_codes_all[bh, :n], z.q_codes[0, h]), (s, h, "q codes")
            assert np.array_equal(rb.k_codes_all[bh, :n], z.k_codes[0, h]), (s, h, "k codes")
            assert np.array_equal(rb.q_scale_p[bh, :n], z.q_scale[0, h]), (s, h, "q scales")
            assert np.array_equal(rb.k_scale_p[bh, :G], z.k_scale[0, h]), (s, h, "k scales")
            assert np.array_equal(rb.q_mean[bh, :nqb], z.q_mean[0, h]), (s, h, "q means")
            assert np.array_equal(rb.k_mean[bh], z.k_mean[0, h]), (s, h, "k means")
            assert np.array_equal(rb.v_mean[bh], z.v_mean[0, h]), (s, h, "v means")
            assert np.array_equal(rb.v_scale[bh], z.v_scale[0, h]), (s, h, "v scales")
            vcodes = gh.unpermute_v(rb.v_codes_raw[bh:bh + 1], 1, rb.NQB, D, maxlen)[0]
            assert np.array_equal(vcodes[:n], z.v_codes[0, h]), (s, h, "v codes")
            # tokens past the sequence, up to its last 128-token block, are
            # padding (blocks beyond are never written nor read)
            npad = nqb * 128
            assert not vcodes[n:npad].any() and not rb.q_codes_all[bh, n:npad].any(), (s, h, "padding")
        O_ref, slack, _ = oracle_lib.attn_mirror(z, causal, scale, eps=EPS_TIE)
        O_gpu = np.transpose(O_all[cu[s]:cu[s + 1]], (1, 0, 2)).reshape(-1, D)
        gh.compare_o(O_gpu, O_ref, f"seq {s} n={n}", slack=slack)


def test_varlen_single_sequence_equals_dense(oracle_lib):
    """One packed sequence gives the dense call's output bit for bit (same kernels, same arithmetic)."""
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    w = wl.custom(1, 2, 300, 128, causal=True, seed=61, k_offset_std=3.0)
    q, k, v = wl.generate(w)
    dense, _ = gh.run_attn(q, k, v, w.dtype, w.causal, w.scale)
    packed = [np.ascontiguousarray(np.transpose(a[0], (1, 0, 2))) for a in (q, k, v)]
    cu = torch.tensor([0, 300], dtype=torch.int32, device="cuda")
    out = sage.attn_varlen(*(_to_dev(a) for a in packed), cu, 300, causal=True, sm_scale=w.scale,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    a = dense.cpu().numpy()[0]                     # [H, N, D]
    b = np.transpose(out.cpu().numpy(), (1, 0, 2))
    assert np.array_equal(a, b)


def test_varlen_split_calls_equal_fwd(oracle_lib):
    """sage_quant_smooth_varlen + sage_attn_quantized_varlen give sage_attn_fwd_varlen's output exactly."""
    import torch
    from fp8_attention_transformer_amd import sage
    lens, H, D = [300, 0, 129, 64], 2, 128
    _, packed, cu = _make(lens, H, D, seed=900)
    q, k, v = (_to_dev(a) for a in packed)
    cu_d = torch.from_numpy(cu).cuda()
    nseq, maxlen, T = len(lens), max(lens), int(cu[-1])
    ref = sage.attn_varlen(q, k, v, cu_d, maxlen, causal=True, out_dtype=torch.float32)
    ws = sage.alloc_workspace(nseq, H, maxlen, D)
    bufs = ws.bufs()
    out = torch.empty((T, H, D), dtype=torch.float32, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    sage.quant_smooth_varlen(q.data_ptr(), k.data_ptr(), v.data_ptr(), sage.BF16, cu_d.data_ptr(), nseq, maxlen, T, H,
                             D, bufs, sh)
    sage.attn_quantized_varlen(bufs, out.data_ptr(), cu_d.data_ptr(), nseq, maxlen, T, H, D, True, 1 / np.sqrt(D),
                               sage.F32, sh)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
