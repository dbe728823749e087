"""The entry point that allocates nothing (sage_attn_fwd_static) against
the workspace entry point (sage_attn_fwd), through the C ABI: the same
kernels over the same inputs, so the outputs must be identical bit for bit.
Two calls in a row, the second with a smaller input (the fixed scratch array
keeps the first call's buffers, which the second must not depend on)."""
import numpy as np
import pytest

from fp8_attention_transformer_amd import workloads as wl

pytestmark = pytest.mark.gpu

CASES = [
    wl.custom(2, 4, 3000, 128, causal=True, seed=301, k_offset_std=4.0, outlier_channels=4, outlier_scale=20.0),
    wl.custom(1, 3, 700, 64, seed=302, k_offset_std=3.0, v_offset_std=1.0),
]


def _run(w, static: bool, out_dtype, qk_bits=4, smooth_v=False):
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    q, k, v = (gh.to_device(a, w.dtype) for a in wl.generate(w))
    odt = {sage.F32: torch.float32, sage.BF16: torch.bfloat16}[out_dtype]
    o = torch.full((w.B, w.H, w.N, w.D), float("nan"), dtype=odt, device="cuda")
    sh = torch.cuda.current_stream().cuda_stream
    args = (q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), w.B, w.H, w.N, w.D, w.causal, w.scale,
            gh.in_code(w.dtype), out_dtype)
    if static:
        sage.attn_fwd_static(*args, sh, qk_bits=qk_bits, smooth_v=smooth_v)
    else:
        ws = sage.alloc_workspace(w.B, w.H, w.N, w.D)
        sage.attn_fwd(*args, ws.ptr, ws.nbytes, sh, qk_bits=qk_bits, smooth_v=smooth_v)
    torch.cuda.synchronize()
    return o.cpu()


@pytest.mark.parametrize("qk_bits,smooth_v", [(4, False), (8, True)])
def test_static_scratch_equals_workspace_call(qk_bits, smooth_v):
    import torch
    from fp8_attention_transformer_amd import sage
    for w in CASES:                       # larger call first, then a smaller one
        for od in (sage.F32, sage.BF16):
            got = _run(w, True, od, qk_bits, smooth_v)
            ref = _run(w, False, od, qk_bits, smooth_v)
            assert not torch.isnan(ref.float()).any()
            assert torch.equal(got, ref), (w.name, od, qk_bits, smooth_v)


def test_static_scratch_rejects_too_large():
    import torch
    from fp8_attention_transformer_amd import sage
    import gpu_helpers as gh
    B, H, N, D = 1, 16, 16384, 128
    assert sage.workspace_bytes(B, H, N, D) > sage.STATIC_SCRATCH_BYTES
    x = torch.zeros((B, H, N, D), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(x)
    with pytest.raises(sage.SageError) as e:
        sage.attn_fwd_static(x.data_ptr(), x.data_ptr(), x.data_ptr(), o.data_ptr(), B, H, N, D, False, 0.1,
                             sage.BF16, sage.BF16, torch.cuda.current_stream().cuda_stream)
    assert e.value.status == sage.ERR_WORKSPACE
