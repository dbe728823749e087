"""SageAttention2 quantized attention forward for AMD MI355X (gfx950).

The compute path is the C-ABI library ``libsage.so`` (HIP kernels for gfx950);
``fp8_attention_transformer_amd.sage`` is the thin ctypes binding over it.
"""
