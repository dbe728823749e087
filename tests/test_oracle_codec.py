"""Pins for the oracle's FP8 (OCP e4m3fn) codec and 16-bit input decoding.

The pages quantize P~ and V to FP8 (SageAttention2 abstract, arXiv 2411.10958);
the OCP e4m3fn format is the one the gfx950 matrix cores consume.  The codec is
checked against an independent library implementation: torch.float8_e4m3fn
(round to nearest even; it returns NaN beyond the 448/480 midpoint where the
oracle saturates, so the exhaustive sweep covers |x| <= 464).
"""
from concurrent.futures import ThreadPoolExecutor

import numpy as np
import pytest
import torch


def test_decode_all_codes(oracle_lib):
    codes = np.arange(256, dtype=np.uint8)
    ours = oracle_lib.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2  # 0x7F and 0xFF
    assert np.array_equal(ours[~nan], ref[~nan])
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_encode_exhaustive_positive(oracle_lib):
    """Every fp32 bit pattern from +0 up to 464.0 (about 1.14e9 values)."""
    hi = int(np.array([464.0], np.float32).view(np.uint32)[0])
    chunk = 1 << 24

    def run(start):
        stop = min(start + chunk, hi + 1)
        x = np.arange(start, stop, dtype=np.uint32).view(np.float32)
        ours = oracle_lib.e4m3_encode(x)
        ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
        bad = np.nonzero(ours != ref)[0]
        return (start, bad[:5], x[bad[:5]]) if bad.size else None

    with ThreadPoolExecutor(8) as ex:
        fails = [r for r in ex.map(run, range(0, hi + 1, chunk)) if r is not None]
    assert not fails, fails[:3]


def test_encode_negative_sample_and_symmetry(oracle_lib):
    rng = np.random.default_rng(7)
    x = rng.uniform(0, 464, 1 << 20).astype(np.float32)
    x = np.concatenate([x, np.ldexp(rng.uniform(1, 2, 1 << 16), rng.integers(-30, -5, 1 << 16)).astype(np.float32)])
    pos = oracle_lib.e4m3_encode(x)
    neg = oracle_lib.e4m3_encode(-x)
    assert np.array_equal(neg, pos | 0x80)
    ref = torch.from_numpy(-x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(neg, ref)


def test_encode_saturates_and_nan(oracle_lib):
    x = np.array([448.0, 463.99, 464.0, 465.0, 1e6, np.inf, -1e6, np.nan], np.float32)
    out = oracle_lib.e4m3_encode(x)
    assert out.tolist() == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x7F]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_inputs_exhaustive(oracle_lib, dtype):
    bits = np.arange(1 << 16, dtype=np.uint16)
    ours = oracle_lib.decode_input(bits, 0 if dtype == "f16" else 1)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.float16 if dtype == "f16" else torch.bfloat16).float().numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert np.array_equal(np.signbit(ours), np.signbit(ref))
