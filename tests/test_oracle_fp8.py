"""Pins of the oracle's FP8 (E4M3) decoding: closed-form code values from the
format's definition, and every one of the 256 codes against torch's CPU
float8_e4m3fn conversion (a library routine independent of the oracle)."""
import math

import numpy as np
import torch

import oracle


def test_e4m3_closed_forms():
    v = oracle.e4m3_to_float
    assert v(0x00) == 0.0 and v(0x80) == 0.0 and math.copysign(1.0, v(0x80)) == -1.0
    assert v(0x38) == 1.0            # exponent field 7 = bias, mantissa 0
    assert v(0x40) == 2.0 and v(0xC0) == -2.0
    assert v(0x3C) == 1.5            # mantissa 100b
    assert v(0x7E) == 448.0          # largest finite: 1.75 * 2^8
    assert v(0x08) == 2.0 ** -6      # smallest normal
    assert v(0x01) == 2.0 ** -9      # smallest subnormal: 1/8 * 2^-6
    assert v(0x07) == 7 / 8 * 2.0 ** -6
    assert np.isnan(v(0x7F)) and np.isnan(v(0xFF))
    assert oracle.dequantize(np.uint8(0x40), 0.25) == 0.5


def test_e4m3_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    ours = oracle.e4m3_to_float(codes)
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(ours)) and nan.sum() == 2
    assert np.array_equal(ref[~nan], ours[~nan])
    # every finite code is exactly a bf16 value (what the decode kernel widens to)
    assert np.array_equal(torch.from_numpy(ours[~nan]).to(torch.bfloat16).to(torch.float64).numpy(), ours[~nan])


def test_fp8_decode_definition_is_the_bf16_definition_on_dequantized_values():
    """Split-KV decode over an fp8 cache is the plain decode of scale * value; the
    partials still merge to one-shot attention."""
    rng = np.random.default_rng(7)
    B, Hq, Hkv, L, D = 1, 4, 2, 96, 16
    kc = rng.integers(0, 256, size=(B, Hkv, L, D), dtype=np.uint8)
    vc = rng.integers(0, 256, size=(B, Hkv, L, D), dtype=np.uint8)
    kc[(kc & 0x7F) == 0x7F] = 0x38     # no NaN codes in a cache
    vc[(vc & 0x7F) == 0x7F] = 0x38
    k = oracle.dequantize(kc, 0.01)
    v = oracle.dequantize(vc, 0.5)
    q = rng.standard_normal((B, Hq, D))
    op, lp, o, lse = oracle.splitkv_decode(q, k, v, n_splits=3, scale=0.25)
    o1, l1 = oracle.attention(q[:, :, None, :], k, v, scale=0.25, causal=False)
    assert np.max(np.abs(o - o1[:, :, 0])) < 1e-12 and np.max(np.abs(lse - l1[:, :, 0])) < 1e-12
