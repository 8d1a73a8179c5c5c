"""Host check of the bf16 dK/dV kernel's score offset, emulated in float32.

The backward needs P = exp(scale q.k - LSE) per visible (query, key) pair (page
"长上下文的第一性挑战", §挑战 1, eq. lc-ch-attention is the function differentiated).
The dK/dV kernel starts the fp32 accumulator of each score's products from
-LSE / scale instead of 0, so that it ends at s - LSE / scale and
P = 2^(scale log2(e) (s - LSE / scale)) takes one multiply. The offset costs the
fp32 accumulation a few ulps of |s - LSE / scale| instead of |s|. This file
emulates that accumulation (16-term partial products per 16-wide step, each step
added to the fp32 accumulator with one rounding) and checks, against the exact
fp64 value, that the resulting P stays within 2^-12 relative (the bf16 rounding
of P that follows is 2^-9) for plain N(0,1) rows, sharp rows (q x 8) and large
key ramps, at D = 64, 128 and 192."""
import math

import numpy as np
import pytest

from workloads import _bf16_round_np, randn_np


def offset_probs(q, k, lse, scale):
    """P of every (row, key) pair the kernel's way: fp32 accumulation of 16-wide
    partial products starting from -lse / scale, then one fp32 multiply and exp2."""
    f32 = np.float32
    acc = np.broadcast_to((-(lse.astype(f32)) / f32(scale))[:, None], (q.shape[0], k.shape[0])).astype(f32)
    for d0 in range(0, q.shape[1], 16):
        part = (q[:, d0:d0 + 16].astype(np.float64) @ k[:, d0:d0 + 16].astype(np.float64).T).astype(f32)
        acc = (acc + part).astype(f32)
    c = f32(scale * math.log2(math.e))
    return np.exp2((acc * c).astype(f32).astype(np.float64))


@pytest.mark.parametrize("D", [64, 128, 192])
@pytest.mark.parametrize("kind", ["plain", "sharp", "ramp"])
def test_offset_scores_keep_p_within_2_pow_minus_12(D, kind):
    S = 256
    q = randn_np((S, D), 500 + D, "bf16")
    k = randn_np((S, D), 510 + D, "bf16")
    if kind == "sharp":
        q = _bf16_round_np(q * 8.0)
    if kind == "ramp":
        k = _bf16_round_np(k * (1.0 + 20.0 * np.arange(S) / S)[:, None].astype(np.float32))
    scale = 1.0 / math.sqrt(D)
    s = q.astype(np.float64) @ k.astype(np.float64).T           # exact scores
    x = scale * s
    lse = np.log(np.sum(np.exp(x - x.max(1, keepdims=True)), 1)) + x.max(1)   # full-row LSE, fp64
    exact = np.exp(x - lse[:, None])
    got = offset_probs(q, k, lse, scale)
    # the LSE goes in as fp32, as the kernel reads it
    exact32 = np.exp(x - lse.astype(np.float32).astype(np.float64)[:, None])
    assert np.allclose(exact, exact32, rtol=1e-5, atol=0)
    sig = exact > 1e-30
    rel = np.abs(got[sig] - exact32[sig]) / exact32[sig]
    assert float(rel.max()) <= 2.0 ** -12
    # rows sum to one, as P over a full row must
    assert np.allclose(got.sum(1), 1.0, rtol=2.0 ** -11)
