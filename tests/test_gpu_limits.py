"""GPU parity at the largest sizes the boundary accepts: a per-(batch, head) slab of
just under 2^31 bytes, the limit of the kernels' 32-bit buffer offsets.

At 8,388,607 keys of d = 128 in bf16 (2^31 - 256 bytes per K or V slab), and at
16,777,208 keys of an fp8 cache, the oracle cannot run, so the expected values
come from closed forms: with Q = 0 every visible key has the same score, P is
uniform and
    O = mean of the visible V rows,  LSE = ln(number of visible keys)
(the definition of softmax attention; page "长上下文的第一性挑战", §挑战 1). V is a
staircase over the key index, V[c, d] = (c >> 20) + t[d] (c >> 21 for the fp8
cache), so every block of 2^20 (2^21) keys has its own value: a key read from the
wrong place (an offset that wrapped, a tile that was skipped or read twice) moves
the mean. These small integers are exact in bf16 and in e4m3, and the products'
fp32 partial sums of 16 equal values stay exact.

Gates: the fp32 outputs (step state, decode partials) 2e-3 and the bf16 output
2e-2 (absolute, |O| <= 10), LSE 1e-4 (its only error is the log of an exactly
summed count)."""
import math

import numpy as np
import pytest
import torch

from gpu_util import say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
D = 128
MAX_ROWS = (2**31 - 1) // (D * 2)     # 8,388,607 rows of 256 bytes: the largest accepted bf16 slab
MAX_ROWS8 = (2**31 - 1) // D          # 16,777,215 rows of 128 one-byte values: the largest fp8 slab


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def staircase(n, t, shift=20):
    """[n, D] bf16 on the device: row c holds (c >> shift) + t[d]."""
    hi = (torch.arange(n, device=DEV) >> shift).to(torch.bfloat16)
    return (hi[:, None] + torch.as_tensor(t, dtype=torch.bfloat16, device=DEV)[None, :]).contiguous()


def staircase_sum(a, b, shift=20):
    """sum over c in [a, b) of (c >> shift), exactly."""
    total = 0
    for k in range(a >> shift, ((b - 1) >> shift) + 1):
        lo, hi = max(a, k << shift), min(b, (k + 1) << shift)
        total += k * max(0, hi - lo)
    return total


T = (np.arange(D) % 7 - 3).astype(np.float64)     # per-column offsets -3 .. 3


def test_step_over_the_largest_slab(ra):
    """One block step from the empty state: 16 query heads (GQA 16:1) of 64 rows,
    all 8,388,607 keys visible."""
    B, Hq, Hkv, Sq, Sk = 1, 16, 1, 64, MAX_ROWS
    say(f"block_attn_step over the largest slab: Sk {Sk}, {Sk * D * 2} bytes per K / V slab")
    q = torch.zeros((B, Hq, Sq, D), dtype=torch.bfloat16, device=DEV)
    k = torch.zeros((B, Hkv, Sk, D), dtype=torch.bfloat16, device=DEV)
    v = staircase(Sk, T).reshape(B, Hkv, Sk, D)
    o_acc, lse_acc = ra.init_state(q, D)
    ra.block_attn_step(q, k, v, o_acc, lse_acc, q_pos0=Sk, k_pos0=0, causal=True)
    torch.cuda.synchronize()
    mean = staircase_sum(0, Sk) / Sk + T
    o = o_acc.double().cpu().numpy()
    lse = lse_acc.double().cpu().numpy()
    err_o = float(np.abs(o - mean[None, None, None, :]).max())
    err_l = float(np.abs(lse - math.log(Sk)).max())
    say(f"max|dO| {err_o:.3e}, max|dLSE| {err_l:.3e}")
    assert err_o <= 2e-3 and err_l <= 1e-4
    del q, k, v, o_acc, lse_acc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("kv8", [False, True])
def test_decode_over_the_largest_cache(ra, kv8):
    """Split-KV decode of one token over the largest cache in 8 splits (8,388,600
    keys in bf16, 16,777,208 in fp8; each split straddles a step of the staircase):
    every partial and the merge."""
    B, Hq, Hkv, n = 1, 8, 1, 8
    L = (MAX_ROWS8 if kv8 else MAX_ROWS) // n * n
    sh = 21 if kv8 else 20
    say(f"splitkv_decode{'_fp8' if kv8 else ''} over L {L} in {n} splits")
    q = torch.zeros((B, Hq, D), dtype=torch.bfloat16, device=DEV)
    v = staircase(L, T, sh).reshape(B, Hkv, L, D)
    if kv8:
        k8 = torch.zeros((B, Hkv, L, D), dtype=torch.float8_e4m3fn, device=DEV)
        v8 = v.to(torch.float8_e4m3fn)          # integers -3 .. 10: exact in e4m3
        del v
        op, lp, o, lse = ra.splitkv_decode_fp8(q, k8, v8, k_scale=1.0, v_scale=1.0, n_splits=n)
        del k8, v8
    else:
        k = torch.zeros((B, Hkv, L, D), dtype=torch.bfloat16, device=DEV)
        op, lp, o, lse = ra.splitkv_decode(q, k, v, n_splits=n)
        del k, v
    torch.cuda.synchronize()
    c = L // n
    for p in range(n):
        mean_p = staircase_sum(p * c, (p + 1) * c, sh) / c + T
        err = float(np.abs(op[0, :, p].double().cpu().numpy() - mean_p[None, :]).max())
        err_l = float(np.abs(lp[0, :, p].double().cpu().numpy() - math.log(c)).max())
        assert err <= 2e-3 and err_l <= 1e-4, (p, err, err_l)
    mean = staircase_sum(0, L, sh) / L + T
    err_o = float(np.abs(o.double().cpu().numpy() - mean[None, None, :]).max())
    err_l = float(np.abs(lse.double().cpu().numpy() - math.log(L)).max())
    say(f"merged: max|dO| {err_o:.3e}, max|dLSE| {err_l:.3e}")
    assert err_o <= 2e-2 and err_l <= 1e-4
    del q, op, lp, o, lse
    torch.cuda.empty_cache()
