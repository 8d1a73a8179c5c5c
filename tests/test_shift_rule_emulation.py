"""Host check of the bf16 prefill's per-row update rule, emulated in float32.

The bf16 prefill kernel keeps, per query row, a reference shift m (log2 units), an
exp-sum l and an output accumulator, and updates them once per 128-key tile:
  * lead = scale*log2(e) * (tile's max raw score) - m;
  * the shift moves by lead when lead > 8, or when the row sees its first visible
    keys; the exp-sum and the accumulator are multiplied by the correction
    2^-(shift move), with the exponent capped at 0;
  * P = 2^(scale*log2(e)*s - m) in fp32, rounded to bf16 for the PV product; l
    adds the fp32 P's.
The rescale must be exact for any finite scores (page "AI 推理系列（十一）：Ring
Attention 如何让多张 GPU 共同计算一条超长序列", §"最容易被忽略的细节：不同 Block 的
Attention 结果不能直接相加"): softmax does not depend on the shift, only on the
shift being applied to both l and the accumulator. This file emulates the rule in
numpy float32, tile by tile, and checks it against the fp64 oracle, including rows
whose first visible tile is strongly negative. The same emulation without the cap
on the correction's exponent gives NaN there (2^+140 overflows fp32 and 0 * inf is
NaN: the row's O comes out NaN and its LSE -inf), which is the failure the cap
removes."""
import math

import numpy as np
import pytest

import oracle
from workloads import _bf16_round_np, randn_np

LAZY = np.float32(8.0)
BK = 128


def emulate_rows(q, k, v, *, scale, visible, cap=True):
    """q [R, D], k [S, D], v [S, Dv] (bf16 values as float32); visible [R, S] bool.
    Returns (o [R, Dv], lse [R]) of the kernel's rule, in float32."""
    f32 = np.float32
    sl2 = f32(scale * math.log2(math.e))
    R, S = q.shape[0], k.shape[0]
    o = np.zeros((R, v.shape[1]), f32)
    lse = np.zeros(R, f32)
    with np.errstate(over="ignore", invalid="ignore"):
        for r in range(R):
            m, l, fresh = f32(0.0), f32(0.0), True
            acc = np.zeros(v.shape[1], f32)
            for t0 in range(0, S, BK):
                s = (k[t0:t0 + BK] @ q[r]).astype(f32)          # exact-enough fp32 scores
                s = np.where(visible[r, t0:t0 + BK], s, f32(-np.inf))
                mx = f32(np.max(s))
                lead = f32(mx * sl2 - m)
                move = bool(lead > LAZY) or (fresh and mx != -np.inf)
                fresh = fresh and mx == -np.inf
                if move:
                    sh = lead
                    m = f32(m + sh)
                    ex = f32(min(-sh, 0.0)) if cap else f32(-sh)
                    alpha = f32(np.exp2(ex))
                    l = f32(l * alpha)
                    acc = (acc * alpha).astype(f32)
                p = np.exp2((s * sl2 - m).astype(f32)).astype(f32)
                l = f32(l + np.sum(p, dtype=f32))
                acc = (acc + _bf16_round_np(p) @ v[t0:t0 + BK]).astype(f32)
            # the kernel's epilogue: O = acc * (1/l), LSE = (m + log2 l) ln 2, both
            # guarded by l > 0 (false for NaN)
            inv = f32(1.0) / l if l > 0 else f32(0.0)
            o[r] = acc * inv
            lse[r] = f32((m + np.log2(l)) * math.log(2.0)) if l > 0 else -np.inf
    return o, lse


def negative_inputs(S, D, seed, mixed=False):
    """q = 4u + noise, k = -4u + noise: every scaled score near -16 sqrt(D).
    mixed: 64-key runs chosen at random keep plain N(0,1) keys."""
    u = np.sign(randn_np((D,), seed)).astype(np.float32)
    q = _bf16_round_np(randn_np((S, D), seed + 1, "bf16") + 4.0 * u)
    k0 = randn_np((S, D), seed + 2, "bf16")
    k = _bf16_round_np(k0 - 4.0 * u)
    if mixed:
        runs = np.random.default_rng(seed + 3).random((S + 63) // 64) < 0.5
        k = np.where(np.repeat(runs, 64)[:S, None], k, k0)
    v = randn_np((S, D), seed + 4, "bf16")
    return q, k, v


def check(o, lse, o_ref, l_ref):
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    assert float(np.max(np.abs(lse - l_ref))) <= 1e-2
    assert float(np.max(np.abs(o - o_ref) - (2e-2 + 2.0 ** -7 * np.abs(o_ref)))) <= 0.0


@pytest.mark.parametrize("D", [64, 128, 192])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("mixed", [False, True])
def test_rule_matches_oracle_on_negative_rows(D, causal, mixed):
    S = 300
    q, k, v = negative_inputs(S, D, seed=70 + D, mixed=mixed)
    scale = 1 / math.sqrt(D)
    rows = np.array([0, 1, 2, 127, 128, 129, 255, 256, 299])
    pos = np.arange(S)
    vis = (pos[None, :] <= rows[:, None]) if causal else np.ones((rows.size, S), bool)
    o, lse = emulate_rows(q[rows], k, v, scale=scale, visible=vis)
    o_ref, l_ref = oracle.attention_rows(q[rows], rows, k, v, scale=scale, causal=causal, k_pos0=0)
    if not mixed:
        assert float(np.max(l_ref)) < -100.0 + math.log(S)
    check(o, lse, o_ref, l_ref)


def test_uncapped_correction_gives_nan():
    """The failure the cap removes: a fresh row whose first tile's max scaled score
    is below -88.7 (log2 lead below -128) gets 2^-lead = +inf and 0 * inf = NaN in
    l and the accumulator, so O is NaN and the l > 0 guard of the epilogue turns the
    LSE into -inf, as if the row had no visible key."""
    S, D = 200, 128
    q, k, v = negative_inputs(S, D, seed=5)
    rows = np.array([0, 150])
    vis = np.arange(S)[None, :] <= rows[:, None]
    o, lse = emulate_rows(q[rows], k, v, scale=1 / math.sqrt(D), visible=vis, cap=False)
    assert np.isnan(o).all() and np.all(lse == -np.inf)
    o, lse = emulate_rows(q[rows], k, v, scale=1 / math.sqrt(D), visible=vis, cap=True)
    o_ref, l_ref = oracle.attention_rows(q[rows], rows, k, v, scale=1 / math.sqrt(D), causal=True, k_pos0=0)
    check(o, lse, o_ref, l_ref)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_rule_matches_oracle_on_sharp_and_plain_rows(seed):
    """N(0,1) rows, sharp rows (q x 8) and a growing key ramp: the shift moves up
    many times; the rule stays exact up to bf16 rounding of P."""
    S, D = 400, 128
    q = randn_np((S, D), 300 + seed, "bf16")
    k = randn_np((S, D), 310 + seed, "bf16")
    v = randn_np((S, D), 320 + seed, "bf16")
    if seed == 1:
        q = q * 8.0
    if seed == 2:
        k = _bf16_round_np(k * (1.0 + 5.0 * np.arange(S) / S)[:, None].astype(np.float32))
    rows = np.array([0, 5, 127, 128, 200, 399])
    vis = np.arange(S)[None, :] <= rows[:, None]
    o, lse = emulate_rows(q[rows], k, v, scale=1 / math.sqrt(D), visible=vis)
    o_ref, l_ref = oracle.attention_rows(q[rows], rows, k, v, scale=1 / math.sqrt(D), causal=True, k_pos0=0)
    check(o, lse, o_ref, l_ref)
