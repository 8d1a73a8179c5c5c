"""GPU parity of the fp32 kernels on sharp attention: the score patterns of
tests/test_gpu_sharp_scores.py (q scaled by 8, a key ramp, strongly negative
scores, and a mix of negative and ordinary runs), in fp32.

The fp32 prefill keeps an exact running maximum per row (and per key stream, merged
at the end), so these cases exercise its rescales, its first tiles of very negative
scores, and the merge of stream states whose maxima lie far apart.

Gates, from the arithmetic of fp32 dot products (unit roundoff u = 2^-24): a score
s = scale q.k summed over D terms is off by at most
    ds = D u scale max_{r,c} sum_d |q_rd k_cd|
(the standard bound for a recursive sum), which reaches 1.4e-3 on the strongly
negative inputs at D = 128 (every |q_d k_d| near 16). The LSE is then within
1e-4 + 2 ds of the exact value (1e-4 is the fp32 tolerance of the N(0,1) cases,
covering the exp and sum roundings), and every P = exp(s - LSE) within a relative
3 ds, so each O element is within 1e-4 + 4 ds max|v|.

Backward: the bf16 analysis of the strongly negative case (dS rounded to bf16,
relative 2^-9, gives a mean dQ error of 2.4 % at D = 128, an amplification of about
12 through the cancellation dP - delta) applied to fp32's dot-product rounding
(D u ~ 7.6e-6 at D = 128) predicts about 1e-4 of the mean |dQ|; the gates are
1e-3 of the largest and of the mean |reference|."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import prefill_inputs_np, randn_np
from gpu_util import np64, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
U = 2.0 ** -24


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(torch.float32).contiguous()


def sharp_inputs_f32(B, Hq, Hkv, S, Dqk, Dv, *, seed, kind):
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, Dqk, Dv, seed=seed, dtype="f32")
    if kind == "q8":
        q = q * 8.0
    elif kind == "ramp":
        q = q * 2.0
        ramp = (1.0 + 5.0 * np.arange(S) / S).astype(np.float32)
        k = (k * ramp[None, None, :, None]).astype(np.float32)
    else:                                                       # "neg", "negmix"
        u = np.sign(randn_np((Dqk,), seed + 40)).astype(np.float32)
        q = (q + 4.0 * u).astype(np.float32)
        kn = (k - 4.0 * u).astype(np.float32)
        if kind == "neg":
            k = kn
        else:
            g = np.random.default_rng(seed + 41)
            runs = g.random((B, Hkv, (S + 63) // 64)) < 0.5
            anti = np.repeat(runs, 64, axis=2)[:, :, :S, None]
            k = np.where(anti, kn, k).astype(np.float32)
    return q.astype(np.float32), k.astype(np.float32), v.astype(np.float32)


def score_bound(q, k, scale):
    """D u scale max over (row, key) of sum_d |q_d k_d|, per the module docstring."""
    B, Hq, _, D = q.shape
    group = Hq // k.shape[1]
    worst = 0.0
    for b in range(B):
        for h in range(Hq):
            a = np.abs(q[b, h].astype(np.float64)) @ np.abs(k[b, h // group].astype(np.float64)).T
            worst = max(worst, float(a.max()))
    return D * U * scale * worst


def sharp_close_f32(o, lse, o_ref, l_ref, v, ds, what):
    fin_ref = np.isfinite(l_ref)
    assert np.array_equal(np.isfinite(lse), fin_ref), f"{what}: -inf rows differ"
    assert not np.isnan(o).any(), f"{what}: NaN in O"
    do = float(np.max(np.abs(o - o_ref)))
    dl = float(np.max(np.abs(lse[fin_ref] - l_ref[fin_ref])))
    gate_o = 1e-4 + 4 * ds * float(np.max(np.abs(v)))
    gate_l = 1e-4 + 2 * ds
    say(f"{what}: max|dO| {do:.3e} (gate {gate_o:.3e}), max|dLSE| {dl:.3e} (gate {gate_l:.3e})")
    assert do <= gate_o, what
    assert dl <= gate_l, what


@pytest.mark.parametrize("kind", ["q8", "ramp", "neg", "negmix"])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_f32_ring_sharp(ra, kind, dims, causal, layout):
    B, Hq, Hkv, Sp, P = 1, 4, 2, 300, 3
    Dqk, Dv = dims
    S = Sp * P
    say(f"ring_attn_fwd fp32 sharp {kind} D{Dqk}/{Dv} causal={causal} {layout}")
    q, k, v = sharp_inputs_f32(B, Hq, Hkv, S, Dqk, Dv, seed=2900 + Dqk, kind=kind)
    scale = 1 / math.sqrt(Dqk)
    o, lse = ra.ring_attn_fwd(to_dev(q), to_dev(k), to_dev(v), P=P, causal=causal, scale=scale, layout=layout)
    torch.cuda.synchronize()
    if layout == "contiguous":
        o_ref, l_ref = oracle.attention(q, k, v, scale=scale, causal=causal)
    else:
        pos = np.concatenate([oracle.partition_positions(P, Sp, p, "striped") for p in range(P)])
        o_ref, l_ref = oracle.attention(q, k, v, scale=scale, causal=causal, q_pos=pos, k_pos=pos)
    sharp_close_f32(np64(o), np64(lse), o_ref, l_ref, v, score_bound(q, k, scale), f"fp32 sharp {kind} {layout}")


@pytest.mark.parametrize("kind", ["neg", "negmix", "ramp"])
@pytest.mark.parametrize("dims", [(64, 64), (128, 128)])
@pytest.mark.parametrize("Sp", [160, 1040])
def test_f32_step_chain_from_empty_sharp(ra, kind, dims, Sp):
    """Every partition's ring as block steps from the empty state (O = 0, LSE = -inf),
    causal: small launches (16 x 16 products) and, at 2 x 32 heads x 1040 rows, the
    32 x 32 product shape."""
    B, Hq, Hkv, P = (1, 4, 2, 3) if Sp == 160 else (2, 32, 8, 2)
    Dqk, Dv = dims
    S = Sp * P
    say(f"block_attn_step fp32 from empty, {kind} D{Dqk}/{Dv} Sp {Sp}")
    q, k, v = sharp_inputs_f32(B, Hq, Hkv, S, Dqk, Dv, seed=3100 + Dqk + Sp, kind=kind)
    scale = 1 / math.sqrt(Dqk)
    o_ref, l_ref = oracle.attention(q, k, v, scale=scale, causal=True)
    ds = score_bound(q, k, scale)
    qd, kd, vd = to_dev(q), to_dev(k), to_dev(v)
    for i in range(P):
        qi = qd[:, :, i * Sp:(i + 1) * Sp].contiguous()
        o_acc, l_acc = ra.init_state(qi, Dv)
        for j, kind_j in ra.ring_schedule(P, i, True):
            if kind_j == "skip":
                continue
            ra.block_attn_step(qi, kd[:, :, j * Sp:(j + 1) * Sp].contiguous(),
                               vd[:, :, j * Sp:(j + 1) * Sp].contiguous(), o_acc, l_acc,
                               q_pos0=i * Sp, k_pos0=j * Sp, causal=True, scale=scale)
        torch.cuda.synchronize()
        sl = slice(i * Sp, (i + 1) * Sp)
        sharp_close_f32(np64(o_acc), np64(l_acc), o_ref[:, :, sl], l_ref[:, :, sl], v, ds,
                        f"fp32 step chain from empty, part {i}")


def grad_close(got, ref, what, rel=1e-3):
    got = np64(got)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    top = float(np.max(np.abs(ref)))
    err = np.abs(got - ref)
    say(f"{what}: max|err| {err.max():.3e} (max|ref| {top:.3e}), mean|err| {err.mean():.3e} "
        f"(mean|ref| {np.abs(ref).mean():.3e})")
    assert err.max() <= rel * top + 1e-9, what
    assert err.mean() <= rel * np.abs(ref).mean() + 1e-10, what


@pytest.mark.parametrize("dims", [(64, 64), (128, 128)])
@pytest.mark.parametrize("kind", ["q8", "ramp", "neg"])
def test_f32_backward_sharp(ra, dims, kind):
    """The fp32 forward, then the whole fp32 backward: exact gradients of the same
    fp32 inputs."""
    B, Hq, Hkv, S = 1, 4, 2, 513
    D, Dv = dims
    say(f"attn_bwd fp32 sharp {kind} D{D}/{Dv}")
    q, k, v = sharp_inputs_f32(B, Hq, Hkv, S, D, Dv, seed=2970 + D, kind=kind)
    if kind == "q8":
        q = q / 2.0                     # score spread ~4: still sharp, gradients not all zero
    do = randn_np((B, Hq, S, Dv), 2980 + D, "f32")
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    o, lse = ra.ring_attn_fwd(tq, tk, tv, P=1, causal=True)
    gq, gk, gv = ra.attn_bwd(tq, tk, tv, o, lse, to_dev(do), causal=True)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, scale=1 / math.sqrt(D), causal=True)
    grad_close(gq, rq, "dq")
    grad_close(gk, rk, "dk")
    grad_close(gv, rv, "dv")
