"""GPU parity of the fp32 backward (fp32 inputs, fp32 arithmetic throughout) against
the oracle's exact gradients: the per-pair step given the oracle's row LSE and
delta, the delta preprocess, the whole-sequence backward after the fp32 GPU
forward, the ring protocol and the striped layout, and the degenerate pairs.

Gate: per gradient tensor, max |g - g_ref| <= 1e-4 * max |g_ref| and the mean
absolute error <= 1e-5 * mean |g_ref|. The kernels round nothing below fp32
(unit roundoff u = 2^-24 ~ 6e-8); the longest sums here run over about a thousand
terms (n u ~ 6e-5 in the worst case, sqrt(n) u ~ 2e-6 typically), and P's exponent
carries the fp32 rounding of the score and of the LSE. A product rounded to bf16
(2^-9 ~ 2e-3 relative) fails the gate by an order of magnitude."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import prefill_inputs_np, randn_np
from gpu_util import np64, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
F32 = torch.float32


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def to_dev(x):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(F32).contiguous()


def grad_close(got, ref, what, rmax=1e-4, rmean=1e-5, atol=1e-9):
    got = np64(got)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = float(np.max(np.abs(ref)))
    err = np.abs(got - ref)
    say(f"{what}: max|err| {err.max():.3e} (max|ref| {scale:.3e}), mean|err| {err.mean():.3e} "
        f"(mean|ref| {np.abs(ref).mean():.3e})")
    assert err.max() <= rmax * scale + atol, what
    assert err.mean() <= rmean * np.abs(ref).mean() + atol, what


DIMS = [(64, 64), (128, 128), (64, 128), (128, 64)]


def zeros(*shape):
    return torch.zeros(shape, dtype=F32, device=DEV)


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("causal,q_pos0,k_pos0", [(False, 0, 0), (True, 0, 0), (True, 300, 0), (True, 100, 180)])
@pytest.mark.parametrize("Sq,Sk", [(300, 257), (40, 530)])
def test_f32_bwd_step_against_oracle(ra, dims, causal, q_pos0, k_pos0, Sq, Sk):
    """Ragged on every tile size: 300 = 18 x 16 + 12 query rows, 257 = 4 x 64 + 1 and
    8 x 32 + 1 keys; batch 2, GQA 2:1."""
    B, Hq, Hkv = 2, 4, 2
    D, Dv = dims
    say(f"block_attn_bwd_step f32 D{D}/{Dv} causal={causal} q_pos0={q_pos0} k_pos0={k_pos0} Sq{Sq} Sk{Sk}")
    q, k, v = prefill_inputs_np(B, Hq, Hkv, Sq, Sk, D, Dv, seed=1500 + Sq + Sk + D + Dv, dtype="f32")
    do = randn_np((B, Hq, Sq, Dv), 1600 + D + Dv, "f32")
    scale = 1 / math.sqrt(D)
    # full-row statistics: the block is part of a longer key range
    kf, vf = (np.concatenate([x, x[:, :, :7]], axis=2) for x in (k, v))
    kpos = np.concatenate([k_pos0 + np.arange(Sk), k_pos0 + Sk + np.arange(7)])
    _, _, _, lse, delta = oracle.attention_bwd(q, kf, vf, do, scale=scale, causal=causal, q_pos0=q_pos0,
                                               k_pos=kpos)
    gq, gk, gv = oracle.block_bwd(q, k, v, do, lse, delta, scale=scale, causal=causal, q_pos0=q_pos0,
                                  k_pos0=k_pos0)
    dq, dk, dv = zeros(B, Hq, Sq, D), zeros(B, Hkv, Sk, D), zeros(B, Hkv, Sk, Dv)
    lse_d = to_dev(np.where(np.isfinite(lse), lse, -np.inf))
    ra.block_attn_bwd_step(to_dev(q), to_dev(do), lse_d, to_dev(delta), to_dev(k), to_dev(v), dq, dk, dv,
                           q_pos0=q_pos0, k_pos0=k_pos0, causal=causal, scale=scale)
    torch.cuda.synchronize()
    grad_close(dq, gq, "dq")
    grad_close(dk, gk, "dk")
    grad_close(dv, gv, "dv")


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("causal,q_pos0,k_pos0", [(False, 0, 0), (True, 900, 0), (True, 100, 180)])
def test_f32_bwd_step_wide_dq(ra, dims, causal, q_pos0, k_pos0):
    """A launch of at least 256 64-row dQ workgroups takes them (4 row blocks x 2 key
    streams; the cases above have fewer and take 32-row ones): 2 x 8 heads x 1040
    rows (17 tiles, the last ragged), 300 keys."""
    B, Hq, Hkv, Sq, Sk = 2, 8, 2, 1040, 300
    D, Dv = dims
    assert B * Hq * ((Sq + 63) // 64) >= 256
    say(f"block_attn_bwd_step f32 wide dQ D{D}/{Dv} causal={causal} q_pos0={q_pos0} k_pos0={k_pos0}")
    q, k, v = prefill_inputs_np(B, Hq, Hkv, Sq, Sk, D, Dv, seed=1540 + D + Dv + q_pos0, dtype="f32")
    do = randn_np((B, Hq, Sq, Dv), 1640 + D + Dv, "f32")
    scale = 1 / math.sqrt(D)
    kf, vf = (np.concatenate([x, x[:, :, :7]], axis=2) for x in (k, v))
    kpos = np.concatenate([k_pos0 + np.arange(Sk), k_pos0 + Sk + np.arange(7)])
    _, _, _, lse, delta = oracle.attention_bwd(q, kf, vf, do, scale=scale, causal=causal, q_pos0=q_pos0,
                                               k_pos=kpos)
    gq, gk, gv = oracle.block_bwd(q, k, v, do, lse, delta, scale=scale, causal=causal, q_pos0=q_pos0,
                                  k_pos0=k_pos0)
    dq, dk, dv = zeros(B, Hq, Sq, D), zeros(B, Hkv, Sk, D), zeros(B, Hkv, Sk, Dv)
    ra.block_attn_bwd_step(to_dev(q), to_dev(do), to_dev(np.where(np.isfinite(lse), lse, -np.inf)),
                           to_dev(delta), to_dev(k), to_dev(v), dq, dk, dv, q_pos0=q_pos0, k_pos0=k_pos0,
                           causal=causal, scale=scale)
    torch.cuda.synchronize()
    grad_close(dq, gq, "dq")
    grad_close(dk, gk, "dk")
    grad_close(dv, gv, "dv")


def test_f32_bwd_step_accumulates(ra):
    """The step adds into the accumulators: two calls give twice one call."""
    B, Hq, Hkv, S, D = 1, 2, 1, 200, 128
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=1077, dtype="f32")
    do = randn_np((B, Hq, S, D), 1078, "f32")
    _, _, _, lse, delta = oracle.attention_bwd(q, k, v, do, scale=0.1, causal=True)
    args = [to_dev(q), to_dev(do), to_dev(lse), to_dev(delta), to_dev(k), to_dev(v)]
    outs = [[zeros(*s) for s in ((B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D))] for _ in range(2)]
    ra.block_attn_bwd_step(*args, *outs[0], q_pos0=0, k_pos0=0, causal=True, scale=0.1)
    for _ in range(2):
        ra.block_attn_bwd_step(*args, *outs[1], q_pos0=0, k_pos0=0, causal=True, scale=0.1)
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.allclose(2 * a, b, rtol=1e-6, atol=1e-6)


@pytest.mark.parametrize("Dv", [64, 128, 8])
def test_f32_bwd_preprocess(ra, Dv):
    """delta = rowsum(dO o O) in fp32: 1001 rows (a ragged last workgroup of 16)."""
    rows = 1001
    o = randn_np((rows, Dv), 1090 + Dv, "f32")
    do = randn_np((rows, Dv), 1091 + Dv, "f32")
    delta = ra.attn_bwd_preprocess(to_dev(o), to_dev(do))
    torch.cuda.synchronize()
    ref = (o.astype(np.float64) * do.astype(np.float64)).sum(1)
    err = np.max(np.abs(np64(delta) - ref))
    say(f"delta f32 Dv{Dv}: max|err| {err:.3e}")
    assert err <= 2e-6 * (1 + np.abs(ref).max())


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_f32_whole_backward_after_gpu_forward(ra, dims, causal):
    """ring_attn_fwd in fp32 on the GPU, then attn_bwd: the exact gradients of the
    same fp32 inputs, GQA 4:1, ragged length."""
    B, Hq, Hkv, S = 1, 8, 2, 555
    D, Dv = dims
    say(f"attn_bwd f32 whole D{D}/{Dv} causal={causal}")
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, Dv, seed=1700 + D + Dv, dtype="f32")
    do = randn_np((B, Hq, S, Dv), 1710 + D + Dv, "f32")
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    o, lse = ra.ring_attn_fwd(tq, tk, tv, P=1, causal=causal)
    gq, gk, gv = ra.attn_bwd(tq, tk, tv, o, lse, to_dev(do), causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, scale=1 / math.sqrt(D), causal=causal)
    grad_close(gq, rq, "dq")
    grad_close(gk, rk, "dk")
    grad_close(gv, rv, "dv")


def test_f32_whole_backward_group3_batch2(ra):
    """A group of three query heads per KV head and two sequences."""
    B, Hq, Hkv, S, D = 2, 6, 2, 301, 64
    say("attn_bwd f32 whole, group 3, batch 2")
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=1720, dtype="f32")
    do = randn_np((B, Hq, S, D), 1730, "f32")
    tq, tk, tv = to_dev(q), to_dev(k), to_dev(v)
    o, lse = ra.ring_attn_fwd(tq, tk, tv, P=1, causal=True)
    gq, gk, gv = ra.attn_bwd(tq, tk, tv, o, lse, to_dev(do), causal=True)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, scale=1 / math.sqrt(D), causal=True)
    grad_close(gq, rq, "dq")
    grad_close(gk, rk, "dk")
    grad_close(gv, rv, "dv")


@pytest.mark.parametrize("causal", [False, True])
def test_f32_ring_backward_protocol(ra, causal):
    """Every (query partition i, ring step s) pair in ring order, accumulating into
    dq_i and the travelling dk_j / dv_j: the sums are the exact gradients."""
    B, Hq, Hkv, Sp, P, D = 1, 4, 2, 150, 4, 128
    S = Sp * P
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=1801, dtype="f32")
    do = randn_np((B, Hq, S, D), 1802, "f32")
    tq, tk, tv, tdo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = ra.ring_attn_fwd(tq, tk, tv, P=P, causal=causal)
    delta = ra.attn_bwd_preprocess(o, tdo)
    part = lambda t, i: t[:, :, i * Sp:(i + 1) * Sp].contiguous()
    dqs = [zeros(B, Hq, Sp, D) for _ in range(P)]
    dks = [zeros(B, Hkv, Sp, D) for _ in range(P)]
    dvs = [zeros(B, Hkv, Sp, D) for _ in range(P)]
    for i in range(P):
        for j, kind in ra.ring_schedule(P, i, causal):
            if kind == "skip":
                continue
            ra.block_attn_bwd_step(part(tq, i), part(tdo, i), part(lse, i), part(delta, i), part(tk, j),
                                   part(tv, j), dqs[i], dks[j], dvs[j], q_pos0=i * Sp, k_pos0=j * Sp,
                                   causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, scale=1 / math.sqrt(D), causal=causal)
    grad_close(torch.cat(dqs, 2), rq, "ring dq")
    grad_close(torch.cat(dks, 2), rk, "ring dk")
    grad_close(torch.cat(dvs, 2), rv, "ring dv")


def test_f32_striped_ring_backward(ra):
    """Striped layout with its virtual positions (query: local row, key: local index
    + [j > i]), back in natural order: the exact gradients."""
    B, Hq, Hkv, Sp, P, D = 1, 4, 2, 100, 4, 64
    S = Sp * P
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=1901, dtype="f32")
    do = randn_np((B, Hq, S, D), 1902, "f32")
    st = lambda x: np.concatenate([x[:, :, p::P] for p in range(P)], axis=2)
    tq, tk, tv, tdo = (to_dev(st(x)) for x in (q, k, v, do))
    o, lse = ra.ring_attn_fwd(tq, tk, tv, P=P, causal=True, layout="striped")
    delta = ra.attn_bwd_preprocess(o, tdo)
    part = lambda t, i: t[:, :, i * Sp:(i + 1) * Sp].contiguous()
    dqs = [zeros(B, Hq, Sp, D) for _ in range(P)]
    dks = [zeros(B, Hkv, Sp, D) for _ in range(P)]
    dvs = [zeros(B, Hkv, Sp, D) for _ in range(P)]
    for i in range(P):
        for j, _ in ra.ring_schedule(P, i, True, "striped"):
            ra.block_attn_bwd_step(part(tq, i), part(tdo, i), part(lse, i), part(delta, i), part(tk, j),
                                   part(tv, j), dqs[i], dks[j], dvs[j], q_pos0=0, k_pos0=1 if j > i else 0,
                                   causal=True)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, scale=1 / math.sqrt(D), causal=True)
    grad_close(torch.cat(dqs, 2), st(rq), "striped dq")
    grad_close(torch.cat(dks, 2), st(rk), "striped dk")
    grad_close(torch.cat(dvs, 2), st(rv), "striped dv")


def test_f32_masked_pair_and_empty_rows(ra):
    """A causal pair whose keys all follow its queries adds exactly nothing; rows with
    LSE = -inf (no visible key anywhere) add nothing to any gradient."""
    B, Hq, Hkv, Sq, Sk, D = 1, 2, 1, 50, 70, 64
    q, k, v = prefill_inputs_np(B, Hq, Hkv, Sq, Sk, D, D, seed=1950, dtype="f32")
    do = randn_np((B, Hq, Sq, D), 1951, "f32")
    lse = to_dev(np.full((B, Hq, Sq), 3.0))
    delta = to_dev(np.ones((B, Hq, Sq)))
    dq, dk, dv = zeros(B, Hq, Sq, D), zeros(B, Hkv, Sk, D), zeros(B, Hkv, Sk, D)
    ra.block_attn_bwd_step(to_dev(q), to_dev(do), lse, delta, to_dev(k), to_dev(v), dq, dk, dv,
                           q_pos0=0, k_pos0=Sq, causal=True)
    lse_inf = torch.full((B, Hq, Sq), -math.inf, dtype=F32, device=DEV)
    ra.block_attn_bwd_step(to_dev(q), to_dev(do), lse_inf, delta, to_dev(k), to_dev(v), dq, dk, dv,
                           q_pos0=0, k_pos0=0, causal=False)
    torch.cuda.synchronize()
    for t, name in ((dq, "dq"), (dk, "dk"), (dv, "dv")):
        assert int(torch.count_nonzero(t)) == 0, name


@pytest.mark.parametrize("Sq,Sk", [(1, 1), (1, 33), (17, 1)])
def test_f32_tiny_pairs(ra, Sq, Sk):
    """Single rows and single keys, non-causal and causal with the key first. With one
    visible key P = 1 and dS = dO.v - delta = 0 exactly, so dQ and dK are zero up to
    the fp32 rounding of dO.v against the oracle's delta (atol 1e-5)."""
    B, Hq, Hkv, D = 1, 2, 2, 128
    for causal in (False, True):
        q, k, v = prefill_inputs_np(B, Hq, Hkv, Sq, Sk, D, D, seed=1960 + Sq + Sk, dtype="f32")
        do = randn_np((B, Hq, Sq, D), 1961, "f32")
        _, _, _, lse, delta = oracle.attention_bwd(q, k, v, do, scale=0.09, causal=causal, q_pos0=Sk - 1)
        gq, gk, gv = oracle.block_bwd(q, k, v, do, lse, delta, scale=0.09, causal=causal, q_pos0=Sk - 1)
        dq, dk, dv = zeros(B, Hq, Sq, D), zeros(B, Hkv, Sk, D), zeros(B, Hkv, Sk, D)
        ra.block_attn_bwd_step(to_dev(q), to_dev(do), to_dev(lse), to_dev(delta), to_dev(k), to_dev(v),
                               dq, dk, dv, q_pos0=Sk - 1, k_pos0=0, causal=causal, scale=0.09)
        torch.cuda.synchronize()
        grad_close(dq, gq, f"dq causal={causal}", atol=1e-5)
        grad_close(dk, gk, f"dk causal={causal}", atol=1e-5)
        grad_close(dv, gv, f"dv causal={causal}", atol=1e-5)
