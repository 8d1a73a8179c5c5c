"""GPU parity of the backward entry points against the oracle's exact gradients:
the per-pair step (given the oracle's row LSE and delta), the delta preprocess, the
whole-sequence backward after the GPU forward, and the ring protocol (every query
partition against every KV block, accumulated) against the whole-sequence result.

Gate (bf16 inputs, fp32 accumulation): per gradient tensor, max |g - g_ref| <=
2e-2 * max |g_ref|, and the mean absolute error <= 5e-3 * mean |g_ref|. The kernel
rounds P and dS to bf16 for the products (relative 2^-9 each) and the whole
backward reads the forward's bf16 output for delta."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import prefill_inputs_np, randn_np
from gpu_util import np64, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def to_dev(x, dtype=torch.bfloat16):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype).contiguous()


def grad_close(got, ref, what, rmax=2e-2, rmean=5e-3):
    got = np64(got)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    scale = float(np.max(np.abs(ref)))
    err = np.abs(got - ref)
    say(f"{what}: max|err| {err.max():.3e} (max|ref| {scale:.3e}), mean|err| {err.mean():.3e} "
        f"(mean|ref| {np.abs(ref).mean():.3e})")
    assert err.max() <= rmax * scale + 1e-6, what
    assert err.mean() <= rmean * np.abs(ref).mean() + 1e-7, what
    return float(err.max())


DIMS = [(64, 64), (128, 128), (192, 128)]


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("causal,q_pos0,k_pos0", [(False, 0, 0), (True, 0, 0), (True, 300, 0), (True, 100, 180)])
@pytest.mark.parametrize("Sq,Sk", [(300, 257), (64, 520)])
def test_bwd_step_against_oracle(ra, dims, causal, q_pos0, k_pos0, Sq, Sk):
    B, Hq, Hkv = 2, 4, 2
    D, Dv = dims
    say(f"block_attn_bwd_step D{D}/{Dv} causal={causal} q_pos0={q_pos0} k_pos0={k_pos0} Sq{Sq} Sk{Sk}")
    q, k, v = prefill_inputs_np(B, Hq, Hkv, Sq, Sk, D, Dv, seed=500 + Sq + Sk + D, dtype="bf16")
    do = randn_np((B, Hq, Sq, Dv), 600 + D, "bf16")
    scale = 1 / math.sqrt(D)
    # full-row statistics: the block is part of a longer key range starting at 0
    kf, vf = (np.concatenate([x, x[:, :, :7]], axis=2) for x in (k, v))   # 7 more keys after the block
    kpos = np.concatenate([k_pos0 + np.arange(Sk), k_pos0 + Sk + np.arange(7)])
    _, _, _, lse, delta = oracle.attention_bwd(q, kf, vf, do, scale=scale, causal=causal, q_pos0=q_pos0,
                                               k_pos=kpos)
    gq, gk, gv = oracle.block_bwd(q, k, v, do, lse, delta, scale=scale, causal=causal, q_pos0=q_pos0,
                                  k_pos0=k_pos0)
    dq = torch.zeros((B, Hq, Sq, D), dtype=torch.float32, device=DEV)
    dk = torch.zeros((B, Hkv, Sk, D), dtype=torch.float32, device=DEV)
    dv = torch.zeros((B, Hkv, Sk, Dv), dtype=torch.float32, device=DEV)
    lse_d = to_dev(np.where(np.isfinite(lse), lse, -np.inf), torch.float32)
    ra.block_attn_bwd_step(to_dev(q), to_dev(do), lse_d, to_dev(delta, torch.float32), to_dev(k), to_dev(v),
                           dq, dk, dv, q_pos0=q_pos0, k_pos0=k_pos0, causal=causal, scale=scale)
    torch.cuda.synchronize()
    grad_close(dq, gq, "dq")
    grad_close(dk, gk, "dk")
    grad_close(dv, gv, "dv")


def test_bwd_step_accumulates(ra):
    """The step adds into the accumulators: two identical calls give twice one call."""
    B, Hq, Hkv, S, D = 1, 2, 1, 200, 128
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=77, dtype="bf16")
    do = randn_np((B, Hq, S, D), 78, "bf16")
    _, _, _, lse, delta = oracle.attention_bwd(q, k, v, do, scale=0.1, causal=True)
    args = [to_dev(q), to_dev(do), to_dev(lse, torch.float32), to_dev(delta, torch.float32), to_dev(k), to_dev(v)]
    outs = [[torch.zeros(s, dtype=torch.float32, device=DEV) for s in ((B, Hq, S, D), (B, Hkv, S, D), (B, Hkv, S, D))]
            for _ in range(2)]
    ra.block_attn_bwd_step(*args, *outs[0], q_pos0=0, k_pos0=0, causal=True, scale=0.1)
    for _ in range(2):
        ra.block_attn_bwd_step(*args, *outs[1], q_pos0=0, k_pos0=0, causal=True, scale=0.1)
    torch.cuda.synchronize()
    for a, b in zip(outs[0], outs[1]):
        assert torch.allclose(2 * a, b, rtol=1e-6, atol=1e-6)


def test_bwd_preprocess(ra):
    rows, Dv = 1001, 128
    o = randn_np((rows, Dv), 90, "bf16")
    do = randn_np((rows, Dv), 91, "bf16")
    delta = ra.attn_bwd_preprocess(to_dev(o), to_dev(do))
    torch.cuda.synchronize()
    ref = (o.astype(np.float64) * do.astype(np.float64)).sum(1)
    assert np.max(np.abs(np64(delta) - ref)) <= 1e-4 * (1 + np.abs(ref).max())


@pytest.mark.parametrize("dims", DIMS)
@pytest.mark.parametrize("causal", [False, True])
def test_whole_backward_after_gpu_forward(ra, dims, causal):
    """ring_attn_fwd on the GPU, then attn_bwd: the exact gradients of the exact
    attention of the same bf16 inputs, GQA 4:1, ragged length."""
    B, Hq, Hkv, S = 1, 8, 2, 777
    D, Dv = dims
    say(f"attn_bwd whole D{D}/{Dv} causal={causal}")
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, Dv, seed=700 + D, dtype="bf16")
    do = randn_np((B, Hq, S, Dv), 710 + D, "bf16")
    dq_, dk_, dv_ = to_dev(q), to_dev(k), to_dev(v)
    o, lse = ra.ring_attn_fwd(dq_, dk_, dv_, P=1, causal=causal)
    gq, gk, gv = ra.attn_bwd(dq_, dk_, dv_, o, lse, to_dev(do), causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, scale=1 / math.sqrt(D), causal=causal)
    grad_close(gq, rq, "dq")
    grad_close(gk, rk, "dk")
    grad_close(gv, rv, "dv")


@pytest.mark.parametrize("dims", DIMS)
def test_whole_backward_group3_batch2(ra, dims):
    """The same after a GPU forward with a group of three query heads per KV head
    (not a power of two) and two sequences: the kernels' (batch, KV head, query
    head) decompositions and the dK/dV sum over a group."""
    B, Hq, Hkv, S = 2, 6, 2, 401
    D, Dv = dims
    say(f"attn_bwd whole, group 3, batch 2, D{D}/{Dv}")
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, Dv, seed=720 + D, dtype="bf16")
    do = randn_np((B, Hq, S, Dv), 730 + D, "bf16")
    dq_, dk_, dv_ = to_dev(q), to_dev(k), to_dev(v)
    o, lse = ra.ring_attn_fwd(dq_, dk_, dv_, P=1, causal=True)
    gq, gk, gv = ra.attn_bwd(dq_, dk_, dv_, o, lse, to_dev(do), causal=True)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, scale=1 / math.sqrt(D), causal=True)
    grad_close(gq, rq, "dq")
    grad_close(gk, rk, "dk")
    grad_close(gv, rv, "dv")


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_ring_backward_protocol_equals_whole(ra, dims, causal):
    """Ring backward on one GPU: for every query partition i and ring step s, the
    step over (partition i, block (i - s) mod P) accumulates into dq_i and into the
    block's travelling dk_j / dv_j. The sums equal the whole-sequence backward."""
    B, Hq, Hkv, Sp, P = 1, 4, 2, 160, 4
    D, Dv = dims
    S = Sp * P
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, Dv, seed=801, dtype="bf16")
    do = randn_np((B, Hq, S, Dv), 802, "bf16")
    dq_, dk_, dv_, ddo = to_dev(q), to_dev(k), to_dev(v), to_dev(do)
    o, lse = ra.ring_attn_fwd(dq_, dk_, dv_, P=P, causal=causal)
    gq, gk, gv = ra.attn_bwd(dq_, dk_, dv_, o, lse, ddo, causal=causal)
    delta = ra.attn_bwd_preprocess(o, ddo)
    part = lambda t, i: t[:, :, i * Sp:(i + 1) * Sp].contiguous()
    dq_parts = [torch.zeros((B, Hq, Sp, D), dtype=torch.float32, device=DEV) for _ in range(P)]
    dk_blk = [torch.zeros((B, Hkv, Sp, D), dtype=torch.float32, device=DEV) for _ in range(P)]
    dv_blk = [torch.zeros((B, Hkv, Sp, Dv), dtype=torch.float32, device=DEV) for _ in range(P)]
    for i in range(P):
        for j, kind in ra.ring_schedule(P, i, causal):
            if kind == "skip":
                continue
            ra.block_attn_bwd_step(part(dq_, i), part(ddo, i), part(lse, i), part(delta, i), part(dk_, j),
                                   part(dv_, j), dq_parts[i], dk_blk[j], dv_blk[j], q_pos0=i * Sp,
                                   k_pos0=j * Sp, causal=causal)
    torch.cuda.synchronize()
    rq, rk, rv = torch.cat(dq_parts, 2), torch.cat(dk_blk, 2), torch.cat(dv_blk, 2)
    for a, b, name in ((rq, gq, "dq"), (rk, gk, "dk"), (rv, gv, "dv")):
        err = float((a - b).abs().max())
        say(f"ring vs whole {name}: {err:.3e}")
        assert err <= 1e-4 * float(b.abs().max()) + 1e-6, name
    ref = oracle.attention_bwd(q, k, v, do, scale=1 / math.sqrt(D), causal=causal)
    grad_close(rq, ref[0], "ring dq")
    grad_close(rk, ref[1], "ring dk")
    grad_close(rv, ref[2], "ring dv")


def test_striped_ring_backward_with_virtual_positions(ra):
    """Striped layout: every (partition i, block j) step uses the virtual positions
    of the striped mask (query: local row, key: local index + [j > i]). The
    accumulated gradients, taken back to natural order, are the exact gradients of
    the natural-order sequence."""
    B, Hq, Hkv, Sp, P, D = 1, 4, 2, 120, 4, 128
    S = Sp * P
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=901, dtype="bf16")
    do = randn_np((B, Hq, S, D), 902, "bf16")
    st = lambda x: np.concatenate([x[:, :, p::P] for p in range(P)], axis=2)
    dq_, dk_, dv_, ddo = (to_dev(st(x)) for x in (q, k, v, do))
    o, lse = ra.ring_attn_fwd(dq_, dk_, dv_, P=P, causal=True, layout="striped")
    delta = ra.attn_bwd_preprocess(o, ddo)
    part = lambda t, i: t[:, :, i * Sp:(i + 1) * Sp].contiguous()
    dqs = [torch.zeros((B, Hq, Sp, D), dtype=torch.float32, device=DEV) for _ in range(P)]
    dks = [torch.zeros((B, Hkv, Sp, D), dtype=torch.float32, device=DEV) for _ in range(P)]
    dvs = [torch.zeros((B, Hkv, Sp, D), dtype=torch.float32, device=DEV) for _ in range(P)]
    for i in range(P):
        for j, _ in ra.ring_schedule(P, i, True, "striped"):
            ra.block_attn_bwd_step(part(dq_, i), part(ddo, i), part(lse, i), part(delta, i), part(dk_, j),
                                   part(dv_, j), dqs[i], dks[j], dvs[j], q_pos0=0, k_pos0=1 if j > i else 0,
                                   causal=True)
    torch.cuda.synchronize()
    rq, rk, rv, _, _ = oracle.attention_bwd(q, k, v, do, scale=1 / math.sqrt(D), causal=True)
    grad_close(torch.cat(dqs, 2), st(rq), "striped dq")
    grad_close(torch.cat(dks, 2), st(rk), "striped dk")
    grad_close(torch.cat(dvs, 2), st(rv), "striped dv")
