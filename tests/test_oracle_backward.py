"""Pins of the oracle's attention gradients: central finite differences of the
forward oracle (a different code path from the gradient formulas), torch autograd
in fp64 (a library routine), and the blockwise decomposition summing back."""
import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

import oracle
from workloads import prefill_inputs_np


def loss(q, k, v, dout, **kw):
    o, _ = oracle.attention(q, k, v, **kw)
    return float((o * dout).sum())


def fd_grad(x, f, eps=1e-6):
    g = np.zeros_like(x)
    it = np.nditer(x, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        xp = x.copy(); xp[i] += eps
        xm = x.copy(); xm[i] -= eps
        g[i] = (f(xp) - f(xm)) / (2 * eps)
    return g


@pytest.mark.parametrize("causal,Hq,Hkv,q_pos0", [(False, 2, 1, 0), (True, 2, 2, 0), (True, 4, 2, 3)])
def test_gradients_match_finite_differences(causal, Hq, Hkv, q_pos0):
    rng = np.random.default_rng(11)
    B, Sq, Sk, Dqk, Dv = 1, 4, 6, 3, 2
    q = rng.standard_normal((B, Hq, Sq, Dqk))
    k = rng.standard_normal((B, Hkv, Sk, Dqk))
    v = rng.standard_normal((B, Hkv, Sk, Dv))
    do = rng.standard_normal((B, Hq, Sq, Dv))
    kw = dict(scale=0.7, causal=causal, q_pos0=q_pos0, k_pos0=0)
    dq, dk, dv, lse, delta = oracle.attention_bwd(q, k, v, do, **kw)
    assert np.max(np.abs(dq - fd_grad(q, lambda x: loss(x, k, v, do, **kw)))) < 1e-7
    assert np.max(np.abs(dk - fd_grad(k, lambda x: loss(q, x, v, do, **kw)))) < 1e-7
    assert np.max(np.abs(dv - fd_grad(v, lambda x: loss(q, k, x, do, **kw)))) < 1e-7
    o, l_ref = oracle.attention(q, k, v, **kw)
    assert np.max(np.abs(lse - l_ref)) < 1e-12
    assert np.max(np.abs(delta - (o * do).sum(-1))) < 1e-12


@pytest.mark.parametrize("causal", [False, True])
def test_gradients_match_torch_autograd(causal):
    B, Hq, Hkv, S, Dqk, Dv = 2, 4, 2, 9, 8, 6
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, Dqk, Dv, seed=321)
    do = np.random.default_rng(5).standard_normal((B, Hq, S, Dv))
    scale = 0.35
    dq, dk, dv, _, _ = oracle.attention_bwd(q, k, v, do, scale=scale, causal=causal)
    tq, tk, tv = (torch.tensor(np.asarray(x, dtype=np.float64), requires_grad=True) for x in (q, k, v))
    kr = tk.repeat_interleave(Hq // Hkv, dim=1)
    vr = tv.repeat_interleave(Hq // Hkv, dim=1)
    s = scale * tq @ kr.transpose(-1, -2)
    if causal:
        s = s.masked_fill(torch.ones(S, S, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vr
    (o * torch.tensor(do)).sum().backward()
    assert np.max(np.abs(dq - tq.grad.numpy())) < 1e-12
    assert np.max(np.abs(dk - tk.grad.numpy())) < 1e-12
    assert np.max(np.abs(dv - tv.grad.numpy())) < 1e-12


@settings(max_examples=30, deadline=None)
@given(cuts=st.lists(st.integers(1, 19), min_size=0, max_size=3, unique=True), causal=st.booleans(),
       seed=st.integers(0, 1000))
def test_blockwise_contributions_sum_to_the_whole(cuts, causal, seed):
    """Cut the keys at arbitrary points and the queries in two: the per-pair
    contributions, computed with the full-row lse and delta, add up to the
    whole-sequence gradients (the ring backward's accumulation)."""
    B, Hq, Hkv, S, D = 1, 2, 1, 20, 4
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=seed)
    do = np.random.default_rng(seed).standard_normal((B, Hq, S, D))
    kw = dict(scale=0.5, causal=causal)
    dq, dk, dv, lse, delta = oracle.attention_bwd(q, k, v, do, **kw)
    kb = [0] + sorted(cuts) + [S]
    qb = [0, 7, S]
    aq, ak, av = np.zeros_like(dq), np.zeros_like(dk), np.zeros_like(dv)
    for a, b in zip(qb[:-1], qb[1:]):
        for c, d in zip(kb[:-1], kb[1:]):
            gq, gk, gv = oracle.block_bwd(q[:, :, a:b], k[:, :, c:d], v[:, :, c:d], do[:, :, a:b],
                                          lse[:, :, a:b], delta[:, :, a:b], q_pos0=a, k_pos0=c, **kw)
            aq[:, :, a:b] += gq
            ak[:, :, c:d] += gk
            av[:, :, c:d] += gv
    assert np.max(np.abs(aq - dq)) < 1e-12
    assert np.max(np.abs(ak - dk)) < 1e-12
    assert np.max(np.abs(av - dv)) < 1e-12


def test_rows_without_visible_keys_have_no_gradient():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 3, 4))
    k = rng.standard_normal((1, 1, 5, 4))
    v = rng.standard_normal((1, 1, 5, 4))
    do = rng.standard_normal((1, 1, 3, 4))
    # keys at positions 10..14, queries at 0..2: nothing visible under a causal mask
    dq, dk, dv, lse, delta = oracle.attention_bwd(q, k, v, do, scale=1.0, causal=True, k_pos0=10)
    assert np.all(dq == 0) and np.all(dk == 0) and np.all(dv == 0)
    assert np.all(np.isneginf(lse)) and np.all(delta == 0)
    gq, gk, gv = oracle.block_bwd(q, k, v, do, lse, delta, scale=1.0, causal=True, k_pos0=10)
    assert np.all(gq == 0) and np.all(gk == 0) and np.all(gv == 0)


def _mutant_bwd(q, k, v, do, scale, kind):
    """The gradient formulas with one planted slip (single head, no mask)."""
    q, k, v, do = q[0, 0], k[0, 0], v[0, 0], do[0, 0]
    s = scale * q @ k.T
    p = np.exp(s - s.max(1, keepdims=True))
    p /= p.sum(1, keepdims=True)
    o = p @ v
    dp = do @ v.T
    delta = (do * o).sum(1)
    if kind == "no_delta":
        delta = 0 * delta
    ds = p * (dp - delta[:, None])
    if kind == "sign":
        ds = -ds
    dq = scale * ds @ k
    dk = (ds.T @ q) * (1.0 if kind == "dk_unscaled" else scale)
    dv = p @ do[: p.shape[1]] if kind == "dv_untransposed" else p.T @ do
    return dq, dk, dv


@pytest.mark.parametrize("kind", ["no_delta", "sign", "dk_unscaled", "dv_untransposed"])
def test_planted_gradient_slips_are_caught_by_finite_differences(kind):
    rng = np.random.default_rng(12)
    S, D = 5, 3
    q = rng.standard_normal((1, 1, S, D))
    k = rng.standard_normal((1, 1, S, D))
    v = rng.standard_normal((1, 1, S, D))
    do = rng.standard_normal((1, 1, S, D))
    kw = dict(scale=0.8, causal=False)
    fq = fd_grad(q, lambda x: loss(x, k, v, do, **kw))[0, 0]
    fk = fd_grad(k, lambda x: loss(q, x, v, do, **kw))[0, 0]
    fv = fd_grad(v, lambda x: loss(q, k, x, do, **kw))[0, 0]
    good = _mutant_bwd(q, k, v, do, 0.8, "none")
    assert max(np.max(np.abs(a - b)) for a, b in zip(good, (fq, fk, fv))) < 1e-7
    bad = _mutant_bwd(q, k, v, do, 0.8, kind)
    assert max(np.max(np.abs(a - b)) for a, b in zip(bad, (fq, fk, fv))) > 1e-3
