"""Planted mistakes in the oracle, on the CPU: each plausible slip (dropped key, wrong
sign, transposed operand, missing scale, off-by-one mask, wrong GQA map, wrong merge
weight) must be caught by at least one of the independent pins. This shows the pins
are discriminating, not that the oracle agrees with itself."""
import math

import numpy as np
import pytest

import oracle
import oracle.exact as oa
from workloads import prefill_inputs_np

mpmath = pytest.importorskip("mpmath")


def _pin_suite(attn, merge):
    """Run a few independent pins against an attention/merge pair. Returns True when
    every pin holds."""
    ok = True
    rng = np.random.default_rng(1)
    # closed form: Q = 0 -> prefix mean, LSE = ln n
    q = np.zeros((1, 2, 6, 3))
    k = rng.standard_normal((1, 1, 6, 3))
    v = rng.standard_normal((1, 1, 6, 2))
    o, l = attn(q, k, v, scale=1.0, causal=True, q_pos0=0, k_pos0=0)
    cs = np.cumsum(v[0, 0], axis=0)
    for r in range(6):
        ok &= abs(l[0, 0, r] - math.log(r + 1)) < 1e-12
        ok &= np.max(np.abs(o[0, 1, r] - cs[r] / (r + 1))) < 1e-12
    # brute force on one row with a non-zero query, in mpmath
    q, k, v = prefill_inputs_np(1, 2, 1, 3, 5, 4, 3, seed=5)
    o, l = attn(q, k, v, scale=0.6, causal=False, q_pos0=0, k_pos0=0)
    mpmath.mp.dps = 40
    for h in range(2):
        w = [mpmath.exp(mpmath.mpf(0.6) * mpmath.fsum(mpmath.mpf(float(q[0, h, 1, d])) * mpmath.mpf(float(k[0, 0, c, d]))
                                                      for d in range(4))) for c in range(5)]
        Z = mpmath.fsum(w)
        ok &= abs(l[0, h, 1] - float(mpmath.log(Z))) < 1e-12
        ob = [float(mpmath.fsum(w[c] * mpmath.mpf(float(v[0, 0, c, e])) for c in range(5)) / Z) for e in range(3)]
        ok &= np.max(np.abs(o[0, h, 1] - np.array(ob))) < 1e-12
    # GQA: heads 2,3 read KV head 1 -> equal to MHA with repeated heads computed by hand
    q, k, v = (x.astype(np.float64) for x in prefill_inputs_np(1, 4, 2, 2, 4, 3, 2, seed=6))
    o, l = attn(q, k, v, scale=0.5, causal=False, q_pos0=0, k_pos0=0)
    for h in range(4):
        s = 0.5 * q[0, h] @ k[0, h // 2].T
        ok &= np.max(np.abs(l[0, h] - np.log(np.exp(s).sum(1)))) < 1e-12
    # blockwise merge == one shot
    q, k, v = prefill_inputs_np(1, 1, 1, 4, 10, 3, 2, seed=7)
    o_ref, l_ref = attn(q, k, v, scale=0.8, causal=True, q_pos0=6, k_pos0=0)
    oa_, la_ = attn(q, k[:, :, :4], v[:, :, :4], scale=0.8, causal=True, q_pos0=6, k_pos0=0)
    ob_, lb_ = attn(q, k[:, :, 4:], v[:, :, 4:], scale=0.8, causal=True, q_pos0=6, k_pos0=4)
    om, lm = merge(oa_, la_, ob_, lb_)
    ok &= np.max(np.abs(om - o_ref)) < 1e-12 and np.max(np.abs(lm - l_ref)) < 1e-12
    return bool(ok)


def _mut_attention(kind):
    def attn(q, k, v, *, scale, causal, q_pos0=0, k_pos0=0):
        q, k, v = (np.asarray(x, float) for x in (q, k, v))
        B, Hq, Sq, _ = q.shape
        Hkv, Sk = k.shape[1], k.shape[2]
        grp = Hq // Hkv
        qp = q_pos0 + np.arange(Sq)
        kp = k_pos0 + np.arange(Sk)
        if kind == "mask_off_by_one":
            vis = kp[None, :] < qp[:, None] if causal else np.ones((Sq, Sk), bool)
        else:
            vis = oa.visible(qp, kp, causal)
        if kind == "drop_last_key":
            vis = vis.copy()
            vis[:, -1] = False
        o = np.zeros((B, Hq, Sq, v.shape[3]))
        l = np.full((B, Hq, Sq), -np.inf)
        for b in range(B):
            for h in range(Hq):
                g = h % Hkv if kind == "gqa_modulo" else h // grp
                sc = 1.0 if kind == "no_scale" else scale
                s = sc * (q[b, h] @ k[b, g].T)
                if kind == "sign":
                    s = -s
                if kind == "transposed_v" and Sk == v.shape[3]:
                    o_, l_ = oa._softmax_rows(s, vis, v[b, g].T)
                else:
                    o_, l_ = oa._softmax_rows(s, vis, v[b, g])
                if kind == "lse_log2":
                    l_ = l_ / math.log(2)
                o[b, h], l[b, h] = o_, l_
        return o, l
    return attn


def _mut_merge(o_a, l_a, o_b, l_b):
    # forgets to rescale the first side
    o, l = oracle.merge(o_a, l_a, o_b, l_b)
    w_b = np.exp(np.asarray(l_b) - l)
    return np.asarray(o_a) + w_b[..., None] * np.asarray(o_b), l


def test_true_oracle_passes_pin_suite():
    assert _pin_suite(oracle.attention, oracle.merge)


@pytest.mark.parametrize("kind", ["mask_off_by_one", "drop_last_key", "gqa_modulo", "no_scale",
                                  "sign", "lse_log2"])
def test_attention_mutants_are_caught(kind):
    assert not _pin_suite(_mut_attention(kind), oracle.merge)


def test_merge_mutant_is_caught():
    assert not _pin_suite(oracle.attention, _mut_merge)
