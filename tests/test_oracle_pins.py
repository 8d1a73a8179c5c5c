"""Pins for the fp64 oracle: brute force, closed forms, library special cases and the
pages' own tables. None of these retypes the oracle's formula: each checks it
against something fixed independently (exact arithmetic, a closed form, scipy's
routines, or numbers printed on the pages)."""
import math

import numpy as np
import pytest

import oracle
from workloads import randn_np, prefill_inputs_np
from conftest import read_golden

mpmath = pytest.importorskip("mpmath")
scipy_special = pytest.importorskip("scipy.special")


# ------------------------------------------------------------------------------
# brute force in 50-digit arithmetic, scalar loops, no max shift
# ------------------------------------------------------------------------------

def _brute(q, k, v, scale, causal, q_pos0, k_pos0):
    mpmath.mp.dps = 50
    B, Hq, Sq, D = q.shape
    Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    grp = Hq // Hkv
    O = np.zeros((B, Hq, Sq, Dv))
    L = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // grp
            for r in range(Sq):
                weights = []
                for c in range(Sk):
                    if causal and (k_pos0 + c) > (q_pos0 + r):
                        continue
                    dot = mpmath.fsum(mpmath.mpf(float(q[b, h, r, d])) * mpmath.mpf(float(k[b, g, c, d]))
                                      for d in range(D))
                    weights.append((c, mpmath.exp(mpmath.mpf(scale) * dot)))
                if not weights:
                    O[b, h, r] = 0.0
                    L[b, h, r] = -np.inf
                    continue
                Z = mpmath.fsum(w for _, w in weights)
                L[b, h, r] = float(mpmath.log(Z))
                for e in range(Dv):
                    O[b, h, r, e] = float(mpmath.fsum(w * mpmath.mpf(float(v[b, g, c, e])) for c, w in weights) / Z)
    return O, L


@pytest.mark.parametrize("Hq,Hkv", [(1, 1), (4, 2), (4, 1)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("pos", [(0, 0), (5, 2), (3, 7)])
def test_bruteforce_tiny(Hq, Hkv, causal, pos):
    q_pos0, k_pos0 = pos
    rng = np.random.default_rng(11 + Hq * 7 + Hkv + int(causal) * 101 + q_pos0)
    Sq, Sk, D, Dv = 5, 7, 3, 4          # D_qk != D_v on purpose
    q = rng.standard_normal((2, Hq, Sq, D))
    k = rng.standard_normal((2, Hkv, Sk, D))
    v = rng.standard_normal((2, Hkv, Sk, Dv))
    scale = 0.7
    o, lse = oracle.attention(q, k, v, scale=scale, causal=causal, q_pos0=q_pos0, k_pos0=k_pos0)
    ob, lb = _brute(q, k, v, scale, causal, q_pos0, k_pos0)
    fin = np.isfinite(lb)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(o - ob)) <= 1e-12
    assert np.max(np.abs(lse[fin] - lb[fin])) <= 1e-12


# ------------------------------------------------------------------------------
# library special cases: scipy's logsumexp / softmax on independently built scores
# ------------------------------------------------------------------------------

def test_matches_scipy_softmax_logsumexp():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 2, 33, 16))
    k = rng.standard_normal((1, 2, 41, 16))
    v = rng.standard_normal((1, 2, 41, 9))
    scale = 0.25
    o, lse = oracle.attention(q, k, v, scale=scale, causal=False)
    for h in range(2):
        s = np.einsum("rd,cd->rc", q[0, h], k[0, h]) * scale
        assert np.allclose(lse[0, h], scipy_special.logsumexp(s, axis=1), atol=1e-12, rtol=0)
        assert np.allclose(o[0, h], scipy_special.softmax(s, axis=1) @ v[0, h], atol=1e-12, rtol=0)


def test_probabilities_via_identity_values():
    """With V = I the output rows are the attention probabilities themselves: they must
    be non-negative, sum to 1, be zero on hidden keys and match scipy's softmax."""
    rng = np.random.default_rng(6)
    S = 12
    q = rng.standard_normal((1, 1, S, 8))
    k = rng.standard_normal((1, 1, S, 8))
    v = np.eye(S)[None, None]
    p, _ = oracle.attention(q, k, v, scale=0.4, causal=True)
    p = p[0, 0]
    assert np.all(p >= 0)
    assert np.max(np.abs(p.sum(axis=1) - 1.0)) <= 1e-14
    assert np.all(np.triu(p, 1) == 0.0)
    s = (q[0, 0] @ k[0, 0].T) * 0.4
    for r in range(S):
        assert np.allclose(p[r, : r + 1], scipy_special.softmax(s[r, : r + 1]), atol=1e-15)


# ------------------------------------------------------------------------------
# closed forms
# ------------------------------------------------------------------------------

@pytest.mark.parametrize("causal", [False, True])
def test_constant_values_give_that_value(causal):
    rng = np.random.default_rng(7)
    q = rng.standard_normal((2, 4, 20, 8)) * 3
    k = rng.standard_normal((2, 2, 20, 8)) * 3
    c = rng.standard_normal(5)
    v = np.broadcast_to(c, (2, 2, 20, 5)).copy()
    o, _ = oracle.attention(q, k, v, scale=0.5, causal=causal)
    assert np.max(np.abs(o - c)) <= 1e-13


@pytest.mark.parametrize("q_pos0,k_pos0", [(0, 0), (10, 4), (3, 3)])
def test_zero_query_gives_prefix_mean_and_log_count(q_pos0, k_pos0):
    """Q = 0 makes every visible score 0: O is the mean of the visible V rows (a running
    mean under the causal mask, computed here by cumulative sums) and LSE = ln(count)."""
    rng = np.random.default_rng(8)
    Sq, Sk = 9, 14
    q = np.zeros((1, 2, Sq, 4))
    k = rng.standard_normal((1, 1, Sk, 4))
    v = rng.standard_normal((1, 1, Sk, 3))
    o, lse = oracle.attention(q, k, v, scale=1.0, causal=True, q_pos0=q_pos0, k_pos0=k_pos0)
    csum = np.cumsum(v[0, 0], axis=0)
    for r in range(Sq):
        n = min(max(q_pos0 + r - k_pos0 + 1, 0), Sk)
        for h in range(2):
            if n == 0:
                assert lse[0, h, r] == -np.inf and np.all(o[0, h, r] == 0)
            else:
                assert abs(lse[0, h, r] - math.log(n)) <= 1e-14
                assert np.max(np.abs(o[0, h, r] - csum[n - 1] / n)) <= 1e-13


def test_ramp_values_with_zero_query():
    """V[c, 0] = c and Q = 0: causal row r averages 0..r, giving r/2; non-causal gives (S-1)/2."""
    S = 64
    q = np.zeros((1, 1, S, 2))
    k = np.ones((1, 1, S, 2))
    v = np.arange(S, dtype=float).reshape(1, 1, S, 1)
    oc, _ = oracle.attention(q, k, v, scale=1.0, causal=True)
    on, _ = oracle.attention(q, k, v, scale=1.0, causal=False)
    assert np.max(np.abs(oc[0, 0, :, 0] - np.arange(S) / 2.0)) <= 1e-12
    assert np.max(np.abs(on[0, 0, :, 0] - (S - 1) / 2.0)) <= 1e-12


def test_single_key_and_causal_first_row():
    rng = np.random.default_rng(9)
    q = rng.standard_normal((1, 1, 6, 5))
    k = rng.standard_normal((1, 1, 6, 5))
    v = rng.standard_normal((1, 1, 6, 3))
    o, lse = oracle.attention(q, k, v, scale=0.3, causal=True)
    s00 = 0.3 * float(np.dot(q[0, 0, 0], k[0, 0, 0]))
    assert abs(lse[0, 0, 0] - s00) <= 1e-15
    assert np.max(np.abs(o[0, 0, 0] - v[0, 0, 0])) <= 1e-15
    o1, l1 = oracle.attention(q[:, :, 2:3], k[:, :, 4:5], v[:, :, 4:5], scale=0.3, causal=False)
    assert abs(l1[0, 0, 0] - 0.3 * float(np.dot(q[0, 0, 2], k[0, 0, 4]))) <= 1e-15
    assert np.max(np.abs(o1[0, 0, 0] - v[0, 0, 4])) <= 1e-15


def test_identical_keys():
    rng = np.random.default_rng(10)
    n = 17
    kk = rng.standard_normal(6)
    q = rng.standard_normal((1, 1, 3, 6))
    k = np.broadcast_to(kk, (1, 1, n, 6)).copy()
    v = rng.standard_normal((1, 1, n, 4))
    o, lse = oracle.attention(q, k, v, scale=0.9, causal=False)
    for r in range(3):
        s = 0.9 * float(np.dot(q[0, 0, r], kk))
        assert abs(lse[0, 0, r] - (s + math.log(n))) <= 1e-13
        assert np.max(np.abs(o[0, 0, r] - v[0, 0].mean(axis=0))) <= 1e-13


def test_empty_rows_are_zero_and_neg_inf():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((1, 1, 4, 3))
    k = rng.standard_normal((1, 1, 5, 3))
    v = rng.standard_normal((1, 1, 5, 2))
    o, lse = oracle.attention(q, k, v, scale=1.0, causal=True, q_pos0=0, k_pos0=100)
    assert np.all(lse == -np.inf)
    assert np.all(o == 0.0)


def test_gqa_equals_repeated_kv_heads():
    q, k, v = prefill_inputs_np(2, 8, 2, 11, 13, 6, 5, seed=3)
    o, lse = oracle.attention(q, k, v, scale=0.4, causal=True, q_pos0=2, k_pos0=0)
    kr = np.repeat(k, 4, axis=1)
    vr = np.repeat(v, 4, axis=1)
    o2, l2 = oracle.attention(q, kr, vr, scale=0.4, causal=True, q_pos0=2, k_pos0=0)
    assert np.max(np.abs(o - o2)) == 0.0 and np.max(np.abs(lse - l2)) == 0.0


def test_scale_sanity_on_normal_inputs():
    """For N(0,1) Q, K with scale 1/sqrt(d), scores are ~N(0,1) so LSE - ln(n) averages
    log E[e^X] = 1/2. A dropped or doubled scale moves this far outside +-0.05."""
    d = 64
    q, k, v = prefill_inputs_np(1, 1, 1, 256, 4096, d, 4, seed=77)
    _, lse = oracle.attention(q, k, v, scale=1 / math.sqrt(d), causal=False)
    assert abs(float(np.mean(lse - math.log(4096))) - 0.5) < 0.05


# ------------------------------------------------------------------------------
# rows of the oracle usable one by one
# ------------------------------------------------------------------------------

def test_attention_rows_matches_full():
    q, k, v = prefill_inputs_np(1, 4, 2, 30, 50, 8, 6, seed=21)
    o, lse = oracle.attention(q, k, v, scale=0.35, causal=True, q_pos0=20, k_pos0=0)
    rows = [3, 0, 29, 17]
    for h in range(4):
        orow, lrow = oracle.attention_rows(q[0, h, rows], 20 + np.array(rows), k[0, h // 2], v[0, h // 2],
                                           scale=0.35, causal=True, k_pos0=0)
        assert np.max(np.abs(orow - o[0, h, rows])) <= 1e-14
        assert np.max(np.abs(lrow - lse[0, h, rows])) <= 1e-14


# ------------------------------------------------------------------------------
# pages' tables
# ------------------------------------------------------------------------------

def test_kv_cache_table():
    for tokens, gib in read_golden("kv_cache_llama3_70b.txt"):
        b = oracle.kv_cache_bytes(layers=80, h_kv=8, d_h=128, n=int(tokens), bytes_per_value=2)
        assert b == int(round(gib * 2**30))


def test_decode_bound_table():
    kv_rows = {int(t): g for t, g in read_golden("kv_cache_llama3_70b.txt")}
    for tokens, per_card_gib, ms, tbps in read_golden("decode_bound_h100.txt"):
        t = oracle.decode_lower_bound_s(per_card_gib * 1e9, tbps * 1e12) * 1e3
        # the page prints one or two significant figures behind "~"
        assert abs(t - ms) <= 0.07 * ms, (tokens, t, ms)
        # the per-card figure is the one-sequence KV over TP=4 (exact for 32K and 128K)
        whole = oracle.kv_cache_bytes(80, 8, 128, int(tokens), 2) / 2**30 / 4
        assert abs(whole - per_card_gib) <= 0.03 * per_card_gib
        if int(tokens) in kv_rows and int(tokens) < 1 << 20:
            assert whole == per_card_gib


def test_ring_order_matches_page_walkthrough():
    for dev, r0, r1 in read_golden("ring_flow_4gpu.txt"):
        sched = oracle.ring_schedule(4, int(dev), causal=False)
        assert sched[0][0] == int(r0) and sched[1][0] == int(r1)
        # every KV block is visited exactly once in P rounds
        assert sorted(j for j, _ in sched) == [0, 1, 2, 3]


@pytest.mark.parametrize("P", [1, 2, 4, 8, 13])
def test_ring_schedule_class_counts(P):
    diag = full = skip = 0
    for i in range(P):
        s = oracle.ring_schedule(P, i, causal=True)
        assert s[0] == (i, "diag")
        diag += sum(1 for _, c in s if c == "diag")
        full += sum(1 for _, c in s if c == "full")
        skip += sum(1 for _, c in s if c == "skip")
        for j, c in s:
            assert c == ("skip" if j > i else "diag" if j == i else "full")
    assert diag == P and full == skip == P * (P - 1) // 2


def test_visible_pair_counts_by_enumeration():
    for Sp, P in [(3, 4), (5, 2), (4, 1)]:
        S = Sp * P
        vis = oracle.visible(np.arange(S), np.arange(S), True)
        assert int(vis.sum()) == oracle.visible_pairs_aligned_causal(S)
        for i in range(P):
            assert int(vis[i * Sp:(i + 1) * Sp].sum()) == oracle.visible_pairs_partition(Sp, P, i, True)
        assert oracle.visible_pairs_partition(Sp, P, 0, False) == Sp * S


def test_flop_count_agrees_with_cp_equation():
    """The per-pair FLOP count (two O(n^2 d) terms, QK^T and PV) times all S^2 pairs of one
    head equals the numerator of the pages' prefill compute-time equation at cp=1, R=1."""
    S, Dqk, Dv = 4096, 192, 128
    assert oracle.attention_flops(S * S, 1, Dqk, Dv) == oracle.prefill_compute_time_s(1, S, Dqk, Dv, 1, 1.0)
