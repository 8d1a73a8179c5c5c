"""Blockwise protocol pins: merging exact per-block results in any order, over any split
of the keys, gives one-shot attention; the ring order over P partitions gives the full
causal / non-causal result; an empty side is the identity of the merge."""
import numpy as np
import pytest
from hypothesis import given, settings, strategies as st

import oracle
from workloads import prefill_inputs_np


@settings(max_examples=60, deadline=None)
@given(
    sk=st.integers(min_value=1, max_value=40),
    cuts=st.lists(st.integers(min_value=1, max_value=39), max_size=6),
    causal=st.booleans(),
    q_pos0=st.integers(min_value=0, max_value=30),
    seed=st.integers(min_value=0, max_value=10_000),
    order_seed=st.integers(min_value=0, max_value=10_000),
)
def test_any_split_any_order_equals_one_shot(sk, cuts, causal, q_pos0, seed, order_seed):
    q, k, v = prefill_inputs_np(1, 2, 1, 7, sk, 5, 3, seed=seed)
    scale = 0.45
    o_ref, l_ref = oracle.attention(q, k, v, scale=scale, causal=causal, q_pos0=q_pos0, k_pos0=0)
    bounds = sorted({c for c in cuts if c < sk} | {0, sk})
    blocks = list(zip(bounds[:-1], bounds[1:]))
    np.random.default_rng(order_seed).shuffle(blocks)
    o = np.zeros_like(o_ref)
    lse = np.full_like(l_ref, -np.inf)
    for a, b in blocks:
        ob, lb = oracle.attention(q, k[:, :, a:b], v[:, :, a:b], scale=scale, causal=causal,
                                  q_pos0=q_pos0, k_pos0=a)
        o, lse = oracle.merge(o, lse, ob, lb)
    fin = np.isfinite(l_ref)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(o - o_ref)) <= 1e-12
    if fin.any():
        assert np.max(np.abs(lse[fin] - l_ref[fin])) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("P", [1, 3, 4])
def test_ring_protocol_equals_full_attention(causal, P):
    Sp = 6
    q, k, v = prefill_inputs_np(2, 4, 2, P * Sp, P * Sp, 8, 7, seed=40 + P)
    o_ref, l_ref = oracle.attention(q, k, v, scale=0.3, causal=causal)
    kb = [k[:, :, j * Sp:(j + 1) * Sp] for j in range(P)]
    vb = [v[:, :, j * Sp:(j + 1) * Sp] for j in range(P)]
    for i in range(P):
        o, lse = oracle.ring_attention(q[:, :, i * Sp:(i + 1) * Sp], kb, vb, i=i, scale=0.3,
                                       causal=causal, Sp=Sp)
        assert np.max(np.abs(o - o_ref[:, :, i * Sp:(i + 1) * Sp])) <= 1e-12
        assert np.max(np.abs(lse - l_ref[:, :, i * Sp:(i + 1) * Sp])) <= 1e-12
        # any other visiting order reaches the same result
        rev = list(range(P))[::-1]
        o2, l2 = oracle.ring_attention(q[:, :, i * Sp:(i + 1) * Sp], kb, vb, i=i, scale=0.3,
                                       causal=causal, Sp=Sp, block_order=rev)
        assert np.max(np.abs(o2 - o)) <= 1e-12 and np.max(np.abs(l2 - lse)) <= 1e-12


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("P", [1, 2, 4])
def test_striped_ring_equals_full_attention_on_strided_rows(causal, P):
    """Striped layout: partition p holds tokens p, p+P, p+2P, ... of the sequence.
    The ring over the striped partitions gives, row for row, one-shot attention
    over the sequence in natural order (positions 0..S-1) taken at those rows."""
    Sp = 5
    q, k, v = prefill_inputs_np(2, 4, 2, P * Sp, P * Sp, 8, 7, seed=140 + P)
    o_ref, l_ref = oracle.attention(q, k, v, scale=0.3, causal=causal)
    kb = [k[:, :, j::P] for j in range(P)]
    vb = [v[:, :, j::P] for j in range(P)]
    for i in range(P):
        o, lse = oracle.ring_attention(q[:, :, i::P], kb, vb, i=i, scale=0.3, causal=causal, Sp=Sp,
                                       layout="striped")
        assert np.max(np.abs(o - o_ref[:, :, i::P])) <= 1e-12
        assert np.max(np.abs(lse - l_ref[:, :, i::P])) <= 1e-12


def test_striped_schedule_and_positions():
    assert list(oracle.partition_positions(4, 3, 1, "striped")) == [1, 5, 9]
    assert list(oracle.partition_positions(4, 3, 1, "contiguous")) == [3, 4, 5]
    # every block of a causal striped ring is masked, none skipped; order unchanged
    for P in (1, 3, 8):
        for i in range(P):
            st_c = oracle.ring_schedule(P, i, True, "striped")
            assert [j for j, _ in st_c] == [j for j, _ in oracle.ring_schedule(P, i, True)]
            assert {kd for _, kd in st_c} == {"diag"}
            assert {kd for _, kd in oracle.ring_schedule(P, i, False, "striped")} == {"full"}
    with pytest.raises(ValueError):
        oracle.ring_schedule(4, 0, True, "zigzag")


@pytest.mark.parametrize("P,Sp", [(1, 7), (3, 5), (4, 8), (8, 3)])
def test_visible_pairs_per_partition_brute_force_and_balance(P, Sp):
    """The closed-form pair counts equal a brute-force count of the visibility
    matrix on the true positions. Causal striped partitions differ by Sp pairs per
    partition index (max - min = (P-1) Sp); contiguous ones by about Sp^2."""
    S = P * Sp
    for layout in ("contiguous", "striped"):
        counts = []
        for i in range(P):
            qp = oracle.partition_positions(P, Sp, i, layout)
            n = sum(int(oracle.visible(qp, oracle.partition_positions(P, Sp, j, layout), True).sum())
                    for j in range(P))
            assert n == oracle.visible_pairs_partition(Sp, P, i, True, layout)
            counts.append(n)
        assert sum(counts) == S * (S + 1) // 2
        if layout == "striped":
            assert max(counts) - min(counts) == (P - 1) * Sp
        else:
            assert max(counts) - min(counts) == (P - 1) * Sp * Sp


def test_dropped_or_doubled_block_moves_lse():
    """A wrong schedule (a block missing or visited twice) is visible in LSE by at
    least log(8/7) when 8 equal-size blocks carry similar mass."""
    P, Sp = 8, 32
    q, k, v = prefill_inputs_np(1, 1, 1, Sp, P * Sp, 16, 4, seed=90)
    kb = [k[:, :, j * Sp:(j + 1) * Sp] for j in range(P)]
    vb = [v[:, :, j * Sp:(j + 1) * Sp] for j in range(P)]
    scale = 0.25
    full, lf = oracle.ring_attention(q, kb, vb, i=P - 1, scale=scale, causal=False, Sp=Sp)
    _, ld = oracle.ring_attention(q, kb, vb, i=P - 1, scale=scale, causal=False, Sp=Sp,
                                  block_order=list(range(P - 1)))
    _, l2 = oracle.ring_attention(q, kb, vb, i=P - 1, scale=scale, causal=False, Sp=Sp,
                                  block_order=list(range(P)) + [3])
    assert np.min(lf - ld) > 0 and np.mean(lf - ld) > 0.5 * np.log(8 / 7)
    assert np.min(l2 - lf) > 0


def test_merge_identity_and_symmetry():
    rng = np.random.default_rng(3)
    o = rng.standard_normal((5, 4))
    l = rng.standard_normal(5)
    empty_o = np.zeros((5, 4))
    empty_l = np.full(5, -np.inf)
    om, lm = oracle.merge(o, l, empty_o, empty_l)
    assert np.array_equal(om, o) and np.array_equal(lm, l)
    om, lm = oracle.merge(empty_o, empty_l, o, l)
    assert np.array_equal(om, o) and np.array_equal(lm, l)
    ob, lb = rng.standard_normal((5, 4)), rng.standard_normal(5) + 100.0   # far apart, no overflow
    o1, l1 = oracle.merge(o, l, ob, lb)
    o2, l2 = oracle.merge(ob, lb, o, l)
    assert np.allclose(o1, o2, atol=1e-15) and np.allclose(l1, l2, atol=1e-13)
    oe, le = oracle.merge(empty_o, empty_l, empty_o, empty_l)
    assert np.all(le == -np.inf) and np.all(oe == 0) and not np.isnan(oe).any()


def test_splitkv_decode_equals_one_shot_for_any_split_count():
    rng = np.random.default_rng(4)
    B, Hq, Hkv, L, D = 2, 8, 2, 48, 6
    q = rng.standard_normal((B, Hq, D))
    k = rng.standard_normal((B, Hkv, L, D))
    v = rng.standard_normal((B, Hkv, L, 5))
    ref_o, ref_l = oracle.attention(q[:, :, None, :], k, v, scale=0.4, causal=False)
    for n in (1, 2, 3, 8):
        op, lp, o, l = oracle.splitkv_decode(q, k, v, n_splits=n, scale=0.4)
        assert np.max(np.abs(o - ref_o[:, :, 0])) <= 1e-13
        assert np.max(np.abs(l - ref_l[:, :, 0])) <= 1e-13
        Ls = L // n
        for p in range(n):
            o1, l1 = oracle.attention(q[:, :, None, :], k[:, :, p * Ls:(p + 1) * Ls],
                                      v[:, :, p * Ls:(p + 1) * Ls], scale=0.4, causal=False)
            assert np.max(np.abs(op[:, :, p] - o1[:, :, 0])) <= 1e-14
            assert np.max(np.abs(lp[:, :, p] - l1[:, :, 0])) <= 1e-14
