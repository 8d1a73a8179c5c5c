"""GPU parity of every C-ABI entry point against the fp64 oracle, element by element,
at sizes that span several tiles and ragged tails, plus the degenerate cases."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import CONFIGS, FP8_K_SCALE, FP8_V_SCALE, fp8_cache_torch, prefill_inputs_np, randn_np
from gpu_util import assert_close, np64, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype).contiguous()


TD = {"f32": torch.float32, "bf16": torch.bfloat16}


def ring_case(ra, *, dtype, B, Hq, Hkv, Sp, P, Dqk, Dv, causal, q_part0=0, nq=None, seed=0):
    nq = P if nq is None else nq
    say(f"ring_attn_fwd {dtype} B{B} Hq{Hq} Hkv{Hkv} Sp{Sp} P{P} D{Dqk}/{Dv} causal={causal} "
        f"parts {q_part0}..{q_part0 + nq - 1} seed {seed}")
    S = P * Sp
    q_all, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, Dqk, Dv, seed=seed, dtype=dtype)
    q = q_all[:, :, q_part0 * Sp:(q_part0 + nq) * Sp]
    scale = 1.0 / math.sqrt(Dqk)
    o, lse = ra.ring_attn_fwd(to_dev(q, TD[dtype]), to_dev(k, TD[dtype]), to_dev(v, TD[dtype]),
                              P=P, causal=causal, scale=scale, q_part0=q_part0)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, scale=scale, causal=causal, q_pos0=q_part0 * Sp, k_pos0=0)
    return assert_close(np64(o), np64(lse), o_ref, l_ref, dtype, "ring_attn_fwd")


# ------------------------------------------------------------------------------ fp32

def test_fp32_c1_all_rows(ra):
    c = CONFIGS["C1"]
    ring_case(ra, dtype="f32", B=c.B, Hq=c.Hq, Hkv=c.Hkv, Sp=c.Sp, P=c.P, Dqk=c.Dqk, Dv=c.Dv,
              causal=c.causal, seed=c.seed)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sp,P", [(37, 3), (100, 1), (65, 2)])
def test_fp32_ring_ragged(ra, dims, causal, Sp, P):
    ring_case(ra, dtype="f32", B=2, Hq=4, Hkv=2, Sp=Sp, P=P, Dqk=dims[0], Dv=dims[1], causal=causal,
              seed=11 + Sp + P)


# fp32 launches with at least 512 workgroups of 32 x 32 products (128 query rows, 64
# at D_qk = D_v = 64) use that shape; smaller ones (the cases above) take 16 x 16
# products in workgroups of 32 or 16 rows. These have ragged row and key tiles.

def f32_wide(B, Hq, rows, nparts, Dqk, Dv):
    """Whether an fp32 launch takes the 32 x 32 product shape."""
    bq = 64 if Dqk + Dv <= 128 else 128
    return B * Hq * nparts * ((rows + bq - 1) // bq) >= 512


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (64, 128), (128, 64)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_fp32_ring_large_grid_ragged(ra, dims, causal, layout):
    B, Hq, Hkv, Sp, P = (2, 8, 2, 1040, 2) if dims == (64, 64) else (2, 16, 4, 1040, 2)
    assert f32_wide(B, Hq, Sp, P, *dims)
    case = ring_case if layout == "contiguous" else striped_case
    case(ra, dtype="f32", B=B, Hq=Hq, Hkv=Hkv, Sp=Sp, P=P, Dqk=dims[0], Dv=dims[1], causal=causal,
         seed=171 + dims[0] + dims[1])


@pytest.mark.parametrize("dims", [(64, 64), (128, 128)])
@pytest.mark.parametrize("Sq", [1040, 520, 40])
def test_fp32_step_chain_three_grid_sizes(ra, dims, Sq):
    """Two causal block steps from the empty state, queries after both blocks: the
    32 x 32 product shape at 1040 rows, then the 16 x 16 one over more and fewer
    workgroups than the chip holds at once."""
    Dqk, Dv = dims
    B, Hq, Hkv, Sk = 2, 16 if Dqk == 64 else 32, 4, 300
    assert f32_wide(B, Hq, Sq, 1, Dqk, Dv) == (Sq == 1040)
    q, k, v = prefill_inputs_np(B, Hq, Hkv, Sq, 2 * Sk, Dqk, Dv, seed=181 + Sq, dtype="f32")
    q_pos0 = 2 * Sk - 20
    tq, tk, tv = (to_dev(x, torch.float32) for x in (q, k, v))
    o_acc, l_acc = ra.init_state(tq, Dv)
    for j in (1, 0):
        ra.block_attn_step(tq, tk[:, :, j * Sk:(j + 1) * Sk].contiguous(), tv[:, :, j * Sk:(j + 1) * Sk].contiguous(),
                           o_acc, l_acc, q_pos0=q_pos0, k_pos0=j * Sk, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, scale=1 / math.sqrt(Dqk), causal=True, q_pos0=q_pos0, k_pos0=0)
    assert_close(np64(o_acc), np64(l_acc), o_ref, l_ref, "f32", f"fp32 step chain Sq {Sq}")


# ------------------------------------------------------------------------------ bf16

@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sp,P", [(300, 3), (513, 1), (256, 2)])
def test_bf16_ring_ragged(ra, dims, causal, Sp, P):
    ring_case(ra, dtype="bf16", B=2, Hq=4, Hkv=2, Sp=Sp, P=P, Dqk=dims[0], Dv=dims[1], causal=causal,
              seed=21 + Sp + P)


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
def test_bf16_one_partition_share(ra, dims):
    """One device's share: only the last query partition, all KV blocks (the shape of
    the MLA-like configuration, scaled down)."""
    ring_case(ra, dtype="bf16", B=1, Hq=4, Hkv=4, Sp=700, P=4, Dqk=dims[0], Dv=dims[1], causal=True,
              q_part0=3, nq=1, seed=5)


def test_bf16_gqa_group8(ra):
    ring_case(ra, dtype="bf16", B=1, Hq=16, Hkv=2, Sp=384, P=4, Dqk=128, Dv=128, causal=True, seed=8)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_bf16_gqa_group3(ra, dims, layout):
    """Three query heads per KV head (not a power of two), two sequences."""
    case = ring_case if layout == "contiguous" else striped_case
    case(ra, dtype="bf16", B=2, Hq=6, Hkv=2, Sp=200, P=3, Dqk=dims[0], Dv=dims[1], causal=True, seed=61 + dims[0])


def test_fp32_gqa_group3(ra):
    ring_case(ra, dtype="f32", B=2, Hq=6, Hkv=2, Sp=70, P=3, Dqk=64, Dv=64, causal=True, seed=66)


def test_single_token_partitions(ra):
    ring_case(ra, dtype="bf16", B=1, Hq=2, Hkv=1, Sp=1, P=5, Dqk=128, Dv=128, causal=True, seed=9)
    ring_case(ra, dtype="f32", B=1, Hq=2, Hkv=1, Sp=1, P=5, Dqk=64, Dv=64, causal=True, seed=9)


def test_c2_all_rows(ra):
    c = CONFIGS["C2"]
    ring_case(ra, dtype="bf16", B=c.B, Hq=c.Hq, Hkv=c.Hkv, Sp=c.Sp, P=c.P, Dqk=c.Dqk, Dv=c.Dv,
              causal=c.causal, seed=c.seed)


def test_deterministic(ra):
    q, k, v = (to_dev(x, torch.bfloat16) for x in prefill_inputs_np(1, 8, 2, 2048, 2048, 128, 128, seed=3,
                                                                       dtype="bf16"))
    o1, l1 = ra.ring_attn_fwd(q, k, v, P=4, causal=True)
    o2, l2 = ra.ring_attn_fwd(q, k, v, P=4, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_gqa_equals_repeated_kv_heads(ra):
    q, k, v = (to_dev(x, torch.bfloat16) for x in prefill_inputs_np(1, 8, 2, 1024, 1024, 128, 128, seed=4,
                                                                       dtype="bf16"))
    o1, l1 = ra.ring_attn_fwd(q, k, v, P=2, causal=True)
    o2, l2 = ra.ring_attn_fwd(q, k.repeat_interleave(4, dim=1).contiguous(),
                              v.repeat_interleave(4, dim=1).contiguous(), P=2, causal=True)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_one_partition_ring_equals_plain_and_split(ra):
    """A ring of one partition is plain attention; cutting the same sequence into 4
    partitions must reach the same result within rounding."""
    q, k, v = prefill_inputs_np(1, 4, 4, 1536, 1536, 128, 128, seed=6, dtype="bf16")
    dq, dk, dv = (to_dev(x, torch.bfloat16) for x in (q, k, v))
    o1, l1 = ra.ring_attn_fwd(dq, dk, dv, P=1, causal=True)
    o4, l4 = ra.ring_attn_fwd(dq, dk, dv, P=4, causal=True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.attention(q, k, v, scale=1 / math.sqrt(128), causal=True)
    assert_close(np64(o1), np64(l1), o_ref, l_ref, "bf16", "P=1")
    assert_close(np64(o4), np64(l4), o_ref, l_ref, "bf16", "P=4")
    assert float((o1.float() - o4.float()).abs().max()) <= 2e-2


# ------------------------------------------------------------------------------ one-stream launches
# A launch of fewer 256-row workgroups than two rounds of the 256 CUs splits every
# workgroup's key range over two wave streams (128 rows each); larger launches run
# one stream per 256-row workgroup. The cases above are small, so they take the
# two-stream path; these have enough heads and rows for one stream, with ragged
# query and key tiles.

ONE_STREAM_ITEMS = 2 * 256


def one_stream_items(B, Hq, rows, nparts=1):
    return B * Hq * nparts * ((rows + 255) // 256)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("layout", ["contiguous", "striped"])
def test_bf16_ring_one_stream_ragged(ra, dims, causal, layout):
    B, Hq, Hkv, Sp, P = 1, 128, 16, 300, 2
    assert one_stream_items(B, Hq, Sp, P) >= ONE_STREAM_ITEMS
    case = ring_case if layout == "contiguous" else striped_case
    case(ra, dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, Sp=Sp, P=P, Dqk=dims[0], Dv=dims[1], causal=causal,
         seed=131 + dims[0])


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
def test_bf16_ring_one_stream_batch2(ra, dims):
    """Two sequences, GQA 8:1, in a launch that runs one key stream per workgroup."""
    B, Hq, Hkv, Sp, P = 2, 64, 8, 300, 2
    assert one_stream_items(B, Hq, Sp, P) >= ONE_STREAM_ITEMS
    ring_case(ra, dtype="bf16", B=B, Hq=Hq, Hkv=Hkv, Sp=Sp, P=P, Dqk=dims[0], Dv=dims[1], causal=True,
              seed=151 + dims[0])


@pytest.mark.parametrize("dims", [(128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
def test_bf16_step_chain_one_stream(ra, dims, causal):
    """Block steps over partitions of 769 rows (three full tiles and one row), from
    the empty state and then carrying it."""
    B, Hq, Hkv, Sp, P = 1, 128, 16, 769, 2
    assert one_stream_items(B, Hq, Sp) >= ONE_STREAM_ITEMS
    Dqk, Dv = dims
    S = Sp * P
    say(f"block_attn_step chain, one stream, D{Dqk}/{Dv} causal={causal}")
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, Dqk, Dv, seed=141 + Dqk, dtype="bf16")
    dq, dk, dv = (to_dev(x, torch.bfloat16) for x in (q, k, v))
    o_ref, l_ref = oracle.attention(q, k, v, scale=1 / math.sqrt(Dqk), causal=causal)
    for i in range(P):
        qi = dq[:, :, i * Sp:(i + 1) * Sp].contiguous()
        o_acc, l_acc = ra.init_state(qi, Dv)
        for j, kind in ra.ring_schedule(P, i, causal):
            if kind == "skip":
                continue
            ra.block_attn_step(qi, dk[:, :, j * Sp:(j + 1) * Sp].contiguous(), dv[:, :, j * Sp:(j + 1) * Sp].contiguous(),
                               o_acc, l_acc, q_pos0=i * Sp, k_pos0=j * Sp, causal=causal)
        torch.cuda.synchronize()
        sl = slice(i * Sp, (i + 1) * Sp)
        assert_close(np64(o_acc), np64(l_acc), o_ref[:, :, sl], l_ref[:, :, sl], "bf16", f"one-stream chain part {i}")


# ------------------------------------------------------------------------------ striped layout

def striped(x, P):
    """[B, H, S, D] in natural token order -> partition-major striped order: the
    rows of partition p are tokens p, p+P, p+2P, ..."""
    return np.concatenate([x[:, :, p::P] for p in range(P)], axis=2)


def striped_case(ra, *, dtype, B, Hq, Hkv, Sp, P, Dqk, Dv, causal, q_part0=0, nq=None, seed=0):
    """Striped ring on the GPU against one-shot attention over the sequence in
    natural order (the oracle's plain definition), taken at the striped rows."""
    nq = P if nq is None else nq
    say(f"ring_attn_fwd_striped {dtype} B{B} Hq{Hq} Hkv{Hkv} Sp{Sp} P{P} D{Dqk}/{Dv} causal={causal} "
        f"parts {q_part0}..{q_part0 + nq - 1} seed {seed}")
    S = P * Sp
    q_nat, k_nat, v_nat = prefill_inputs_np(B, Hq, Hkv, S, S, Dqk, Dv, seed=seed, dtype=dtype)
    q_st, k_st, v_st = striped(q_nat, P), striped(k_nat, P), striped(v_nat, P)
    q = q_st[:, :, q_part0 * Sp:(q_part0 + nq) * Sp]
    scale = 1.0 / math.sqrt(Dqk)
    o, lse = ra.ring_attn_fwd(to_dev(q, TD[dtype]), to_dev(k_st, TD[dtype]), to_dev(v_st, TD[dtype]),
                              P=P, causal=causal, scale=scale, q_part0=q_part0, layout="striped")
    torch.cuda.synchronize()
    o_nat, l_nat = oracle.attention(q_nat, k_nat, v_nat, scale=scale, causal=causal)
    o_ref = striped(o_nat, P)[:, :, q_part0 * Sp:(q_part0 + nq) * Sp]
    l_ref = striped(l_nat[..., None], P)[..., 0][:, :, q_part0 * Sp:(q_part0 + nq) * Sp]
    return assert_close(np64(o), np64(lse), o_ref, l_ref, dtype, "ring_attn_fwd_striped")


@pytest.mark.parametrize("dims", [(64, 64), (128, 128), (192, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sp,P", [(300, 3), (129, 4), (256, 2), (1, 5)])
def test_bf16_striped_ring(ra, dims, causal, Sp, P):
    striped_case(ra, dtype="bf16", B=2, Hq=4, Hkv=2, Sp=Sp, P=P, Dqk=dims[0], Dv=dims[1], causal=causal,
                 seed=71 + Sp + P)


@pytest.mark.parametrize("dims", [(64, 64), (128, 128)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Sp,P", [(37, 3), (65, 2)])
def test_fp32_striped_ring(ra, dims, causal, Sp, P):
    striped_case(ra, dtype="f32", B=2, Hq=4, Hkv=2, Sp=Sp, P=P, Dqk=dims[0], Dv=dims[1], causal=causal,
                 seed=81 + Sp + P)


def test_bf16_striped_one_partition_share(ra):
    """One device's share of a striped ring (the last partition, all KV blocks),
    GQA 8:1 -- the shape of one rank's work, scaled down."""
    striped_case(ra, dtype="bf16", B=1, Hq=16, Hkv=2, Sp=384, P=8, Dqk=128, Dv=128, causal=True,
                 q_part0=7, nq=1, seed=91)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_striped_ring_equals_step_chain_with_virtual_positions(ra, dtype):
    """The striped causal mask is k_pos <= q_pos on virtual positions (query: local
    row; key: local index + [j > i]), so P block steps with q_pos0 = 0 and
    k_pos0 = [j > i] reproduce the striped ring."""
    B, Hq, Hkv, Sp, P = 1, 4, 2, 150, 4
    D = 128
    S = Sp * P
    say(f"striped ring vs step chain {dtype}")
    q_nat, k_nat, v_nat = prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=93, dtype=dtype)
    dq, dk, dv = (to_dev(striped(x, P), TD[dtype]) for x in (q_nat, k_nat, v_nat))
    o_ring, l_ring = ra.ring_attn_fwd(dq, dk, dv, P=P, causal=True, layout="striped")
    for i in range(P):
        qi = dq[:, :, i * Sp:(i + 1) * Sp].contiguous()
        o_acc, l_acc = ra.init_state(qi, D)
        for j, kind in ra.ring_schedule(P, i, True, "striped"):
            assert kind == "diag"
            ra.block_attn_step(qi, dk[:, :, j * Sp:(j + 1) * Sp].contiguous(), dv[:, :, j * Sp:(j + 1) * Sp].contiguous(),
                               o_acc, l_acc, q_pos0=0, k_pos0=1 if j > i else 0, causal=True)
        torch.cuda.synchronize()
        sl = slice(i * Sp, (i + 1) * Sp)
        tol_o, tol_l = (2e-2, 1e-2) if dtype == "bf16" else (1e-4, 1e-4)
        assert float((o_acc - o_ring[:, :, sl].float()).abs().max()) <= tol_o
        assert float((l_acc - l_ring[:, :, sl]).abs().max()) <= tol_l


# ------------------------------------------------------------------------------ step API

@pytest.mark.parametrize("dtype,dims", [("bf16", (128, 128)), ("bf16", (192, 128)), ("f32", (64, 64))])
@pytest.mark.parametrize("causal", [False, True])
def test_step_chain_equals_ring_and_oracle(ra, dtype, dims, causal):
    """P chained block steps in ring order give the ring result and the oracle's."""
    B, Hq, Hkv, Sp, P = 1, 4, 2, 200, 4
    Dqk, Dv = dims
    S = Sp * P
    say(f"block_attn_step chain {dtype} D{Dqk}/{Dv} causal={causal}")
    q, k, v = prefill_inputs_np(B, Hq, Hkv, S, S, Dqk, Dv, seed=31, dtype=dtype)
    dq, dk, dv = (to_dev(x, TD[dtype]) for x in (q, k, v))
    o_ring, l_ring = ra.ring_attn_fwd(dq, dk, dv, P=P, causal=causal)
    o_ref, l_ref = oracle.attention(q, k, v, scale=1 / math.sqrt(Dqk), causal=causal)
    for i in range(P):
        qi = dq[:, :, i * Sp:(i + 1) * Sp].contiguous()
        o_acc, l_acc = ra.init_state(qi, Dv)
        for j, kind in ra.ring_schedule(P, i, causal):
            if kind == "skip":
                continue
            ra.block_attn_step(qi, dk[:, :, j * Sp:(j + 1) * Sp].contiguous(), dv[:, :, j * Sp:(j + 1) * Sp].contiguous(),
                               o_acc, l_acc, q_pos0=i * Sp, k_pos0=j * Sp, causal=causal)
        torch.cuda.synchronize()
        sl = slice(i * Sp, (i + 1) * Sp)
        assert_close(np64(o_acc), np64(l_acc), o_ref[:, :, sl], l_ref[:, :, sl], dtype, f"chain part {i}")
        tol = 2e-2 if dtype == "bf16" else 1e-4
        assert float((o_acc - o_ring[:, :, sl].float()).abs().max()) <= tol
        assert float((l_acc - l_ring[:, :, sl]).abs().max()) <= (1e-2 if dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_step_fully_masked_block_is_a_noop(ra, dtype):
    B, Hq, Sq, Sk, D = 1, 2, 100, 64, 64 if dtype == "f32" else 128
    q, k, v = prefill_inputs_np(B, Hq, Hq, Sq, Sk, D, D, seed=41, dtype=dtype)
    dq, dk, dv = (to_dev(x, TD[dtype]) for x in (q, k, v))
    o_acc = to_dev(randn_np((B, Hq, Sq, D), 42), torch.float32)
    l_acc = to_dev(randn_np((B, Hq, Sq), 43), torch.float32)
    o0, l0 = o_acc.clone(), l_acc.clone()
    ra.block_attn_step(dq, dk, dv, o_acc, l_acc, q_pos0=0, k_pos0=Sq, causal=True)   # keys all in the future
    torch.cuda.synchronize()
    assert torch.equal(o_acc, o0) and torch.equal(l_acc, l0)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 128), ("bf16", 64)])
def test_step_partial_overlap_positions(ra, dtype, D):
    """Arbitrary query/key positions: the block's keys straddle the queries, so the
    mask cuts through tiles; the incoming state is a genuine partial result."""
    B, Hq, Hkv, Sq, Sk = 2, 4, 1, 177, 150
    q_pos0, k_pos0 = 100, 37
    q, k, v = prefill_inputs_np(B, Hq, Hkv, Sq, Sk, D, D, seed=51, dtype=dtype)
    k0, v0 = randn_np((B, Hkv, 30, D), 52, dtype), randn_np((B, Hkv, 30, D), 53, dtype)
    o_a, l_a = oracle.attention(q, k0, v0, scale=1 / math.sqrt(D), causal=True, q_pos0=q_pos0, k_pos0=0)
    o_b, l_b = oracle.attention(q, k, v, scale=1 / math.sqrt(D), causal=True, q_pos0=q_pos0, k_pos0=k_pos0)
    o_ref, l_ref = oracle.merge(o_a, l_a, o_b, l_b)
    o_acc = to_dev(o_a.astype(np.float32), torch.float32)
    l_acc = to_dev(l_a.astype(np.float32), torch.float32)
    ra.block_attn_step(to_dev(q, TD[dtype]), to_dev(k, TD[dtype]), to_dev(v, TD[dtype]), o_acc, l_acc,
                       q_pos0=q_pos0, k_pos0=k_pos0, causal=True)
    torch.cuda.synchronize()
    assert_close(np64(o_acc), np64(l_acc), o_ref, l_ref, dtype, "step partial")


# ------------------------------------------------------------------------------ merges

@pytest.mark.parametrize("alias", [False, True])
def test_lse_merge(ra, alias):
    rows, Dv = 3001, 128
    rng = np.random.default_rng(61)
    o_a = rng.standard_normal((rows, Dv)).astype(np.float32)
    o_b = rng.standard_normal((rows, Dv)).astype(np.float32)
    l_a = (rng.standard_normal(rows) * 30).astype(np.float32)
    l_b = (rng.standard_normal(rows) * 30).astype(np.float32)
    l_a[::7] = -np.inf
    l_b[::11] = -np.inf
    o_a[::7] = 0
    o_b[::11] = 0
    o_ref, l_ref = oracle.merge(o_a, l_a, o_b, l_b)
    da, dla, db, dlb = (to_dev(x, torch.float32) for x in (o_a, l_a, o_b, l_b))
    if alias:
        o, l = ra.lse_merge(da, dla, db, dlb, out=da, lse_out=dla)
        assert o.data_ptr() == da.data_ptr()
    else:
        o, l = ra.lse_merge(da, dla, db, dlb)
    torch.cuda.synchronize()
    assert_close(np64(o), np64(l), o_ref, l_ref, "f32", "lse_merge")


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_lse_merge_n(ra, out_dtype):
    rows, n, Dv = 517, 8, 128
    rng = np.random.default_rng(62)
    op = rng.standard_normal((rows, n, Dv)).astype(np.float32)
    lp = (rng.standard_normal((rows, n)) * 5).astype(np.float32)
    lp[::5, 3] = -np.inf
    lp[7, :] = -np.inf
    op[7] = 0
    o_ref, l_ref = oracle.merge_n(op, lp)
    o, l = ra.lse_merge_n(to_dev(op, torch.float32), to_dev(lp, torch.float32), out_dtype=out_dtype)
    torch.cuda.synchronize()
    assert_close(np64(o), np64(l), o_ref, l_ref, "f32" if out_dtype == torch.float32 else "bf16", "merge_n")


# ------------------------------------------------------------------------------ decode

@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (8, 8), (12, 3)])
@pytest.mark.parametrize("L,n", [(768, 1), (768, 3), (768, 8), (1000, 8)])
def test_splitkv_decode_small(ra, D, Hq, Hkv, L, n):
    B = 2
    say(f"splitkv_decode B{B} Hq{Hq} Hkv{Hkv} L{L} n{n} D{D}")
    q = randn_np((B, Hq, D), 71, "bf16")
    k = randn_np((B, Hkv, L, D), 72, "bf16")
    v = randn_np((B, Hkv, L, D), 73, "bf16")
    op, lp, o, l = ra.splitkv_decode(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16),
                                     to_dev(v, torch.bfloat16), n_splits=n)
    torch.cuda.synchronize()
    op_r, lp_r, o_r, l_r = oracle.splitkv_decode(q, k, v, n_splits=n, scale=1 / math.sqrt(D))
    assert_close(np64(op), np64(lp), op_r, lp_r, "bf16", "decode partials")
    assert_close(np64(o), np64(l), o_r, l_r, "bf16", "decode merged")


# ------------------------------------------------------------------------------ fp8 KV decode

def fp8_codes(t):
    return t.view(torch.uint8).cpu().numpy()


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("Hq,Hkv", [(16, 2), (8, 8), (12, 3)])
@pytest.mark.parametrize("L,n", [(768, 1), (768, 3), (1000, 8)])
def test_splitkv_decode_fp8_small(ra, D, Hq, Hkv, L, n):
    """FP8 e4m3 cache with per-tensor scales against the oracle's decode of the
    dequantised values (the oracle decodes the stored codes itself)."""
    B = 2
    say(f"splitkv_decode_fp8 B{B} Hq{Hq} Hkv{Hkv} L{L} n{n} D{D}")
    q = randn_np((B, Hq, D), 171, "bf16")
    kc = fp8_cache_torch((B, Hkv, L, D), 172, DEV)
    vc = fp8_cache_torch((B, Hkv, L, D), 173, DEV)
    op, lp, o, l = ra.splitkv_decode_fp8(to_dev(q, torch.bfloat16), kc, vc, k_scale=FP8_K_SCALE,
                                         v_scale=FP8_V_SCALE, n_splits=n)
    torch.cuda.synchronize()
    k = oracle.dequantize(fp8_codes(kc), FP8_K_SCALE)
    v = oracle.dequantize(fp8_codes(vc), FP8_V_SCALE)
    op_r, lp_r, o_r, l_r = oracle.splitkv_decode(q, k, v, n_splits=n, scale=1 / math.sqrt(D))
    assert_close(np64(op), np64(lp), op_r, lp_r, "bf16", "fp8 decode partials")
    assert_close(np64(o), np64(l), o_r, l_r, "bf16", "fp8 decode merged")
    op2, lp2 = ra.splitkv_partial_fp8(to_dev(q, torch.bfloat16), kc, vc, k_scale=FP8_K_SCALE,
                                      v_scale=FP8_V_SCALE, n_splits=n)
    torch.cuda.synchronize()
    assert torch.equal(op2, op) and torch.equal(lp2, lp)


@pytest.mark.parametrize("kv8", [False, True])
@pytest.mark.parametrize("D,Hq,Hkv,L,n", [
    (128, 32, 2, 40, 8),    # 16 heads per group, 5 keys per split: three waves see only masked keys
    (64, 16, 1, 33, 1),     # 16 heads per group, a last chunk of one key
    (128, 16, 1, 96, 3),    # one whole chunk per split
])
def test_splitkv_decode_edges(ra, kv8, D, Hq, Hkv, L, n):
    """The largest supported group and splits shorter than the four waves' chunks."""
    B = 2
    say(f"splitkv_decode edges kv8={kv8} B{B} Hq{Hq} Hkv{Hkv} L{L} n{n} D{D}")
    q = randn_np((B, Hq, D), 191, "bf16")
    if kv8:
        kc = fp8_cache_torch((B, Hkv, L, D), 192, DEV)
        vc = fp8_cache_torch((B, Hkv, L, D), 193, DEV)
        op, lp, o, l = ra.splitkv_decode_fp8(to_dev(q, torch.bfloat16), kc, vc, k_scale=FP8_K_SCALE,
                                             v_scale=FP8_V_SCALE, n_splits=n)
        k = oracle.dequantize(fp8_codes(kc), FP8_K_SCALE)
        v = oracle.dequantize(fp8_codes(vc), FP8_V_SCALE)
    else:
        k = randn_np((B, Hkv, L, D), 192, "bf16")
        v = randn_np((B, Hkv, L, D), 193, "bf16")
        op, lp, o, l = ra.splitkv_decode(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16),
                                         to_dev(v, torch.bfloat16), n_splits=n)
    torch.cuda.synchronize()
    op_r, lp_r, o_r, l_r = oracle.splitkv_decode(q, k, v, n_splits=n, scale=1 / math.sqrt(D))
    assert_close(np64(op), np64(lp), op_r, lp_r, "bf16", "decode partials")
    assert_close(np64(o), np64(l), o_r, l_r, "bf16", "decode merged")


def test_splitkv_decode_fp8_equals_bf16_path_on_the_widened_cache(ra):
    """The fp8 path widens codes exactly to bf16 and folds the scales into the
    score scale and the output: with scales 1 it reproduces the bf16 decode of the
    widened cache to fp32 rounding of the scale folding."""
    B, Hq, Hkv, L, D, n = 2, 8, 2, 2048, 128, 4
    say("splitkv_decode_fp8 vs bf16 path on the widened cache")
    q = to_dev(randn_np((B, Hq, D), 181, "bf16"), torch.bfloat16)
    kc = fp8_cache_torch((B, Hkv, L, D), 182, DEV)
    vc = fp8_cache_torch((B, Hkv, L, D), 183, DEV)
    op8, lp8, o8, l8 = ra.splitkv_decode_fp8(q, kc, vc, k_scale=1.0, v_scale=1.0, n_splits=n)
    op, lp, o, l = ra.splitkv_decode(q, kc.to(torch.bfloat16), vc.to(torch.bfloat16), n_splits=n)
    torch.cuda.synchronize()
    assert float((op8 - op).abs().max()) <= 1e-5 and float((lp8 - lp).abs().max()) <= 1e-5


# ------------------------------------------------------------------------------ streams

def test_calls_on_two_streams_match_the_default_stream(ra):
    """Every call runs on torch's current stream and keeps no state between calls:
    a ring prefill, a block step and a decode issued on two side streams at once
    (default priority) give bit-identical results to the same calls on the default
    stream."""
    q, k, v = (to_dev(x, torch.bfloat16) for x in prefill_inputs_np(1, 8, 2, 2048, 2048, 128, 128, seed=171,
                                                                       dtype="bf16"))
    dq_ = to_dev(randn_np((4, 16, 128), 172, "bf16"), torch.bfloat16)
    dk_ = to_dev(randn_np((4, 2, 3000, 128), 173, "bf16"), torch.bfloat16)
    dv_ = to_dev(randn_np((4, 2, 3000, 128), 174, "bf16"), torch.bfloat16)

    def work():
        o, lse = ra.ring_attn_fwd(q, k, v, P=4, causal=True)
        oa, la = ra.init_state(q[:, :, :512].contiguous(), 128)
        ra.block_attn_step(q[:, :, :512].contiguous(), k[:, :, 512:1024].contiguous(), v[:, :, 512:1024].contiguous(),
                           oa, la, q_pos0=1024, k_pos0=512, causal=True)
        _, _, od, ld = ra.splitkv_decode(dq_, dk_, dv_, n_splits=3)
        return o, lse, oa, la, od, ld

    ref = work()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    with torch.cuda.stream(s1):
        r1 = work()
    with torch.cuda.stream(s2):
        r2 = work()
    torch.cuda.synchronize()
    for a, b, c in zip(ref, r1, r2):
        assert torch.equal(a, b) and torch.equal(a, c)


def test_fp32_forward_on_two_side_streams(ra):
    """The fp32 ring prefill (32 x 32 products at 2 x 32 heads, and 16 x 16 ones on
    one head) and an fp32 block step on two side streams at once: bit-identical to
    the default stream."""
    q, k, v = (to_dev(x, torch.float32) for x in prefill_inputs_np(2, 32, 8, 1040, 1040, 128, 128, seed=175,
                                                                      dtype="f32"))
    assert f32_wide(2, 32, 520, 2, 128, 128) and not f32_wide(1, 2, 520, 2, 128, 128)

    def work():
        o, lse = ra.ring_attn_fwd(q, k, v, P=2, causal=True)
        o1, l1 = ra.ring_attn_fwd(q[:1, :2].contiguous(), k[:1, :1].contiguous(), v[:1, :1].contiguous(), P=2,
                                  causal=True)
        oa, la = ra.init_state(q[:, :, :520].contiguous(), 128)
        ra.block_attn_step(q[:, :, :520].contiguous(), k[:, :, 300:800].contiguous(), v[:, :, 300:800].contiguous(),
                           oa, la, q_pos0=520, k_pos0=300, causal=True)
        return o, lse, o1, l1, oa, la

    ref = work()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        r1 = work()
    with torch.cuda.stream(s2):
        r2 = work()
    torch.cuda.synchronize()
    for a, b, c in zip(ref, r1, r2):
        assert torch.equal(a, b) and torch.equal(a, c)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_backward_on_two_side_streams(ra, dtype):
    """The backward entry points issued on two side streams at once give results
    bit-identical to the same calls on the default stream (bf16 and fp32)."""
    B, Hq, Hkv, S, D = 1, 8, 2, 1000, 128
    q, k, v = (to_dev(x, dtype) for x in prefill_inputs_np(B, Hq, Hkv, S, S, D, D, seed=177, dtype="f32"))
    dout = to_dev(randn_np((B, Hq, S, D), 178, "f32"), dtype)
    o, lse = ra.ring_attn_fwd(q, k, v, P=2, causal=True)
    torch.cuda.synchronize()

    def work():
        return ra.attn_bwd(q, k, v, o, lse, dout, causal=True)

    ref = work()
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s1):
        r1 = work()
    with torch.cuda.stream(s2):
        r2 = work()
    torch.cuda.synchronize()
    for a, b, c in zip(ref, r1, r2):
        assert torch.equal(a, b) and torch.equal(a, c)
