"""GPU parity on seeded random shapes: every entry point against the oracle on
cases drawn from one fixed seed, so that odd combinations of sizes, positions,
group sizes, head dims and masks that the hand-picked cases miss are covered too.
The draw is deterministic (the same cases on every run); each case prints its
parameters before it runs.

Sizes stay small enough for the fp64 oracle (at most a few hundred rows and keys
per block). Gates are those of the other parity tests (gpu_util.TOL for forward
and decode, the backward gates of tests/test_gpu_backward.py and, for fp32 inputs,
tests/test_gpu_backward_f32.py)."""
import math

import numpy as np
import pytest
import torch

import oracle
from workloads import prefill_inputs_np, randn_np
from gpu_util import assert_close, np64, say

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TD = {"f32": torch.float32, "bf16": torch.bfloat16}
DIMS = {"bf16": [(64, 64), (128, 128), (192, 128)], "f32": [(64, 64), (128, 128), (64, 128), (128, 64)]}


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as m
    m.load_library()
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    return m


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dtype).contiguous()


def heads(g):
    hkv = int(g.integers(1, 4))
    group = int(g.choice([1, 2, 3, 4, 8]))
    return hkv * group, hkv


def step_cases(n, seed=2024):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dt = str(g.choice(["bf16", "bf16", "f32"]))
        dims = DIMS[dt][int(g.integers(len(DIMS[dt])))]
        hq, hkv = heads(g)
        out.append(dict(dt=dt, dims=dims, B=int(g.integers(1, 3)), Hq=hq, Hkv=hkv, Sq=int(g.integers(1, 500)),
                        Sk=int(g.integers(1, 500)), q_pos0=int(g.integers(0, 900)), k_pos0=int(g.integers(0, 900)),
                        causal=bool(g.integers(2)), prior=int(g.integers(0, 300)) if g.random() < 0.5 else 0,
                        seed=int(g.integers(1 << 30))))
    return out


def ring_cases(n, seed=2025):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dt = str(g.choice(["bf16", "bf16", "f32"]))
        dims = DIMS[dt][int(g.integers(len(DIMS[dt])))]
        hq, hkv = heads(g)
        P = int(g.integers(1, 7))
        q_part0 = int(g.integers(0, P))
        out.append(dict(dt=dt, dims=dims, B=int(g.integers(1, 3)), Hq=hq, Hkv=hkv, Sp=int(g.integers(1, 300)), P=P,
                        q_part0=q_part0, nq=int(g.integers(1, P - q_part0 + 1)), causal=bool(g.integers(2)),
                        layout=str(g.choice(["contiguous", "striped"])), seed=int(g.integers(1 << 30))))
    return out


def decode_cases(n, seed=2026):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        hkv = int(g.integers(1, 4))
        group = int(g.choice([1, 2, 3, 5, 8, 16]))
        ns = int(g.integers(1, 9))
        out.append(dict(D=int(g.choice([64, 128])), B=int(g.integers(1, 4)), Hq=hkv * group, Hkv=hkv,
                        L=ns * int(g.integers(1, 400)), n=ns, fp8=bool(g.integers(2)), seed=int(g.integers(1 << 30))))
    return out


def bwd_cases(n, seed=2027, dt="bf16"):
    g = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        dims = DIMS[dt][int(g.integers(len(DIMS[dt])))]
        hq, hkv = heads(g)
        out.append(dict(dt=dt, dims=dims, B=int(g.integers(1, 3)), Hq=hq, Hkv=hkv, Sq=int(g.integers(1, 400)),
                        Sk=int(g.integers(1, 400)), q_pos0=int(g.integers(0, 600)), k_pos0=int(g.integers(0, 600)),
                        causal=bool(g.integers(2)), seed=int(g.integers(1 << 30))))
    return out


STEP = step_cases(40)
RING = ring_cases(30)
DECODE = decode_cases(20)
BWD = bwd_cases(20) + bwd_cases(12, seed=2028, dt="f32")


@pytest.mark.parametrize("c", STEP, ids=[f"step{i}" for i in range(len(STEP))])
def test_random_block_step(ra, c):
    """block_attn_step on a random block, from the empty state or from a genuine
    partial state (an earlier block of `prior` keys), against the oracle's merge."""
    say(f"block_attn_step {c}")
    Dqk, Dv = c["dims"]
    scale = 1 / math.sqrt(Dqk)
    q, k, v = prefill_inputs_np(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"], Dqk, Dv, seed=c["seed"], dtype=c["dt"])
    o_ref, l_ref = oracle.attention(q, k, v, scale=scale, causal=c["causal"], q_pos0=c["q_pos0"], k_pos0=c["k_pos0"])
    qd = to_dev(q, TD[c["dt"]])
    if c["prior"]:
        _, k0, v0 = prefill_inputs_np(c["B"], c["Hq"], c["Hkv"], 1, c["prior"], Dqk, Dv, seed=c["seed"] + 1,
                                      dtype=c["dt"])
        k0_pos = max(0, c["k_pos0"] - c["prior"])
        o0, l0 = oracle.attention(q, k0, v0, scale=scale, causal=c["causal"], q_pos0=c["q_pos0"], k_pos0=k0_pos)
        o_ref, l_ref = oracle.merge(o0, l0, o_ref, l_ref)
        o_acc = to_dev(o0, torch.float32)
        l_acc = to_dev(l0, torch.float32)
    else:
        o_acc, l_acc = ra.init_state(qd, Dv)
    ra.block_attn_step(qd, to_dev(k, TD[c["dt"]]), to_dev(v, TD[c["dt"]]), o_acc, l_acc, q_pos0=c["q_pos0"],
                       k_pos0=c["k_pos0"], causal=c["causal"], scale=scale)
    torch.cuda.synchronize()
    assert_close(np64(o_acc), np64(l_acc), o_ref, l_ref, c["dt"], "step")


@pytest.mark.parametrize("c", RING, ids=[f"ring{i}" for i in range(len(RING))])
def test_random_ring(ra, c):
    """ring_attn_fwd (contiguous or striped) over random partitions against one-shot
    attention at the tokens' global positions."""
    say(f"ring_attn_fwd {c}")
    Dqk, Dv = c["dims"]
    Sp, P = c["Sp"], c["P"]
    S = Sp * P
    scale = 1 / math.sqrt(Dqk)
    q, k, v = prefill_inputs_np(c["B"], c["Hq"], c["Hkv"], S, S, Dqk, Dv, seed=c["seed"], dtype=c["dt"])
    rows = slice(c["q_part0"] * Sp, (c["q_part0"] + c["nq"]) * Sp)
    o, lse = ra.ring_attn_fwd(to_dev(q[:, :, rows], TD[c["dt"]]), to_dev(k, TD[c["dt"]]), to_dev(v, TD[c["dt"]]),
                              P=P, causal=c["causal"], scale=scale, q_part0=c["q_part0"], layout=c["layout"])
    torch.cuda.synchronize()
    # row r of the stored arrays is global token pos[r]
    pos = np.concatenate([oracle.partition_positions(P, Sp, p, c["layout"]) for p in range(P)])
    o_ref, l_ref = oracle.attention(q, k, v, scale=scale, causal=c["causal"], q_pos=pos, k_pos=pos)
    assert_close(np64(o), np64(lse), o_ref[:, :, rows], l_ref[:, :, rows], c["dt"], "ring")


@pytest.mark.parametrize("c", DECODE, ids=[f"decode{i}" for i in range(len(DECODE))])
def test_random_decode(ra, c):
    """splitkv_decode over a bf16 or fp8 cache: every partial and the merge."""
    say(f"splitkv_decode {c}")
    D, B, Hq, Hkv, L, n = c["D"], c["B"], c["Hq"], c["Hkv"], c["L"], c["n"]
    scale = 1 / math.sqrt(D)
    q = randn_np((B, Hq, D), c["seed"], "bf16")
    k = randn_np((B, Hkv, L, D), c["seed"] + 1, "bf16")
    v = randn_np((B, Hkv, L, D), c["seed"] + 2, "bf16")
    if c["fp8"]:
        k8 = to_dev(k, torch.float32).to(torch.float8_e4m3fn)
        v8 = to_dev(v, torch.float32).to(torch.float8_e4m3fn)
        op, lp, o, lse = ra.splitkv_decode_fp8(to_dev(q, torch.bfloat16), k8, v8, k_scale=1.0, v_scale=1.0,
                                               n_splits=n, scale=scale)
        k = k8.float().cpu().numpy().astype(np.float64)       # the values the kernel sees
        v = v8.float().cpu().numpy().astype(np.float64)
    else:
        op, lp, o, lse = ra.splitkv_decode(to_dev(q, torch.bfloat16), to_dev(k, torch.bfloat16),
                                           to_dev(v, torch.bfloat16), n_splits=n, scale=scale)
    torch.cuda.synchronize()
    op_r, lp_r, o_r, l_r = oracle.splitkv_decode(q, k, v, n_splits=n, scale=scale)
    assert_close(np64(op), np64(lp), op_r, lp_r, "bf16", "partials")   # fp32 partials of bf16 inputs
    assert_close(np64(o), np64(lse), o_r, l_r, "bf16", "merged")


# (max error / max |ref|, mean error / mean |ref|, absolute floors): the bf16 gates of
# tests/test_gpu_backward.py and the fp32 gates of tests/test_gpu_backward_f32.py
BWD_TOL = {"bf16": (2e-2, 5e-3, 1e-6, 1e-7), "f32": (1e-4, 1e-5, 1e-5, 1e-6)}


def bwd_close(got, ref, what, dt):
    rmax, rmean, amax, amean = BWD_TOL[dt]
    got = np64(got)
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    top = float(np.max(np.abs(ref))) if ref.size else 0.0
    err = np.abs(got - ref)
    assert err.max(initial=0.0) <= rmax * top + amax, (what, float(err.max(initial=0.0)), top)
    assert err.mean() <= rmean * np.abs(ref).mean() + amean, (what, float(err.mean()))


@pytest.mark.parametrize("c", BWD, ids=[f"bwd{i}" for i in range(len(BWD))])
def test_random_backward_step(ra, c):
    """block_attn_bwd_step on a random pair, with the queries' full-row LSE and delta
    taken from a longer key range (the block plus 7 keys after it)."""
    say(f"block_attn_bwd_step {c}")
    D, Dv = c["dims"]
    B, Hq, Hkv, Sq, Sk = c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sk"]
    scale = 1 / math.sqrt(D)
    dt = c["dt"]
    q, k, v = prefill_inputs_np(B, Hq, Hkv, Sq, Sk, D, Dv, seed=c["seed"], dtype=dt)
    do = randn_np((B, Hq, Sq, Dv), c["seed"] + 3, dt)
    # 7 more keys of their own after the block. (Copies of the block's keys would,
    # for a one-key block, make every visible key of a row identical: then dS is
    # exactly zero and the kernels' rounding has nothing to be relative to.)
    kx = randn_np((B, Hkv, 7, D), c["seed"] + 4, dt)
    vx = randn_np((B, Hkv, 7, Dv), c["seed"] + 5, dt)
    kf, vf = np.concatenate([k, kx], axis=2), np.concatenate([v, vx], axis=2)
    kpos = np.concatenate([c["k_pos0"] + np.arange(Sk), c["k_pos0"] + Sk + np.arange(7)])
    _, _, _, lse, delta = oracle.attention_bwd(q, kf, vf, do, scale=scale, causal=c["causal"], q_pos0=c["q_pos0"],
                                               k_pos=kpos)
    gq, gk, gv = oracle.block_bwd(q, k, v, do, lse, delta, scale=scale, causal=c["causal"], q_pos0=c["q_pos0"],
                                  k_pos0=c["k_pos0"])
    dq = torch.zeros((B, Hq, Sq, D), dtype=torch.float32, device=DEV)
    dk = torch.zeros((B, Hkv, Sk, D), dtype=torch.float32, device=DEV)
    dv = torch.zeros((B, Hkv, Sk, Dv), dtype=torch.float32, device=DEV)
    ra.block_attn_bwd_step(to_dev(q, TD[dt]), to_dev(do, TD[dt]),
                           to_dev(np.where(np.isfinite(lse), lse, -np.inf), torch.float32),
                           to_dev(delta, torch.float32), to_dev(k, TD[dt]), to_dev(v, TD[dt]),
                           dq, dk, dv, q_pos0=c["q_pos0"], k_pos0=c["k_pos0"], causal=c["causal"], scale=scale)
    torch.cuda.synchronize()
    bwd_close(dq, gq, "dq", dt)
    bwd_close(dk, gk, "dk", dt)
    bwd_close(dv, gv, "dv", dt)
