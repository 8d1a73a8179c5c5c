"""Full-size parity on the large workloads, in the launch configuration bench.py times:
sampled query rows checked one by one against the fp64 oracle, every decode row and
partial, and closed forms that hold at any size (Q = 0 turns attention into a
prefix mean of V with LSE = ln(number of visible keys))."""
import math
from collections import defaultdict

import numpy as np
import pytest
import torch

import oracle
from workloads import (CONFIGS, FP8_K_SCALE, FP8_V_SCALE, decode_inputs_fp8_torch, decode_inputs_torch,
                       prefill_inputs_torch, sample_rows)
from gpu_util import assert_close, np64, say

pytestmark = [pytest.mark.gpu, pytest.mark.slow]

DEV = torch.device("cuda:0")


@pytest.fixture(scope="module")
def ra():
    import blockwise_exact_attention_block_amd as m
    m.load_library()
    return m


def run_prefill(ra, cfg, q, k, v):
    say(f"ring_attn_fwd {cfg.name}: {cfg.description}")
    o, lse = ra.ring_attn_fwd(q, k, v, P=cfg.P, causal=cfg.causal, scale=cfg.scale, q_part0=cfg.q_part0)
    torch.cuda.synchronize()
    return o, lse


def check_sampled_rows(cfg, q, k, v, o, lse, rows):
    """Group the sampled (b, h, r) rows by KV head, pull that head's K/V to the host
    once, and compare each row with the oracle's definition."""
    group = cfg.Hq // cfg.Hkv
    by_kv = defaultdict(list)
    for b, h, r in rows:
        by_kv[(b, h // group)].append((h, r))
    worst_o = worst_l = 0.0
    for (b, g), hr in sorted(by_kv.items()):
        k_np = k[b, g].float().cpu().numpy()
        v_np = v[b, g].float().cpu().numpy()
        hs = torch.tensor([x[0] for x in hr], device=q.device)
        rs = torch.tensor([x[1] for x in hr], device=q.device)
        q_rows = q[b, hs, rs].float().cpu().numpy()
        pos = cfg.q_part0 * cfg.Sp + rs.cpu().numpy()
        o_ref, l_ref = oracle.attention_rows(q_rows, pos, k_np, v_np, scale=cfg.scale, causal=cfg.causal, k_pos0=0)
        do, dl = assert_close(np64(o[b, hs, rs]), np64(lse[b, hs, rs]), o_ref, l_ref, cfg.dtype,
                              f"{cfg.name} kv head {g}")
        worst_o, worst_l = max(worst_o, do), max(worst_l, dl)
    say(f"{cfg.name}: {len(rows)} rows, max|dO| {worst_o:.3e}, max|dLSE| {worst_l:.3e}")


def check_zero_query_closed_form(ra, cfg, k, v):
    """Q = 0: every visible score is 0, so O(row) = mean of V over keys 0..pos and
    LSE = ln(pos + 1) (causal) -- checked on every row of every head. The prefix
    means are taken in float64 with torch on the device (no kernel of this library)."""
    q0 = torch.zeros((cfg.B, cfg.Hq, cfg.Sq, cfg.Dqk), dtype=torch.bfloat16, device=DEV)
    o, lse = run_prefill(ra, cfg, q0, k, v)
    del q0
    group = cfg.Hq // cfg.Hkv
    pos = torch.arange(cfg.q_part0 * cfg.Sp, (cfg.q_part0 + cfg.n_qparts) * cfg.Sp, device=DEV, dtype=torch.float64)
    cnt = pos + 1 if cfg.causal else torch.full_like(pos, float(cfg.S))
    lse_ref = torch.log(cnt)
    worst_o = worst_l = 0.0
    for b in range(cfg.B):
        for g in range(cfg.Hkv):
            csum = torch.cumsum(v[b, g].double(), dim=0)
            if cfg.causal:
                mean = csum[cfg.q_part0 * cfg.Sp:(cfg.q_part0 + cfg.n_qparts) * cfg.Sp] / cnt[:, None]
            else:
                mean = (csum[-1] / cfg.S).expand(cfg.Sq, cfg.Dv)
            for h in range(g * group, (g + 1) * group):
                worst_o = max(worst_o, float((o[b, h].double() - mean).abs().max()))
                worst_l = max(worst_l, float((lse[b, h].double() - lse_ref).abs().max()))
            del csum, mean
    say(f"{cfg.name} Q=0 closed form: max|dO| {worst_o:.3e}, max|dLSE| {worst_l:.3e}")
    assert worst_o <= 2e-2 and worst_l <= 1e-2, (worst_o, worst_l)


@pytest.mark.timeout(900)
def test_c3_sampled_rows_and_closed_form(ra):
    cfg = CONFIGS["C3"]
    q, k, v = prefill_inputs_torch(cfg, DEV)
    o, lse = run_prefill(ra, cfg, q, k, v)
    rows = sample_rows(cfg, cfg.check_rows)
    check_sampled_rows(cfg, q, k, v, o, lse, rows)
    del o, lse, q
    torch.cuda.empty_cache()
    check_zero_query_closed_form(ra, cfg, k, v)


@pytest.mark.timeout(900)
def test_c3_ring_step_sampled_rows(ra):
    """The step API at the C3 partition size, as bench.py times it (partition 1
    against KV block 0, fp32 state), then the diagonal block 1: after the first
    step the state is attention over block 0 alone, after the second it is the
    partition's causal attention. Sampled rows against the oracle, both times."""
    cfg = CONFIGS["C3"]
    Sp, group = cfg.Sp, cfg.Hq // cfg.Hkv
    q, k, v = prefill_inputs_torch(cfg, DEV)
    qi = q[:, :, Sp:2 * Sp].contiguous()
    del q
    o_acc, l_acc = ra.init_state(qi, cfg.Dv)
    rng = np.random.default_rng(cfg.seed + 17)
    rows = sorted({(0, int(h), int(r)) for h, r in zip(rng.integers(0, cfg.Hq, 192), rng.integers(0, Sp, 192))}
                  | {(0, 0, 0), (0, cfg.Hq - 1, Sp - 1), (0, 5, 255), (0, 5, 256)})
    for nblk in (1, 2):
        j = nblk - 1
        say(f"block_attn_step {cfg.name}: partition 1 x KV block {j}")
        ra.block_attn_step(qi, k[:, :, j * Sp:(j + 1) * Sp].contiguous(), v[:, :, j * Sp:(j + 1) * Sp].contiguous(),
                           o_acc, l_acc, q_pos0=Sp, k_pos0=j * Sp, causal=True, scale=cfg.scale)
        torch.cuda.synchronize()
        by_kv = defaultdict(list)
        for b, h, r in rows:
            by_kv[(b, h // group)].append((h, r))
        worst_o = worst_l = 0.0
        for (b, g), hr in sorted(by_kv.items()):
            k_np = k[b, g, :nblk * Sp].float().cpu().numpy()
            v_np = v[b, g, :nblk * Sp].float().cpu().numpy()
            hs = torch.tensor([x[0] for x in hr], device=DEV)
            rs = torch.tensor([x[1] for x in hr], device=DEV)
            o_ref, l_ref = oracle.attention_rows(qi[b, hs, rs].float().cpu().numpy(), Sp + rs.cpu().numpy(), k_np,
                                                 v_np, scale=cfg.scale, causal=True, k_pos0=0)
            do, dl = assert_close(np64(o_acc[b, hs, rs]), np64(l_acc[b, hs, rs]), o_ref, l_ref, "bf16",
                                  f"{cfg.name} step {nblk} kv head {g}")
            worst_o, worst_l = max(worst_o, do), max(worst_l, dl)
        say(f"{cfg.name} after {nblk} step(s): {len(rows)} rows, max|dO| {worst_o:.3e}, max|dLSE| {worst_l:.3e}")


@pytest.mark.timeout(1200)
def test_c4_sampled_rows_and_closed_form(ra):
    cfg = CONFIGS["C4"]
    q, k, v = prefill_inputs_torch(cfg, DEV)
    o, lse = run_prefill(ra, cfg, q, k, v)
    rows = sample_rows(cfg, cfg.check_rows)
    check_sampled_rows(cfg, q, k, v, o, lse, rows)
    del o, lse, q
    torch.cuda.empty_cache()
    check_zero_query_closed_form(ra, cfg, k, v)
    del k, v
    torch.cuda.empty_cache()


@pytest.mark.timeout(900)
def test_c5_every_row_and_partial(ra):
    cfg = CONFIGS["C5"]
    q, k, v = decode_inputs_torch(cfg, DEV)
    say(f"splitkv_decode {cfg.name}: {cfg.description}")
    op, lp, o, l = ra.splitkv_decode(q, k, v, n_splits=cfg.n_splits, scale=cfg.scale)
    torch.cuda.synchronize()
    worst = [0.0, 0.0, 0.0, 0.0]
    for b in range(cfg.B):
        opr, lpr, orf, lrf = oracle.splitkv_decode(q[b:b + 1].float().cpu().numpy(), k[b:b + 1].float().cpu().numpy(),
                                                   v[b:b + 1].float().cpu().numpy(), n_splits=cfg.n_splits,
                                                   scale=cfg.scale)
        d1 = assert_close(np64(op[b:b + 1]), np64(lp[b:b + 1]), opr, lpr, "bf16", f"C5 partials b={b}")
        d2 = assert_close(np64(o[b:b + 1]), np64(l[b:b + 1]), orf, lrf, "bf16", f"C5 merged b={b}")
        worst = [max(worst[0], d1[0]), max(worst[1], d1[1]), max(worst[2], d2[0]), max(worst[3], d2[1])]
    say(f"C5: partials max|dO| {worst[0]:.3e} |dLSE| {worst[1]:.3e}; merged max|dO| {worst[2]:.3e} "
        f"|dLSE| {worst[3]:.3e}")
    # the partial kernel alone reproduces the partials bit for bit
    op2, lp2 = ra.splitkv_partial(q, k, v, n_splits=cfg.n_splits, scale=cfg.scale)
    torch.cuda.synchronize()
    assert torch.equal(op2, op) and torch.equal(lp2, lp)


@pytest.mark.timeout(900)
def test_c5f_fp8_cache_every_row_and_partial(ra):
    cfg = CONFIGS["C5F"]
    q, k, v = decode_inputs_fp8_torch(cfg, DEV)
    say(f"splitkv_decode_fp8 {cfg.name}: {cfg.description}")
    op, lp, o, l = ra.splitkv_decode_fp8(q, k, v, k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE,
                                         n_splits=cfg.n_splits, scale=cfg.scale)
    torch.cuda.synchronize()
    worst = [0.0, 0.0, 0.0, 0.0]
    for b in range(cfg.B):
        kb = oracle.dequantize(k[b:b + 1].view(torch.uint8).cpu().numpy(), FP8_K_SCALE)
        vb = oracle.dequantize(v[b:b + 1].view(torch.uint8).cpu().numpy(), FP8_V_SCALE)
        opr, lpr, orf, lrf = oracle.splitkv_decode(q[b:b + 1].float().cpu().numpy(), kb, vb,
                                                   n_splits=cfg.n_splits, scale=cfg.scale)
        d1 = assert_close(np64(op[b:b + 1]), np64(lp[b:b + 1]), opr, lpr, "bf16", f"C5F partials b={b}")
        d2 = assert_close(np64(o[b:b + 1]), np64(l[b:b + 1]), orf, lrf, "bf16", f"C5F merged b={b}")
        worst = [max(worst[0], d1[0]), max(worst[1], d1[1]), max(worst[2], d2[0]), max(worst[3], d2[1])]
    say(f"C5F: partials max|dO| {worst[0]:.3e} |dLSE| {worst[1]:.3e}; merged max|dO| {worst[2]:.3e} "
        f"|dLSE| {worst[3]:.3e}")


@pytest.mark.timeout(900)
def test_c3_backward_sampled_rows_and_keys(ra):
    """Backward at the full C3 shape, in the launch configuration bench.py times.
    dQ rows: exact gradients (the oracle's forward statistics of each sampled row
    over its whole causal key range). dK / dV keys: the definition of one key's
    gradient summed over every query of its group that sees it, given the GPU's
    saved row LSE and delta (the step's inputs, checked themselves above)."""
    cfg = CONFIGS["C3"]
    q, k, v = prefill_inputs_torch(cfg, DEV)
    o, lse = run_prefill(ra, cfg, q, k, v)
    gen = torch.Generator(device=DEV).manual_seed(cfg.seed + 7)
    dout = torch.empty_like(o).normal_(0.0, 1.0, generator=gen)
    say(f"attn_bwd {cfg.name} (whole sequence)")
    dq, dk, dv = ra.attn_bwd(q, k, v, o, lse, dout, causal=True, scale=cfg.scale)
    delta = ra.attn_bwd_preprocess(o, dout)
    torch.cuda.synchronize()
    del o
    group = cfg.Hq // cfg.Hkv
    rng = np.random.default_rng(cfg.seed + 11)
    worst = 0.0
    # dQ of sampled rows, exact
    for g in (0, cfg.Hkv - 1):
        k_np, v_np = k[0, g].float().cpu().numpy(), v[0, g].float().cpu().numpy()
        for h in (g * group, g * group + group - 1):
            rows = np.unique(np.concatenate([rng.integers(0, cfg.Sq, 6), [0, cfg.Sq - 1, cfg.Sp, cfg.Sp - 1]]))
            rt = torch.as_tensor(rows, device=DEV)
            qr = q[0, h, rt].float().cpu().numpy()
            dr = dout[0, h, rt].float().cpu().numpy()
            o_r, l_r = oracle.attention_rows(qr, rows, k_np, v_np, scale=cfg.scale, causal=True)
            d_r = (dr * o_r).sum(-1)
            ref, _, _ = oracle.block_bwd(qr[None, None], k_np[None, None], v_np[None, None], dr[None, None],
                                         l_r[None, None], d_r[None, None], scale=cfg.scale, causal=True,
                                         q_pos=rows, k_pos0=0)
            got = dq[0, h, rt].double().cpu().numpy()
            err = np.abs(got - ref[0, 0]).max() / np.abs(ref[0, 0]).max()
            worst = max(worst, err)
            assert err <= 2e-2, (g, h, err)
    # dK, dV of sampled keys, given the saved row statistics
    for g in (0, cfg.Hkv // 2):
        keys = np.unique(np.concatenate([rng.integers(0, cfg.S, 3), [0, cfg.S - 1]]))
        kt = torch.as_tensor(keys, device=DEV)
        k_s = k[0, g, kt].float().cpu().numpy()
        v_s = v[0, g, kt].float().cpu().numpy()
        ref_k = np.zeros_like(k_s, dtype=np.float64)
        ref_v = np.zeros_like(v_s, dtype=np.float64)
        for h in range(g * group, (g + 1) * group):
            qh = q[0, h].float().cpu().numpy()
            dh = dout[0, h].float().cpu().numpy()
            _, gk, gv = oracle.block_bwd(qh[None, None], k_s[None, None], v_s[None, None], dh[None, None],
                                         lse[0, h].double().cpu().numpy()[None, None],
                                         delta[0, h].double().cpu().numpy()[None, None], scale=cfg.scale,
                                         causal=True, q_pos0=0, k_pos=keys)
            ref_k += gk[0, 0]
            ref_v += gv[0, 0]
        for got, ref, name in ((dk[0, g, kt], ref_k, "dk"), (dv[0, g, kt], ref_v, "dv")):
            err = np.abs(got.double().cpu().numpy() - ref).max() / np.abs(ref).max()
            worst = max(worst, err)
            assert err <= 2e-2, (name, g, err)
    say(f"C3 backward: worst relative max error {worst:.3e}")
