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
    """Backward at the full C3 shape, in the launch configuration bench.py times,
    against references computed from the inputs alone (no GPU output enters them).
    dQ rows: exact gradients, with the oracle's forward statistics of each sampled
    row over its whole causal key range. dK / dV keys: keys in the sequence's last
    tiles (its last key, the tile boundaries around it and random ones), whose
    gradients sum over only the few hundred query rows at or after them; each of
    those rows' LSE and delta = dO . O comes from the oracle's forward over the
    row's whole causal range."""
    cfg = CONFIGS["C3"]
    q, k, v = prefill_inputs_torch(cfg, DEV)
    o, lse = run_prefill(ra, cfg, q, k, v)
    gen = torch.Generator(device=DEV).manual_seed(cfg.seed + 7)
    dout = torch.empty_like(o).normal_(0.0, 1.0, generator=gen)
    say(f"attn_bwd {cfg.name} (whole sequence)")
    dq, dk, dv = ra.attn_bwd(q, k, v, o, lse, dout, causal=True, scale=cfg.scale)
    torch.cuda.synchronize()
    del o, lse
    group = cfg.Hq // cfg.Hkv
    rng = np.random.default_rng(cfg.seed + 11)
    worst = 0.0
    # dQ of sampled rows, exact
    for g in (0, cfg.Hkv - 1):
        k_np, v_np = k[0, g].double().cpu().numpy(), v[0, g].double().cpu().numpy()
        for h in (g * group, g * group + group - 1):
            rows = np.unique(np.concatenate([rng.integers(0, cfg.Sq, 6), [0, cfg.Sq - 1, cfg.Sp, cfg.Sp - 1]]))
            rt = torch.as_tensor(rows, device=DEV)
            qr = q[0, h, rt].double().cpu().numpy()
            dr = dout[0, h, rt].double().cpu().numpy()
            o_r, l_r = oracle.attention_rows(qr, rows, k_np, v_np, scale=cfg.scale, causal=True)
            d_r = (dr * o_r).sum(-1)
            ref, _, _ = oracle.block_bwd(qr[None, None], k_np[None, None], v_np[None, None], dr[None, None],
                                         l_r[None, None], d_r[None, None], scale=cfg.scale, causal=True,
                                         q_pos=rows, k_pos0=0)
            got = dq[0, h, rt].double().cpu().numpy()
            err = np.abs(got - ref[0, 0]).max() / np.abs(ref[0, 0]).max()
            worst = max(worst, err)
            assert err <= 2e-2, (g, h, err)
    # dK, dV of keys in the last 256 positions: every query row that sees them
    S = cfg.S
    for g in (0, cfg.Hkv // 2):
        keys = np.unique(np.concatenate([S - 1 - rng.integers(0, 256, 3),
                                         [S - 1, S - 2, S - 64, S - 127, S - 128, S - 129, S - 256]]))
        r0 = int(keys.min())
        rows = np.arange(r0, S)
        k_np, v_np = k[0, g].double().cpu().numpy(), v[0, g].double().cpu().numpy()
        k_s, v_s = k_np[keys], v_np[keys]
        ref_k = np.zeros_like(k_s)
        ref_v = np.zeros_like(v_s)
        for h in range(g * group, (g + 1) * group):
            qh = q[0, h, r0:].double().cpu().numpy()
            dh = dout[0, h, r0:].double().cpu().numpy()
            o_ref, l_ref = oracle.attention_rows(qh, rows, k_np, v_np, scale=cfg.scale, causal=True)
            d_ref = (dh * o_ref).sum(-1)
            _, gk, gv = oracle.block_bwd(qh[None, None], k_s[None, None], v_s[None, None], dh[None, None],
                                         l_ref[None, None], d_ref[None, None], scale=cfg.scale, causal=True,
                                         q_pos=rows, k_pos=keys)
            ref_k += gk[0, 0]
            ref_v += gv[0, 0]
        kt = torch.as_tensor(keys, device=DEV)
        for got, ref, name in ((dk[0, g, kt], ref_k, "dk"), (dv[0, g, kt], ref_v, "dv")):
            err = np.abs(got.double().cpu().numpy() - ref).max() / np.abs(ref).max()
            worst = max(worst, err)
            assert err <= 2e-2, (name, g, err)
    say(f"C3 backward: worst relative max error {worst:.3e}")


@pytest.mark.timeout(900)
def test_c3_backward_zero_query_closed_form(ra):
    """Q = 0 at the full C3 shape: every visible probability is 1 / (r + 1) for
    query row r (causal), so dV at key c is sum_{r >= c} dO_r / (r + 1), summed over
    the KV head's query heads -- a reverse cumulative sum, taken here in float64
    with torch on the device (no kernel of this library) -- and dK = scale dS^T Q
    is exactly zero. Checked at every key of every KV head, through the GPU
    forward and the whole backward."""
    cfg = CONFIGS["C3"]
    _, k, v = prefill_inputs_torch(cfg, DEV)
    q0 = torch.zeros((cfg.B, cfg.Hq, cfg.Sq, cfg.Dqk), dtype=torch.bfloat16, device=DEV)
    o, lse = run_prefill(ra, cfg, q0, k, v)
    gen = torch.Generator(device=DEV).manual_seed(cfg.seed + 8)
    dout = torch.empty_like(o).normal_(0.0, 1.0, generator=gen)
    say(f"attn_bwd {cfg.name} with Q = 0 (whole sequence)")
    dq, dk, dv = ra.attn_bwd(q0, k, v, o, lse, dout, causal=True, scale=cfg.scale)
    torch.cuda.synchronize()
    del o, lse, dq
    assert torch.count_nonzero(dk).item() == 0, "dK must be exactly zero when Q = 0"
    group = cfg.Hq // cfg.Hkv
    inv = 1.0 / torch.arange(1, cfg.S + 1, device=DEV, dtype=torch.float64)
    worst_max = worst_mean = 0.0
    for g in range(cfg.Hkv):
        x = dout[0, g * group:(g + 1) * group].double().sum(0) * inv[:, None]
        ref = torch.flip(torch.cumsum(torch.flip(x, (0,)), 0), (0,))
        err = (dv[0, g].double() - ref).abs()
        rmax = float(err.max()) / float(ref.abs().max())
        rmean = float(err.mean()) / float(ref.abs().mean())
        worst_max, worst_mean = max(worst_max, rmax), max(worst_mean, rmean)
        del x, ref, err
    say(f"C3 backward Q=0: dV worst relative max error {worst_max:.3e}, mean {worst_mean:.3e}")
    assert worst_max <= 2e-2 and worst_mean <= 5e-3, (worst_max, worst_mean)


@pytest.mark.timeout(1200)
def test_c4_backward_sampled_rows_keys_and_closed_form(ra):
    """Backward of the MLA-shaped share (query partition 7 of 8 of S 524288, 128
    heads, D_qk 192, D_v 128) in the launch configuration bench.py times: one step
    of the partition's queries against all 8 KV blocks. References come from the
    inputs alone:
      * dQ of sampled rows: exact, with the oracle's row statistics over each row's
        whole causal key range;
      * dK / dV of keys in the last 256 positions of two heads: every query row that
        sees them (MHA: one query head per KV head), with its LSE and delta from the
        oracle's forward;
      * Q = 0 at every key of every head: each visible probability is 1/(r+1) for the
        query at position r, so dV at key c is sum over the partition's queries
        r >= c of dO_r/(r+1) (fp64 on the device with torch), and dK is exactly 0."""
    cfg = CONFIGS["C4"]
    q0pos = cfg.q_part0 * cfg.Sp
    S = cfg.S
    q, k, v = prefill_inputs_torch(cfg, DEV)
    o, lse = run_prefill(ra, cfg, q, k, v)
    gen = torch.Generator(device=DEV).manual_seed(cfg.seed + 7)
    dout = torch.empty_like(o).normal_(0.0, 1.0, generator=gen)
    say(f"attn_bwd step {cfg.name}: partition 7 against all KV blocks")
    delta = ra.attn_bwd_preprocess(o, dout)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    ra.block_attn_bwd_step(q, dout, lse, delta, k, v, dq, dk, dv, q_pos0=q0pos, k_pos0=0, causal=True,
                           scale=cfg.scale)
    torch.cuda.synchronize()
    del o, lse, delta
    rng = np.random.default_rng(cfg.seed + 11)
    worst = 0.0
    for h in (0, cfg.Hq - 1):
        k_np, v_np = k[0, h].double().cpu().numpy(), v[0, h].double().cpu().numpy()
        # dQ of sampled rows (local indices), exact
        rows = np.unique(np.concatenate([rng.integers(0, cfg.Sq, 4), [0, cfg.Sq - 1]]))
        rt = torch.as_tensor(rows, device=DEV)
        qr = q[0, h, rt].double().cpu().numpy()
        dr = dout[0, h, rt].double().cpu().numpy()
        o_r, l_r = oracle.attention_rows(qr, q0pos + rows, k_np, v_np, scale=cfg.scale, causal=True)
        ref, _, _ = oracle.block_bwd(qr[None, None], k_np[None, None], v_np[None, None], dr[None, None],
                                     l_r[None, None], ((dr * o_r).sum(-1))[None, None], scale=cfg.scale,
                                     causal=True, q_pos=q0pos + rows, k_pos0=0)
        err = np.abs(dq[0, h, rt].double().cpu().numpy() - ref[0, 0]).max() / np.abs(ref[0, 0]).max()
        worst = max(worst, err)
        assert err <= 2e-2, ("dq", h, err)
        # dK, dV of keys in the last 256 positions: every query row at or after them
        keys = np.unique(np.concatenate([S - 1 - rng.integers(0, 256, 3), [S - 1, S - 2, S - 128, S - 129, S - 256]]))
        r0 = int(keys.min()) - q0pos
        lrows = np.arange(r0, cfg.Sq)
        qh = q[0, h, r0:].double().cpu().numpy()
        dh = dout[0, h, r0:].double().cpu().numpy()
        o_ref, l_ref = oracle.attention_rows(qh, q0pos + lrows, k_np, v_np, scale=cfg.scale, causal=True)
        _, gk, gv = oracle.block_bwd(qh[None, None], k_np[keys][None, None], v_np[keys][None, None], dh[None, None],
                                     l_ref[None, None], ((dh * o_ref).sum(-1))[None, None], scale=cfg.scale,
                                     causal=True, q_pos=q0pos + lrows, k_pos=keys)
        kt = torch.as_tensor(keys, device=DEV)
        for got, refg, name in ((dk[0, h, kt], gk[0, 0], "dk"), (dv[0, h, kt], gv[0, 0], "dv")):
            err = np.abs(got.double().cpu().numpy() - refg).max() / np.abs(refg).max()
            worst = max(worst, err)
            assert err <= 2e-2, (name, h, err)
        del k_np, v_np
    say(f"C4 backward: worst relative max error {worst:.3e}")
    del dq, dk, dv, dout
    torch.cuda.empty_cache()

    # Q = 0 closed form at every key
    qz = torch.zeros_like(q)
    del q
    o, lse = run_prefill(ra, cfg, qz, k, v)
    gen = torch.Generator(device=DEV).manual_seed(cfg.seed + 8)
    dout = torch.empty_like(o).normal_(0.0, 1.0, generator=gen)
    delta = ra.attn_bwd_preprocess(o, dout)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    dq = torch.zeros(qz.shape, dtype=torch.float32, device=DEV)
    say(f"attn_bwd step {cfg.name} with Q = 0")
    ra.block_attn_bwd_step(qz, dout, lse, delta, k, v, dq, dk, dv, q_pos0=q0pos, k_pos0=0, causal=True,
                           scale=cfg.scale)
    torch.cuda.synchronize()
    del o, lse, delta, dq
    assert torch.count_nonzero(dk).item() == 0, "dK must be exactly zero when Q = 0"
    del dk
    inv = 1.0 / torch.arange(q0pos + 1, S + 1, device=DEV, dtype=torch.float64)
    worst_max = worst_mean = 0.0
    for h in range(cfg.Hq):
        x = dout[0, h].double() * inv[:, None]                       # [Sq, Dv], query r at q0pos + r
        tail = torch.flip(torch.cumsum(torch.flip(x, (0,)), 0), (0,))  # keys at q0pos + c, c < Sq
        err_tail = (dv[0, h, q0pos:].double() - tail).abs()
        err_head = (dv[0, h, :q0pos].double() - tail[0]).abs()        # keys before the partition see every query
        rmax = max(float(err_tail.max()), float(err_head.max())) / float(tail.abs().max())
        rmean = (float(err_tail.sum()) + float(err_head.sum())) / (S * cfg.Dv) / \
            ((float(tail.abs().sum()) + q0pos * float(tail[0].abs().sum())) / (S * cfg.Dv))
        worst_max, worst_mean = max(worst_max, rmax), max(worst_mean, rmean)
        del x, tail, err_tail, err_head
    say(f"C4 backward Q=0: dV worst relative max error {worst_max:.3e}, mean {worst_mean:.3e}")
    assert worst_max <= 2e-2 and worst_mean <= 5e-3, (worst_max, worst_mean)


@pytest.mark.timeout(600)
def test_fp32_backward_workload_sampled_rows_keys_and_closed_form(ra):
    """The fp32 backward at the shape bench.py times it on (causal, GQA 8:2, S 8192 in
    4 partitions, d 128, fp32), in the same launch configuration: the fp32 ring
    forward, then the delta preprocess and one step over the whole sequence. The
    references come from the inputs alone, as for C3 (dQ of sampled rows; dK / dV of
    keys in the last 256 positions, over every query row that sees them), at the
    fp32 gate of the backward parity tests: max error <= 1e-4 of the largest
    reference value.

    Then Q = 0: dV at key c is sum_{r >= c} dO_r / (r + 1) over the KV head's four
    query heads (fp64 on the device with torch) and dK is exactly 0, at every key.
    That sum runs over up to n = 32768 terms in fp32, so its rounding is about
    sqrt(n) 2^-24 ~ 1e-5 of each value: the mean gate there is 5e-5 of the mean
    |reference| (and max 1e-4 of the largest)."""
    from bench import F32B as cfg
    S = cfg.S
    q, k, v = prefill_inputs_torch(cfg, DEV)
    o, lse = run_prefill(ra, cfg, q, k, v)
    gen = torch.Generator(device=DEV).manual_seed(cfg.seed + 7)
    dout = torch.empty_like(o).normal_(0.0, 1.0, generator=gen)
    say(f"attn_bwd {cfg.name} (whole sequence, fp32)")
    delta = ra.attn_bwd_preprocess(o, dout)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=DEV)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=DEV)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=DEV)
    ra.block_attn_bwd_step(q, dout, lse, delta, k, v, dq, dk, dv, q_pos0=0, k_pos0=0, causal=True, scale=cfg.scale)
    torch.cuda.synchronize()
    del o, lse, delta
    group = cfg.Hq // cfg.Hkv
    rng = np.random.default_rng(cfg.seed + 11)
    worst = 0.0
    for g in (0, cfg.Hkv - 1):
        k_np, v_np = k[0, g].double().cpu().numpy(), v[0, g].double().cpu().numpy()
        for h in (g * group, g * group + group - 1):
            rows = np.unique(np.concatenate([rng.integers(0, S, 6), [0, S - 1, cfg.Sp, cfg.Sp - 1]]))
            rt = torch.as_tensor(rows, device=DEV)
            qr = q[0, h, rt].double().cpu().numpy()
            dr = dout[0, h, rt].double().cpu().numpy()
            o_r, l_r = oracle.attention_rows(qr, rows, k_np, v_np, scale=cfg.scale, causal=True)
            ref, _, _ = oracle.block_bwd(qr[None, None], k_np[None, None], v_np[None, None], dr[None, None],
                                         l_r[None, None], ((dr * o_r).sum(-1))[None, None], scale=cfg.scale,
                                         causal=True, q_pos=rows, k_pos0=0)
            err = np.abs(dq[0, h, rt].double().cpu().numpy() - ref[0, 0]).max() / np.abs(ref[0, 0]).max()
            worst = max(worst, err)
            assert err <= 1e-4, ("dq", g, h, err)
        keys = np.unique(np.concatenate([S - 1 - rng.integers(0, 256, 3),
                                         [S - 1, S - 2, S - 32, S - 33, S - 64, S - 128, S - 256]]))
        r0 = int(keys.min())
        rows = np.arange(r0, S)
        ref_k = np.zeros((len(keys), cfg.Dqk))
        ref_v = np.zeros((len(keys), cfg.Dv))
        for h in range(g * group, (g + 1) * group):
            qh = q[0, h, r0:].double().cpu().numpy()
            dh = dout[0, h, r0:].double().cpu().numpy()
            o_ref, l_ref = oracle.attention_rows(qh, rows, k_np, v_np, scale=cfg.scale, causal=True)
            _, gk, gv = oracle.block_bwd(qh[None, None], k_np[keys][None, None], v_np[keys][None, None],
                                         dh[None, None], l_ref[None, None], ((dh * o_ref).sum(-1))[None, None],
                                         scale=cfg.scale, causal=True, q_pos=rows, k_pos=keys)
            ref_k += gk[0, 0]
            ref_v += gv[0, 0]
        kt = torch.as_tensor(keys, device=DEV)
        for got, refg, name in ((dk[0, g, kt], ref_k, "dk"), (dv[0, g, kt], ref_v, "dv")):
            err = np.abs(got.double().cpu().numpy() - refg).max() / np.abs(refg).max()
            worst = max(worst, err)
            assert err <= 1e-4, (name, g, err)
    say(f"{cfg.name} backward: worst relative max error {worst:.3e}")
    del dq, dk, dv, dout

    qz = torch.zeros_like(q)
    del q
    o, lse = run_prefill(ra, cfg, qz, k, v)
    gen = torch.Generator(device=DEV).manual_seed(cfg.seed + 8)
    dout = torch.empty_like(o).normal_(0.0, 1.0, generator=gen)
    say(f"attn_bwd {cfg.name} with Q = 0")
    dq, dk, dv = ra.attn_bwd(qz, k, v, o, lse, dout, causal=True, scale=cfg.scale)
    torch.cuda.synchronize()
    del o, lse, dq
    assert torch.count_nonzero(dk).item() == 0, "dK must be exactly zero when Q = 0"
    inv = 1.0 / torch.arange(1, S + 1, device=DEV, dtype=torch.float64)
    worst_max = worst_mean = 0.0
    for g in range(cfg.Hkv):
        x = dout[0, g * group:(g + 1) * group].double().sum(0) * inv[:, None]
        ref = torch.flip(torch.cumsum(torch.flip(x, (0,)), 0), (0,))
        err = (dv[0, g].double() - ref).abs()
        worst_max = max(worst_max, float(err.max()) / float(ref.abs().max()))
        worst_mean = max(worst_mean, float(err.mean()) / float(ref.abs().mean()))
    say(f"{cfg.name} backward Q=0: dV worst relative max error {worst_max:.3e}, mean {worst_mean:.3e}")
    assert worst_max <= 1e-4 and worst_mean <= 5e-5, (worst_max, worst_mean)
