#!/usr/bin/env python3
"""One-GPU benchmark of the ring-ordered blockwise exact attention hot path (MI355X).

Headline (``value``): causal ring prefill throughput in algorithmic TFLOP/s (only
visible query/key pairs count, 2 (D_qk + D_v) FLOP each) on the largest workload
that fits one GPU, one GPU's share of an MLA-shaped prefill at a ring of 8: the
last query partition (65536 tokens, index 7 of 8) of S = 524288, 128 heads,
D_qk 192, D_v 128, bf16, attending to all 8 KV blocks of 65536 tokens in ring
order with causal masking. A step is one ring launch over that share; inputs are
resident in HBM before the timed region.

The same JSON line carries:
  prefill_other the 70B-class GQA ring (B 1, 64/8 heads, S 131072 in 8 partitions,
                d 128, bf16), the small bf16 MHA ring (H 8, S 8192 in 4, d 128) and
                the fp32 non-causal ring (H 1, S 1024 in 4, d 64), each timed with
                its own roofline;
  striped, ring_step, backward   on the 70B-class GQA workload;
  decode        split-KV decode (B 16, 64/8 heads, KV length 131072 in 8 splits,
                bf16) in HBM GB/s of algorithmic bytes, and the same over an fp8
                cache;
  roofline      for each dominant kernel: algorithmic work per launch over its
                average launch time, taken with HIP events on the launch stream
                during the timed region, against the MI355X peak (bf16 dense MFMA
                2.5 PFLOP/s; HBM 8 TB/s), and the HBM traffic from rocprofv3
                counters when they were taken on the current kernel source; for
                the bf16 prefill also the shader clock rocprofv3 measured over
                that kernel (GRBM_GUI_ACTIVE per XCD over the launch) and the
                fraction of the MFMA peak recomputed at that clock;
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload,
                timed on this host's cores, with the full workload's oracle time
                extrapolated at that rate; the other workloads likewise (the two
                small ones run in full).

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C4|C3|C2]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBPS = 8000.0      # MI355X HBM3E
CSRC = os.path.join(ROOT, "blockwise_exact_attention_block_amd", "csrc")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.txt")
SCLK_FILE = os.path.join(ROOT, "profiles", "sclk.txt")
# dense bf16 MFMA work per clock: 256 CUs x 4 SIMDs x one 32x32x16 product (32768 FLOP)
# per 32 cycles; 2.4 GHz gives the 2.5 PFLOP/s peak
MFMA_BF16_FLOP_PER_CLK = 256 * 4 * 1024
KERNEL_SOURCES = {
    "prefill": ["prefill_bf16.hip", "common.hpp"],
    "decode": ["decode_bf16.hip", "common.hpp"],
}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def source_sha(kind: str) -> str:
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[kind]:
        with open(os.path.join(CSRC, name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def recorded(path: str, kind: str, workload: str, nvalues: int):
    """The values recorded in a profiles/ table for (kernel kind, workload) on this
    exact kernel source, or None."""
    if not os.path.exists(path):
        return None
    sha = source_sha(kind)
    with open(path) as f:
        for line in f:
            parts = line.split("#", 1)[0].split()
            if len(parts) == 3 + nvalues and parts[:3] == [kind, workload, sha]:
                return [float(x) for x in parts[3:]]
    return None


def recorded_traffic(kind: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE,
    scaled by the copy-kernel calibration), if recorded for this exact source."""
    r = recorded(TRAFFIC_FILE, kind, workload, 2)
    return None if r is None else r[0] + r[1]


def prefill_flops(cfg) -> int:
    """Algorithmic FLOPs of one ring prefill launch: visible pairs x 2 (D_qk + D_v),
    over every computed query partition and head."""
    Sp, P = cfg.Sp, cfg.P
    pairs = 0
    for i in range(cfg.q_part0, cfg.q_part0 + cfg.n_qparts):
        pairs += (i * Sp * Sp + Sp * (Sp + 1) // 2) if cfg.causal else P * Sp * Sp
    return 2 * (cfg.Dqk + cfg.Dv) * pairs * cfg.Hq * cfg.B


def partition_pairs(Sp: int, P: int, i: int, causal: bool, layout: str) -> int:
    """Visible (query, key) pairs of query partition i in a ring of P partitions of
    Sp tokens. Contiguous: i full blocks and the diagonal triangle. Striped
    (partition p = tokens p, p+P, ...): blocks j <= i hold the triangle with its
    diagonal, blocks j > i the triangle without it."""
    if not causal:
        return P * Sp * Sp
    if layout == "striped":
        return (i + 1) * Sp * (Sp + 1) // 2 + (P - 1 - i) * Sp * (Sp - 1) // 2
    return i * Sp * Sp + Sp * (Sp + 1) // 2


def run_striped(args, ra, torch, stream, cfg, q, k, v):
    """Striped layout on the same workload: the whole ring (same visible pairs as
    the contiguous one), and the last partition's share -- the work of the ring's
    slowest rank -- under both layouts."""
    out = torch.empty((cfg.B, cfg.Hq, cfg.Sq, cfg.Dv), dtype=torch.bfloat16, device=q.device)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.Sq), dtype=torch.float32, device=q.device)
    steps, warm = max(2, min(args.steps, 5)), 1
    flops = prefill_flops(cfg)
    log(f"[bench] striped ring: {warm} warmup + {steps} timed steps")
    w_all, e_all = timed(lambda: ra.ring_attn_fwd(q, k, v, P=cfg.P, causal=cfg.causal, scale=cfg.scale,
                                                  q_part0=cfg.q_part0, out=out, lse=lse, layout="striped"),
                         steps, warm, stream, torch)
    last = cfg.P - 1
    qs = q[:, :, (last - cfg.q_part0) * cfg.Sp:(last - cfg.q_part0 + 1) * cfg.Sp] if cfg.q_part0 <= last < cfg.q_part0 + cfg.n_qparts else None
    share = {}
    if qs is not None:
        qs = qs.contiguous()
        o1 = torch.empty((cfg.B, cfg.Hq, cfg.Sp, cfg.Dv), dtype=torch.bfloat16, device=q.device)
        l1 = torch.empty((cfg.B, cfg.Hq, cfg.Sp), dtype=torch.float32, device=q.device)
        for layout in ("contiguous", "striped"):
            _, ev = timed(lambda: ra.ring_attn_fwd(qs, k, v, P=cfg.P, causal=cfg.causal, scale=cfg.scale,
                                                   q_part0=last, out=o1, lse=l1, layout=layout),
                          steps, warm, stream, torch)
            pairs = partition_pairs(cfg.Sp, cfg.P, last, cfg.causal, layout)
            f = 2 * (cfg.Dqk + cfg.Dv) * pairs * cfg.Hq * cfg.B
            share[layout] = {"launch_ms": round(ev, 4), "flops": f, "tflops": round(f / (ev * 1e-3) / 1e12, 2)}
        del o1, l1
    res = {
        "workload": f"{cfg.name} in the striped layout (partition p = tokens p, p+P, ...)",
        "ring_ms_per_step": round(w_all, 4),
        "ring_tflops": round(flops / (w_all * 1e-3) / 1e12, 2),
        "ring_launch_ms": round(e_all, 4),
    }
    if share:
        c, s_ = share["contiguous"], share["striped"]
        res["last_partition_share"] = {
            "partition": last,
            "contiguous": c,
            "striped": s_,
            "speedup": round(c["launch_ms"] / s_["launch_ms"], 3),
            "pair_ratio": round(c["flops"] / s_["flops"], 3),
        }
        log(f"[bench] striped: ring {w_all:.3f} ms; last partition {c['launch_ms']:.3f} ms contiguous vs "
            f"{s_['launch_ms']:.3f} ms striped ({c['launch_ms'] / s_['launch_ms']:.2f}x)")
    del out, lse
    return res


def run_ring_step(args, ra, torch, stream, cfg, q, k, v):
    """One full ring step through the step API, as one rank runs it when a KV block
    arrives: the queries of a partition against a whole earlier block (every pair
    visible), merged into the running fp32 (O, LSE) state read from and written
    back to HBM. FLOPs count the block's pairs."""
    if cfg.q_part0 != 0 or cfg.n_qparts < 2:
        return None                                      # needs partitions 0 and 1 in the launch
    Sp = cfg.Sp
    qi = q[:, :, Sp:2 * Sp].contiguous()                  # queries of partition 1
    kb = k[:, :, :Sp].contiguous()                        # KV block 0
    vb = v[:, :, :Sp].contiguous()
    o_acc, l_acc = ra.init_state(qi, cfg.Dv)
    steps, warm = max(2, min(args.steps, 5)), 1
    log(f"[bench] ring step: {warm} warmup + {steps} timed steps")
    w, ev = timed(lambda: ra.block_attn_step(qi, kb, vb, o_acc, l_acc, q_pos0=Sp, k_pos0=0, causal=cfg.causal,
                                             scale=cfg.scale), steps, warm, stream, torch)
    f = 2 * (cfg.Dqk + cfg.Dv) * Sp * Sp * cfg.Hq * cfg.B
    del qi, kb, vb, o_acc, l_acc
    return {
        "workload": f"{cfg.name}: one full ring step (partition 1 against KV block 0), "
                    "fp32 running state in HBM",
        "launch_ms": round(ev, 4),
        "flops": f,
        "tflops": round(f / (ev * 1e-3) / 1e12, 2),
        "frac_of_bf16_peak": round(f / (ev * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
    }


def backward_flops(cfg) -> int:
    """Algorithmic FLOPs of the backward pass: the five products per visible pair
    (S = Q K^T, dP = dO V^T, dV = P^T dO, dK = dS^T Q, dQ = dS K), 2 (3 D_qk + 2 D_v)
    per pair; recomputed S and dP are not counted."""
    return prefill_flops(cfg) // (2 * (cfg.Dqk + cfg.Dv)) * 2 * (3 * cfg.Dqk + 2 * cfg.Dv)


def run_backward(args, ra, torch, stream, cfg, q, k, v):
    """Backward of the prefill workload's computed query partitions: delta
    preprocess plus one step over those queries against all P KV blocks (every
    visible (query partition, KV block) pair), fp32 gradients. For the whole
    sequence that is the full backward; for one partition it is one rank's share."""
    out, lse = ra.ring_attn_fwd(q, k, v, P=cfg.P, causal=cfg.causal, scale=cfg.scale, q_part0=cfg.q_part0)
    dout = torch.empty_like(out).normal_(0.0, 1.0, generator=torch.Generator(device=q.device).manual_seed(cfg.seed + 7))
    delta = ra.attn_bwd_preprocess(out, dout)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=q.device)
    steps, warm = max(2, min(args.steps, 3)), 1
    log(f"[bench] {cfg.name} backward: {warm} warmup + {steps} timed steps")
    q_pos0 = cfg.q_part0 * cfg.Sp

    def step():
        ra.attn_bwd_preprocess(out, dout, delta)
        ra.block_attn_bwd_step(q, dout, lse, delta, k, v, dq, dk, dv, q_pos0=q_pos0, k_pos0=0, causal=cfg.causal,
                               scale=cfg.scale)

    wall, ev = timed(step, steps, warm, stream, torch)
    flops = backward_flops(cfg)
    log(f"[bench] backward {wall:.3f} ms/step, {flops / (wall * 1e-3) / 1e12:.1f} TFLOP/s (algorithmic)")
    del out, lse, dout, delta, dq, dk, dv
    torch.cuda.empty_cache()
    whole = cfg.q_part0 == 0 and cfg.n_qparts == cfg.P
    return {
        "workload": (f"{cfg.name} backward (delta + dK/dV + dQ over all pairs, fp32 gradients)" if whole else
                     f"{cfg.name} backward of query partitions {cfg.q_part0}..{cfg.q_part0 + cfg.n_qparts - 1} "
                     f"against all {cfg.P} KV blocks (delta + dK/dV + dQ, fp32 gradients)"),
        "ms_per_step": round(wall, 4),
        "launch_ms": round(ev, 4),
        "algorithmic_flops": flops,
        "tflops": round(flops / (wall * 1e-3) / 1e12, 2),
        # both run on the matrix cores: bf16 against the bf16 peak, fp32 the fp32 one
        ("frac_of_bf16_peak" if cfg.dtype == "bf16" else "frac_of_fp32_peak"):
            round(flops / (wall * 1e-3) / 1e12 / (PEAK_BF16_TFLOPS if cfg.dtype == "bf16" else PEAK_FP32_TFLOPS), 4),
    }


def decode_partial_bytes(cfg) -> int:
    """Algorithmic HBM bytes of the split-KV partial kernel: K and V read once (2
    bytes per value, 1 for an fp8 cache), q read, fp32 partial outputs and LSEs
    written."""
    kv = cfg.B * cfg.Hkv * cfg.L * (cfg.Dqk + cfg.Dv) * (1 if cfg.kv_dtype == "fp8" else 2)
    q = cfg.B * cfg.Hq * cfg.Dqk * 2
    parts = cfg.B * cfg.Hq * cfg.n_splits * (cfg.Dv + 1) * 4
    return kv + q + parts


def decode_total_bytes(cfg) -> int:
    """Whole decode: the partial kernel plus the reduction (partials read back,
    bf16 output and fp32 LSE written)."""
    parts = cfg.B * cfg.Hq * cfg.n_splits * (cfg.Dv + 1) * 4
    out = cfg.B * cfg.Hq * (cfg.Dv * 2 + 4)
    return decode_partial_bytes(cfg) + parts + out


def guarded(name, fn, *args):
    """A secondary measurement: an exception in it is recorded in its place on the
    line ({"error": ...}) instead of losing the headline measured before it."""
    try:
        return fn(*args)
    except Exception as e:   # noqa: BLE001 -- reported on the line, not hidden
        log(f"[bench] {name} failed: {e!r}")
        return {"error": f"{type(e).__name__}: {e}"}


def timed(fn, steps, warmup, stream, torch, launches=None):
    """Run warmup untimed steps, then exactly `steps` timed ones bracketed by full
    synchronisation; returns (wall ms per step, mean per-launch ms from events).
    `launches`, if given, receives every step's event time."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        starts[i].record(stream)
        fn()
        ends[i].record(stream)
    torch.cuda.synchronize()
    wall_ms = (time.perf_counter() - t0) * 1e3 / steps
    per = [s.elapsed_time(e) for s, e in zip(starts, ends)]
    if launches is not None:
        launches.extend(per)
    return wall_ms, sum(per) / steps


def launch_stats(per):
    """min / median / max of per-step event times (ms)."""
    v = sorted(per)
    n = len(v)
    med = v[n // 2] if n % 2 else 0.5 * (v[n // 2 - 1] + v[n // 2])
    return {"min": round(v[0], 5), "median": round(med, 5), "max": round(v[-1], 5), "n": n}


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def oracle_sample_inputs(cfg, q, k, v, n_batches: int = 4096):
    """Host copies of what the bounded oracle sample reads: K and V of KV head 0
    (batch 0) and seeded uniform query rows of that head's group, 16 per batch. Taken
    while the device inputs are resident, so that the GPU memory can be released
    before the oracle runs."""
    import numpy as np
    import torch

    rng = np.random.default_rng(cfg.seed + 99)
    group = cfg.Hq // cfg.Hkv
    heads = rng.integers(0, group, size=(n_batches, 16))
    rows = rng.integers(0, cfg.Sq, size=(n_batches, 16))
    # the first batches only: the oracle stops at its time budget long before 4096
    nb = min(n_batches, 256)
    qr = q[0, torch.as_tensor(heads[:nb].ravel()), torch.as_tensor(rows[:nb].ravel())].float().cpu().numpy()
    # fp64 host copies (bf16 and fp32 values convert exactly), made once
    return {
        "k": k[0, 0].float().cpu().numpy().astype(np.float64),
        "v": v[0, 0].float().cpu().numpy().astype(np.float64),
        "q_rows": qr.reshape(nb, 16, cfg.Dqk),
        "rows": rows[:nb],
        "group": group,
    }


def cpu_baseline(cfg, sample, budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of a prefill workload:
    query rows of KV group 0 (batch 0) at seeded uniform positions, each against its
    full causal key range. Rate = algorithmic FLOPs of those rows / oracle time; the
    full workload's oracle time is extrapolated at that rate."""
    import numpy as np

    import oracle

    q0 = cfg.q_part0 * cfg.Sp
    rows_done, flops, elapsed = 0, 0, 0.0
    for b in range(sample["q_rows"].shape[0]):
        if elapsed >= budget_s:
            break
        rows = sample["rows"][b]
        pos = q0 + rows
        t0 = time.perf_counter()
        oracle.attention_rows(sample["q_rows"][b], pos, sample["k"], sample["v"], scale=cfg.scale,
                              causal=cfg.causal, k_pos0=0)
        elapsed += time.perf_counter() - t0
        vis = (pos + 1) if cfg.causal else np.full_like(pos, cfg.S)
        flops += int(2 * (cfg.Dqk + cfg.Dv) * int(vis.sum()))
        rows_done += len(rows)
    rate = flops / elapsed
    total = prefill_flops(cfg)
    group = sample["group"]
    return {
        "value": round(rate / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"{cfg.name}: {rows_done} query rows of KV group 0 (heads 0-{group - 1}, batch 0) at seeded "
                   f"uniform positions, each against its full causal key range; numpy float64 with the "
                   f"score rows materialised; {elapsed:.1f} s of oracle time"),
        "seconds": round(elapsed, 2),
        "flops": flops,
        "extrapolated_full_config_s": round(total / rate, 1),
        "extrapolated_note": (f"extrapolated, not measured: the workload's {total:.4e} algorithmic FLOP at the "
                              f"sample's measured rate"),
    }


def cpu_full_run(cfg, q, k, v):
    """The fp64 oracle over every row of a small prefill workload (its full run):
    oracle.attention on the whole query block against all keys."""
    import oracle

    qn, kn, vn = (x.float().cpu().numpy() for x in (q, k, v))
    t0 = time.perf_counter()
    oracle.attention(qn, kn, vn, scale=cfg.scale, causal=cfg.causal, q_pos0=cfg.q_part0 * cfg.Sp, k_pos0=0)
    elapsed = time.perf_counter() - t0
    flops = prefill_flops(cfg)
    return {
        "value": round(flops / elapsed / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": f"{cfg.name}: the full workload, every query row; numpy float64, score matrix materialised",
        "seconds": round(elapsed, 3),
        "flops": flops,
    }


def copy_calibration(torch, steps: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    n = 1 << 28   # 1 GiB of fp32
    src = torch.ones(n, dtype=torch.float32, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n * 4, "copy_bytes_written": n * 4, "launches": steps}), flush=True)


def run_decode(args, ra, torch, dev, stream, dcfg, decode_inputs_torch):
    """Time split-KV decode (partials + reduction) and the partial kernel alone."""
    log(f"[bench] generating {dcfg.name} inputs ({dcfg.description})")
    dq, dk, dvv = decode_inputs_torch(dcfg, dev)
    if dcfg.kv_dtype == "fp8":
        from workloads import FP8_K_SCALE, FP8_V_SCALE
        dec = lambda: ra.splitkv_decode_fp8(dq, dk, dvv, k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE,
                                            n_splits=dcfg.n_splits, scale=dcfg.scale)
        part = lambda: ra.splitkv_partial_fp8(dq, dk, dvv, k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE,
                                              n_splits=dcfg.n_splits, scale=dcfg.scale, o_part=o_part,
                                              lse_part=lse_part)
        kname = f"decode_partial_kernel<{dcfg.Dqk},fp8>"
    else:
        dec = lambda: ra.splitkv_decode(dq, dk, dvv, n_splits=dcfg.n_splits, scale=dcfg.scale)
        part = lambda: ra.splitkv_partial(dq, dk, dvv, n_splits=dcfg.n_splits, scale=dcfg.scale,
                                          o_part=o_part, lse_part=lse_part)
        kname = f"decode_partial_kernel<{dcfg.Dqk}>"
    o_part = torch.empty((dcfg.B, dcfg.Hq, dcfg.n_splits, dcfg.Dv), dtype=torch.float32, device=dev)
    lse_part = torch.empty((dcfg.B, dcfg.Hq, dcfg.n_splits), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    nsteps = max(args.decode_steps, args.steps)
    log(f"[bench] decode: {max(args.warmup, 2)} warmup + {nsteps} timed steps")
    d_wall, d_ev = timed(dec, nsteps, max(args.warmup, 2), stream, torch)
    per = []
    p_wall, p_ev = timed(part, nsteps, max(args.warmup, 2), stream, torch, per)
    tot_bytes = decode_total_bytes(dcfg)
    part_bytes = decode_partial_bytes(dcfg)
    d_value = tot_bytes / (d_wall * 1e-3) / 1e9
    p_ach = part_bytes / (p_ev * 1e-3) / 1e9
    log(f"[bench] decode {d_wall:.4f} ms/step ({d_value:.0f} GB/s); partial kernel {p_ev:.4f} ms "
        f"({p_ach:.0f} GB/s)")
    del dq, dk, dvv
    torch.cuda.empty_cache()
    return {
        "workload": f"{dcfg.name}: {dcfg.description}",
        "value": round(d_value, 2),
        "unit": "GB/s",
        "ms_per_step": round(d_wall, 5),
        "steps": nsteps,
        "algorithmic_bytes_per_step": tot_bytes,
        "roofline": {
            "kernel": kname,
            "bound": "hbm",
            "achieved": round(p_ach, 2),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(p_ach / PEAK_HBM_GBPS, 4),
            "traffic": recorded_traffic("decode", dcfg.name),
            "algorithmic_bytes_per_launch": part_bytes,
            "launch_ms": round(p_ev, 5),
            "launch_ms_stats": launch_stats(per),
        },
    }


PEAK_FP32_TFLOPS = 157.3   # MI355X fp32 (published: dense matrix, and vector with packed math)


def _f32_wide_workload():
    from workloads import PrefillConfig
    return PrefillConfig(name="F32B", dtype="f32", causal=True, B=1, Hq=8, Hkv=2, Sp=2048, P=4, Dqk=128, Dv=128,
                         seed=1300, description="fp32, causal, GQA 8:2, S 8192 = 4 x 2048, d 128")


F32B = _f32_wide_workload()


def prefill_line(args, ra, torch, stream, cfg, q, k, v, steps, warmup):
    """Times `steps` ring prefill launches of a workload (after `warmup` untimed
    ones) and returns its measurement: wall ms per step, per-launch ms from HIP
    events on the launch stream, algorithmic rate and its roofline fraction."""
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = torch.empty((cfg.B, cfg.Hq, cfg.Sq, cfg.Dv), dtype=dt, device=q.device)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.Sq), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()

    def step():
        ra.ring_attn_fwd(q, k, v, P=cfg.P, causal=cfg.causal, scale=cfg.scale, q_part0=cfg.q_part0,
                         out=out, lse=lse)

    log(f"[bench] {cfg.name} prefill: {warmup} warmup + {steps} timed steps")
    per = []
    wall_ms, ev_ms = timed(step, steps, warmup, stream, torch, per)
    flops = prefill_flops(cfg)
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (ev_ms * 1e-3) / 1e12
    log(f"[bench] {cfg.name} prefill {wall_ms:.4f} ms/step wall, {ev_ms:.4f} ms/launch events, "
        f"{value:.1f} TFLOP/s")
    del out, lse
    if cfg.dtype == "bf16":
        roof = {"kernel": f"prefill_bf16_kernel<{cfg.Dqk},{cfg.Dv},ring>", "bound": "mfma",
                "peak": PEAK_BF16_TFLOPS, "traffic": recorded_traffic("prefill", cfg.name)}
    else:
        # fp32 inputs run on the fp32 matrix cores (v_mfma_f32_32x32x2_f32 or
        # 16x16x4, by launch size), whose dense peak is the fp32 figure
        roof = {"kernel": f"prefill_f32_kernel<{cfg.Dqk},{cfg.Dv},ring>", "bound": "mfma",
                "peak": PEAK_FP32_TFLOPS, "traffic": None}
    roof.update({"achieved": round(achieved, 3), "unit": "TFLOP/s", "frac": round(achieved / roof["peak"], 4),
                 "algorithmic_flops_per_launch": flops, "launch_ms": round(ev_ms, 5),
                 "launch_ms_stats": launch_stats(per)})
    sclk = recorded(SCLK_FILE, "prefill", cfg.name, 1) if cfg.dtype == "bf16" else None
    if sclk is not None:
        # the clock is a property of the box and its load: recorded on one box, it
        # rescales this run's peak only approximately
        peak_at = MFMA_BF16_FLOP_PER_CLK * sclk[0] * 1e9 / 1e12
        roof.update({"sclk_ghz_recorded": sclk[0], "peak_at_sclk": round(peak_at, 1),
                     "frac_at_sclk": round(achieved / peak_at, 4)})
    return {
        "workload": f"{cfg.name}: {cfg.description}",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "steps": steps,
        "ms_per_step": round(wall_ms, 5),
        "roofline": roof,
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="C4", choices=["C2", "C3", "C4"],
                    help="headline prefill workload (default: C4, the largest that fits one GPU)")
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--small-steps", type=int, default=50, help="timed steps of the small workloads C1 and C2")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="decode only (for kernel profiling)")
    ap.add_argument("--no-secondary", action="store_true",
                    help="headline prefill only: no C3/C2/C1 lines, no striped, ring-step or backward runs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=12.0, help="seconds of oracle work on the headline")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-striped", action="store_true", help="skip the striped-layout measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-cache decode measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--decode-workload", default="C5", choices=["C5", "C5F"],
                    help="decode workload of a --no-prefill run")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: the library has no multi-GPU path "
              f"(--gpus {args.gpus} requested)", file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import blockwise_exact_attention_block_amd as ra
    from workloads import CONFIGS, decode_inputs_fp8_torch, decode_inputs_torch, prefill_inputs_torch

    if args.copy_calibration:
        copy_calibration(torch, max(args.steps, 1))
        return

    dev = torch.device("cuda:0")
    ra.load_library()
    stream = torch.cuda.current_stream(dev)

    if args.no_prefill:
        args.no_cpu_baseline = True
        dcfg = CONFIGS[args.decode_workload]
        gen = decode_inputs_fp8_torch if dcfg.kv_dtype == "fp8" else decode_inputs_torch
        line = run_decode(args, ra, torch, dev, stream, dcfg, gen)
        print(json.dumps(line), flush=True)
        return

    cfg = CONFIGS[args.workload]
    samples = {}      # host copies for the oracle, taken while the inputs are resident
    small_inputs = {}

    # ---- headline: the ring prefill of the chosen workload ------------------------
    log(f"[bench] generating {cfg.name} inputs ({cfg.description})")
    q, k, v = prefill_inputs_torch(cfg, dev)
    head = prefill_line(args, ra, torch, stream, cfg, q, k, v, args.steps, args.warmup)
    line = {
        "metric": "causal prefill attn TFLOP/s (% MFMA peak); decode KV GB/s (% HBM) on 1 MI355X",
        "value": head["value"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": f"{cfg.name}: {cfg.description}",
            "global_batch": cfg.B,
            "seq_len": cfg.S,
            "query_partitions": f"{cfg.q_part0}..{cfg.q_part0 + cfg.n_qparts - 1} of {cfg.P}",
            "heads_q_kv": [cfg.Hq, cfg.Hkv],
            "head_dims_qk_v": [cfg.Dqk, cfg.Dv],
            "causal": cfg.causal,
            "parallelism": "single GPU; the ring's KV blocks are visited in ring order inside one launch",
        },
        "roofline": head["roofline"],
    }
    if not args.no_cpu_baseline:
        samples[cfg.name] = oracle_sample_inputs(cfg, q, k, v)
    if cfg.name == "C3" and not args.no_secondary:
        run_c3_extras(args, ra, torch, stream, cfg, q, k, v, line)
    elif not args.no_backward:
        line["backward_" + cfg.name] = guarded("backward", run_backward, args, ra, torch, stream, cfg, q, k, v)
    del q, k, v
    torch.cuda.empty_cache()

    # ---- the other prefill workloads, each with a line of its own -----------------
    if not args.no_secondary:
        line["prefill_other"] = {}
        for name in ("C3", "C2", "C1"):
            if name == cfg.name:
                continue
            c = CONFIGS[name]
            log(f"[bench] generating {c.name} inputs ({c.description})")
            q, k, v = prefill_inputs_torch(c, dev)
            small = name in ("C1", "C2")
            steps = max(args.small_steps, args.steps) if small else args.steps
            line["prefill_other"][name] = guarded(name, prefill_line, args, ra, torch, stream, c, q, k, v, steps,
                                                  max(args.warmup, 2))
            if not args.no_cpu_baseline:
                if small:
                    small_inputs[name] = tuple(x.cpu() for x in (q, k, v))
                else:
                    samples[name] = oracle_sample_inputs(c, q, k, v)
            if name == "C3":
                run_c3_extras(args, ra, torch, stream, c, q, k, v, line)
            elif name == "C1" and not args.no_backward:
                line["backward_C1"] = guarded("backward C1", run_backward, args, ra, torch, stream, c, q, k, v)
            del q, k, v
            torch.cuda.empty_cache()
            if name == "C1" and not args.no_backward:
                # C1 (one head, 1024 rows) is far too small to load the chip, so the
                # fp32 prefill and backward are also timed on a GQA sequence of 8192
                # tokens
                log(f"[bench] generating {F32B.name} inputs ({F32B.description})")
                q, k, v = prefill_inputs_torch(F32B, dev)
                line["prefill_other"][F32B.name] = guarded(F32B.name, prefill_line, args, ra, torch, stream,
                                                              F32B, q, k, v, args.steps, max(args.warmup, 2))
                line["backward_f32"] = guarded("backward f32", run_backward, args, ra, torch, stream, F32B, q,
                                               k, v)
                del q, k, v
                torch.cuda.empty_cache()

    # ---- decode ----------------------------------------------------------------------
    if not args.no_decode:
        line["decode"] = guarded("decode", run_decode, args, ra, torch, dev, stream, CONFIGS["C5"],
                                 decode_inputs_torch)
        if not args.no_fp8:
            fp8 = guarded("fp8 decode", run_decode, args, ra, torch, dev, stream, CONFIGS["C5F"],
                          decode_inputs_fp8_torch)
            if "error" not in fp8 and "error" not in line["decode"]:
                fp8["speedup_vs_bf16_cache"] = round(line["decode"]["ms_per_step"] / fp8["ms_per_step"], 3)
            line["decode_fp8"] = fp8

    # ---- the fp64 oracle on the host, after every GPU measurement -------------------
    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: fp64 oracle for ~{args.cpu_budget:.0f} s on {cfg.name}")
        line["cpu_baseline"] = guarded("cpu baseline", cpu_baseline, cfg, samples.pop(cfg.name), args.cpu_budget)
        others = {}
        for name, smp in samples.items():
            log(f"[bench] cpu baseline: fp64 oracle for ~{args.cpu_budget / 2:.0f} s on {name}")
            others[name] = guarded(f"cpu baseline {name}", cpu_baseline, CONFIGS[name], smp, args.cpu_budget / 2)
        for name, (q, k, v) in small_inputs.items():
            log(f"[bench] cpu baseline: fp64 oracle over all of {name}")
            others[name] = guarded(f"cpu baseline {name}", cpu_full_run, CONFIGS[name], q, k, v)
        if others:
            line["cpu_baseline"]["other_workloads"] = others

    print(json.dumps(line), flush=True)


def run_c3_extras(args, ra, torch, stream, cfg, q, k, v, line):
    """The striped layout, one ring step through the step API and the backward pass,
    on the 70B-class GQA workload."""
    if not args.no_striped and cfg.causal:
        line["striped"] = guarded("striped", run_striped, args, ra, torch, stream, cfg, q, k, v)
    step = guarded("ring step", run_ring_step, args, ra, torch, stream, cfg, q, k, v)
    if step is not None:
        line["ring_step"] = step
    if not args.no_backward:
        bwd = guarded("backward", run_backward, args, ra, torch, stream, cfg, q, k, v)
        if bwd is not None:
            line["backward"] = bwd


if __name__ == "__main__":
    main()
