#!/usr/bin/env python3
"""One-GPU benchmark of the ring-ordered blockwise exact attention hot path (MI355X).

Headline (``value``): causal ring prefill throughput in algorithmic TFLOP/s (only
visible query/key pairs count, 2 (D_qk + D_v) FLOP each) on the 70B-class GQA
workload: B 1, 64 query heads over 8 KV heads, S = 131072 cut into 8 ring
partitions of 16384, d 128, bf16 -- every partition's queries visiting the KV
blocks in ring order, in one launch. A step is one such launch over the whole
sequence; inputs are resident in HBM before the timed region.

The same JSON line carries:
  decode        split-KV decode (B 16, 64/8 heads, KV length 131072 in 8 splits,
                bf16) in HBM GB/s of algorithmic bytes;
  roofline      for each dominant kernel: algorithmic work per launch over its
                average launch time, taken with HIP events on the launch stream
                during the timed region, against the MI355X peak (bf16 dense MFMA
                2.5 PFLOP/s; HBM 8 TB/s), and the HBM traffic from rocprofv3
                counters when they were taken on the current kernel source;
  cpu_baseline  the fp64 CPU oracle on a bounded sample of the same workload,
                timed on this host's cores.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload C3|C2|C4]
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


def recorded_traffic(kind: str, workload: str):
    """HBM bytes per launch measured by rocprofv3 counters (FETCH_SIZE + WRITE_SIZE,
    scaled by the copy-kernel calibration), if recorded for this exact source."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    sha = source_sha(kind)
    with open(TRAFFIC_FILE) as f:
        for line in f:
            parts = line.split("#", 1)[0].split()
            if len(parts) == 5 and parts[0] == kind and parts[1] == workload and parts[2] == sha:
                return float(parts[3]) + float(parts[4])
    return None


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
    """Whole-sequence backward of the prefill workload: delta preprocess plus one
    step over all (query partition, KV block) pairs, fp32 gradients."""
    if cfg.q_part0 != 0 or cfg.n_qparts != cfg.P:
        return None
    out, lse = ra.ring_attn_fwd(q, k, v, P=cfg.P, causal=cfg.causal, scale=cfg.scale)
    dout = torch.empty_like(out).normal_(0.0, 1.0, generator=torch.Generator(device=q.device).manual_seed(cfg.seed + 7))
    delta = ra.attn_bwd_preprocess(out, dout)
    dq = torch.zeros(q.shape, dtype=torch.float32, device=q.device)
    dk = torch.zeros(k.shape, dtype=torch.float32, device=q.device)
    dv = torch.zeros(v.shape, dtype=torch.float32, device=q.device)
    steps, warm = max(2, min(args.steps, 3)), 1
    log(f"[bench] backward: {warm} warmup + {steps} timed steps")

    def step():
        ra.attn_bwd_preprocess(out, dout, delta)
        ra.block_attn_bwd_step(q, dout, lse, delta, k, v, dq, dk, dv, q_pos0=0, k_pos0=0, causal=cfg.causal,
                               scale=cfg.scale)

    wall, ev = timed(step, steps, warm, stream, torch)
    flops = backward_flops(cfg)
    log(f"[bench] backward {wall:.3f} ms/step, {flops / (wall * 1e-3) / 1e12:.1f} TFLOP/s (algorithmic)")
    del out, lse, dout, delta, dq, dk, dv
    torch.cuda.empty_cache()
    return {
        "workload": f"{cfg.name} backward (delta + dK/dV + dQ over all pairs, fp32 gradients)",
        "ms_per_step": round(wall, 4),
        "launch_ms": round(ev, 4),
        "algorithmic_flops": flops,
        "tflops": round(flops / (wall * 1e-3) / 1e12, 2),
        "frac_of_bf16_peak": round(flops / (wall * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
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


def timed(fn, steps, warmup, stream, torch):
    """Run warmup untimed steps, then exactly `steps` timed ones bracketed by full
    synchronisation; returns (wall ms per step, mean per-launch ms from events)."""
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
    ev_ms = sum(s.elapsed_time(e) for s, e in zip(starts, ends)) / steps
    return wall_ms, ev_ms


def blas_threads() -> int:
    try:
        from threadpoolctl import threadpool_info
        n = [d.get("num_threads", 0) for d in threadpool_info() if d.get("user_api") == "blas"]
        if n:
            return int(max(n))
    except Exception:
        pass
    return len(os.sched_getaffinity(0))


def cpu_baseline(cfg, q, k, v, budget_s: float):
    """The fp64 oracle, as it stands, on a bounded sample of the prefill workload:
    query rows of KV group 0 (batch 0) at seeded uniform positions, each against its
    full causal key range. Rate = algorithmic FLOPs of those rows / oracle time."""
    import numpy as np
    import torch

    import oracle

    rng = np.random.default_rng(cfg.seed + 99)
    group = cfg.Hq // cfg.Hkv
    k_np = k[0, 0].float().cpu().numpy()
    v_np = v[0, 0].float().cpu().numpy()
    q0 = cfg.q_part0 * cfg.Sp
    rows_done, flops, elapsed, batches = 0, 0, 0.0, 0
    while elapsed < budget_s and batches < 4096:
        heads = rng.integers(0, group, size=16)
        rows = rng.integers(0, cfg.Sq, size=16)
        qr = q[0, torch.as_tensor(heads), torch.as_tensor(rows)].float().cpu().numpy()
        pos = q0 + rows
        t0 = time.perf_counter()
        oracle.attention_rows(qr, pos, k_np, v_np, scale=cfg.scale, causal=cfg.causal, k_pos0=0)
        elapsed += time.perf_counter() - t0
        vis = (pos + 1) if cfg.causal else np.full_like(pos, cfg.S)
        flops += int(2 * (cfg.Dqk + cfg.Dv) * int(vis.sum()))
        rows_done += 16
        batches += 1
    return {
        "value": round(flops / elapsed / 1e12, 6),
        "unit": "TFLOP/s",
        "cores": blas_threads(),
        "kind": "oracle",
        "sample": (f"{cfg.name}: {rows_done} query rows of KV group 0 (heads 0-{group - 1}, batch 0) at seeded "
                   f"uniform positions, each against its full causal key range; numpy float64 with the "
                   f"score rows materialised; {elapsed:.1f} s of oracle time"),
        "seconds": round(elapsed, 2),
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
    p_wall, p_ev = timed(part, nsteps, max(args.warmup, 2), stream, torch)
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
        },
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="C3", choices=["C2", "C3", "C4"])
    ap.add_argument("--decode-steps", type=int, default=50)
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-prefill", action="store_true", help="decode only (for kernel profiling)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0, help="seconds of oracle work")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--no-striped", action="store_true", help="skip the striped-layout measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the fp8-cache decode measurement")
    ap.add_argument("--no-backward", action="store_true", help="skip the backward-pass measurement")
    ap.add_argument("--decode-workload", default="C5", choices=["C5", "C5F"],
                    help="decode workload of a --no-prefill run")
    args = ap.parse_args()

    if args.gpus != 1:
        print(f"bench.py measures one GPU only: this build has no multi-GPU path "
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
    cfg = CONFIGS[args.workload]

    line = {}
    if args.no_prefill:
        args.no_cpu_baseline = True
        dcfg = CONFIGS[args.decode_workload]
        gen = decode_inputs_fp8_torch if dcfg.kv_dtype == "fp8" else decode_inputs_torch
        line = run_decode(args, ra, torch, dev, stream, dcfg, gen)
        print(json.dumps(line), flush=True)
        return

    log(f"[bench] generating {cfg.name} inputs ({cfg.description})")
    q, k, v = prefill_inputs_torch(cfg, dev)
    out = torch.empty((cfg.B, cfg.Hq, cfg.Sq, cfg.Dv), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.Sq), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step():
        ra.ring_attn_fwd(q, k, v, P=cfg.P, causal=cfg.causal, scale=cfg.scale, q_part0=cfg.q_part0,
                         out=out, lse=lse)

    log(f"[bench] prefill: {args.warmup} warmup + {args.steps} timed steps")
    wall_ms, ev_ms = timed(step, args.steps, args.warmup, stream, torch)
    flops = prefill_flops(cfg)
    value = flops / (wall_ms * 1e-3) / 1e12
    achieved = flops / (ev_ms * 1e-3) / 1e12
    log(f"[bench] prefill {wall_ms:.3f} ms/step wall, {ev_ms:.3f} ms/launch events, {value:.1f} TFLOP/s")
    traffic = recorded_traffic("prefill", cfg.name)
    line = {
        "metric": "causal prefill attn TFLOP/s (% MFMA peak); decode KV GB/s (% HBM) on 1 MI355X",
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 4),
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
            "parallelism": "single GPU; the P ring partitions are query partitions of one launch",
        },
        "roofline": {
            "kernel": f"prefill_bf16_kernel<{cfg.Dqk},{cfg.Dv},ring>",
            "bound": "mfma",
            "achieved": round(achieved, 3),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "algorithmic_flops_per_launch": flops,
            "launch_ms": round(ev_ms, 4),
        },
    }
    del out, lse
    if not args.no_striped and cfg.causal:
        line["striped"] = run_striped(args, ra, torch, stream, cfg, q, k, v)
    step = run_ring_step(args, ra, torch, stream, cfg, q, k, v)
    if step is not None:
        line["ring_step"] = step
    if not args.no_backward:
        bwd = run_backward(args, ra, torch, stream, cfg, q, k, v)
        if bwd is not None:
            line["backward"] = bwd

    if not args.no_decode:
        # the prefill inputs are dropped to make room and regenerated (same seeds) below
        del q, k, v
        torch.cuda.empty_cache()
        line["decode"] = run_decode(args, ra, torch, dev, stream, CONFIGS["C5"], decode_inputs_torch)
        if not args.no_fp8:
            fp8 = run_decode(args, ra, torch, dev, stream, CONFIGS["C5F"], decode_inputs_fp8_torch)
            fp8["speedup_vs_bf16_cache"] = round(line["decode"]["ms_per_step"] / fp8["ms_per_step"], 3)
            line["decode_fp8"] = fp8
        if not args.no_cpu_baseline:
            q, k, v = prefill_inputs_torch(cfg, dev)

    if not args.no_cpu_baseline:
        log(f"[bench] cpu baseline: fp64 oracle for ~{args.cpu_budget:.0f} s")
        line["cpu_baseline"] = cpu_baseline(cfg, q, k, v, args.cpu_budget)

    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
