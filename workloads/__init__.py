"""Synthetic workloads: the configurations and their seeded input generators.

This module holds shapes, seeds and random-number draws only. It computes no part
of attention, so both the fp64 oracle side (tests, cpu baseline) and the GPU side
(tests, bench) may take their inputs from it without sharing any arithmetic.

Citation keys used in this file:
  [RING]  page "AI 推理系列（十一）：Ring Attention 如何让多张 GPU 共同计算一条超长序列"
  [CH]    page "长上下文的第一性挑战"
  [CPEV]  page "上下文并行 (CP) 收益评估实验设计"

Inputs are i.i.d. N(0,1). bf16 configurations draw directly in bf16 on the device
(round-to-nearest-even of an fp32 draw); the oracle then reads back the stored
values, so parity never depends on how the draw is made.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, List, Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class PrefillConfig:
    """A ring prefill workload on one GPU.

    The sequence of S = P * Sp tokens is cut into P contiguous partitions ([RING]
    §"KV 在 Ring 中如何流动": every device keeps its own query block while the KV
    blocks travel round a logical ring). On one GPU the P "devices" are query
    partitions; `q_part0`/`nq` select which partitions' queries are computed
    (all of them, or one device's share).
    """
    name: str
    dtype: str          # "f32" or "bf16"
    causal: bool
    B: int
    Hq: int
    Hkv: int
    Sp: int             # tokens per partition
    P: int              # ring size (partitions / KV blocks)
    Dqk: int
    Dv: int
    q_part0: int = 0
    nq: Optional[int] = None   # number of query partitions computed (default: P)
    seed: int = 0
    check_rows: Optional[int] = None   # sampled rows for the oracle (None = all rows)
    description: str = ""

    @property
    def n_qparts(self) -> int:
        return self.P if self.nq is None else self.nq

    @property
    def S(self) -> int:
        return self.P * self.Sp

    @property
    def Sq(self) -> int:
        return self.n_qparts * self.Sp

    @property
    def scale(self) -> float:
        # softmax(QK^T / sqrt(d_k)) V  ([CH] §挑战 1, eq. lc-ch-attention)
        return 1.0 / math.sqrt(self.Dqk)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    """Split-KV ("pass-Q") decode: one new query token per sequence; the KV cache
    of length L is cut into n_splits contiguous chunks, each producing a partial
    (O, LSE) that a log-sum-exp weighted reduction merges ([CPEV] §名词定义,
    pass-KV / pass-Q; §Decode：cp 只解容量、不省计算)."""
    name: str
    dtype: str
    B: int
    Hq: int
    Hkv: int
    L: int
    Dqk: int
    Dv: int
    n_splits: int
    seed: int = 0
    description: str = ""
    kv_dtype: str = "bf16"      # "fp8": e4m3 cache with per-tensor K / V scales

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.Dqk)


CONFIGS: Dict[str, object] = {
    "C1": PrefillConfig(
        name="C1", dtype="f32", causal=False, B=1, Hq=1, Hkv=1, Sp=256, P=4,
        Dqk=64, Dv=64, seed=1000,
        description="non-causal single head, S=1024 in 4 ring partitions of 256, d=64, fp32"),
    "C2": PrefillConfig(
        name="C2", dtype="bf16", causal=True, B=1, Hq=8, Hkv=8, Sp=2048, P=4,
        Dqk=128, Dv=128, seed=2000,
        description="causal MHA, H=8, S=8192 in 4 partitions of 2048, d=128, bf16"),
    "C3": PrefillConfig(
        name="C3", dtype="bf16", causal=True, B=1, Hq=64, Hkv=8, Sp=16384, P=8,
        Dqk=128, Dv=128, seed=3000, check_rows=4096,
        description="causal GQA 64/8 (70B-class layer), S=131072 in 8 partitions, d=128, bf16"),
    "C4": PrefillConfig(
        name="C4", dtype="bf16", causal=True, B=1, Hq=128, Hkv=128, Sp=65536, P=8,
        Dqk=192, Dv=128, q_part0=7, nq=1, seed=4000, check_rows=2048,
        description="MLA-shaped causal share: query partition 7 of 8 (65536 tokens) of "
                    "S=524288, 128 heads, D_qk=192, D_v=128, bf16, all 8 KV blocks"),
    "C5": DecodeConfig(
        name="C5", dtype="bf16", B=16, Hq=64, Hkv=8, L=131072, Dqk=128, Dv=128,
        n_splits=8, seed=5000,
        description="split-KV decode, B=16, 64/8 heads, KV length 131072 in 8 splits, bf16"),
    "C5F": DecodeConfig(
        name="C5F", dtype="bf16", B=16, Hq=64, Hkv=8, L=131072, Dqk=128, Dv=128,
        n_splits=8, seed=5500, kv_dtype="fp8",
        description="split-KV decode over an fp8 e4m3 KV cache, B=16, 64/8 heads, KV length 131072 "
                    "in 8 splits, bf16 query"),
}

# per-tensor dequantisation scales of the synthetic fp8 caches (key = K_SCALE * code)
FP8_K_SCALE = 0.25
FP8_V_SCALE = 0.5


# ----------------------------------------------------------------------------------
# numpy generators (CPU side: oracle pins and small parity cases)
# ----------------------------------------------------------------------------------

def _bf16_round_np(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even), returned as fp32."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    lsb = (u >> 16) & 1
    r = (u + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return r.view(np.float32)


def randn_np(shape, seed: int, dtype: str = "f32") -> np.ndarray:
    """Seeded i.i.d. N(0,1) array (fp32 values, bf16-representable when dtype='bf16')."""
    g = np.random.default_rng(seed)
    x = g.standard_normal(size=shape, dtype=np.float32)
    if dtype == "bf16":
        x = _bf16_round_np(x)
    return x


def prefill_inputs_np(B, Hq, Hkv, Sq, Sk, Dqk, Dv, seed, dtype="f32"):
    """Q [B,Hq,Sq,Dqk], K [B,Hkv,Sk,Dqk], V [B,Hkv,Sk,Dv] from seeds seed+1..+3."""
    q = randn_np((B, Hq, Sq, Dqk), seed + 1, dtype)
    k = randn_np((B, Hkv, Sk, Dqk), seed + 2, dtype)
    v = randn_np((B, Hkv, Sk, Dv), seed + 3, dtype)
    return q, k, v


# ----------------------------------------------------------------------------------
# torch generators (device side)
# ----------------------------------------------------------------------------------

def _torch_dtype(name: str):
    import torch
    return {"f32": torch.float32, "bf16": torch.bfloat16}[name]


def randn_torch(shape, seed: int, dtype: str, device) -> "torch.Tensor":
    """Seeded N(0,1) drawn on `device` in the target dtype, in slabs along dim 0..1 so
    that large bf16 tensors never need an fp32 copy of themselves."""
    import torch
    t = torch.empty(shape, dtype=_torch_dtype(dtype), device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    flat = t.view(-1, *shape[2:]) if len(shape) > 2 else t.view(1, -1)
    for i in range(flat.shape[0]):
        flat[i].normal_(0.0, 1.0, generator=gen)
    return t


def prefill_inputs_torch(cfg: PrefillConfig, device):
    """Device tensors for a prefill config: q holds only the computed query
    partitions, k/v hold all P blocks, contiguous BHSD."""
    q = randn_torch((cfg.B, cfg.Hq, cfg.Sq, cfg.Dqk), cfg.seed + 1, cfg.dtype, device)
    k = randn_torch((cfg.B, cfg.Hkv, cfg.S, cfg.Dqk), cfg.seed + 2, cfg.dtype, device)
    v = randn_torch((cfg.B, cfg.Hkv, cfg.S, cfg.Dv), cfg.seed + 3, cfg.dtype, device)
    return q, k, v


def fp8_cache_torch(shape, seed: int, device) -> "torch.Tensor":
    """Seeded fp8 e4m3 cache: N(0,1) drawn in bf16 slab by slab and cast to
    torch.float8_e4m3fn (round to nearest even; no draw comes near 448)."""
    import torch
    t = torch.empty(shape, dtype=torch.float8_e4m3fn, device=device)
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    flat = t.view(-1, *shape[2:])
    tmp = torch.empty(flat.shape[1:], dtype=torch.bfloat16, device=device)
    for i in range(flat.shape[0]):
        tmp.normal_(0.0, 1.0, generator=gen)
        flat[i].copy_(tmp)
    return t


def decode_inputs_fp8_torch(cfg: DecodeConfig, device):
    """bf16 query, fp8 K and V caches (dequantised by FP8_K_SCALE / FP8_V_SCALE)."""
    q = randn_torch((cfg.B, cfg.Hq, cfg.Dqk), cfg.seed + 1, cfg.dtype, device)
    k = fp8_cache_torch((cfg.B, cfg.Hkv, cfg.L, cfg.Dqk), cfg.seed + 2, device)
    v = fp8_cache_torch((cfg.B, cfg.Hkv, cfg.L, cfg.Dv), cfg.seed + 3, device)
    return q, k, v


def decode_inputs_torch(cfg: DecodeConfig, device):
    q = randn_torch((cfg.B, cfg.Hq, cfg.Dqk), cfg.seed + 1, cfg.dtype, device)
    k = randn_torch((cfg.B, cfg.Hkv, cfg.L, cfg.Dqk), cfg.seed + 2, cfg.dtype, device)
    v = randn_torch((cfg.B, cfg.Hkv, cfg.L, cfg.Dv), cfg.seed + 3, cfg.dtype, device)
    return q, k, v


# ----------------------------------------------------------------------------------
# row sampling for parity checks on large configs
# ----------------------------------------------------------------------------------

def sample_rows(cfg: PrefillConfig, n: Optional[int] = None, tile: int = 256,
                seed: Optional[int] = None) -> List[tuple]:
    """(b, h, r) query rows to check, r indexing the computed query tensor.

    All rows when n is None. Otherwise a seeded uniform sample plus forced rows:
    row 0, the first and last row of every computed partition, and rows on either
    side of every `tile` boundary inside the first and last partition.
    """
    Sq = cfg.Sq
    if n is None:
        return [(b, h, r) for b in range(cfg.B) for h in range(cfg.Hq) for r in range(Sq)]
    g = np.random.default_rng(cfg.seed + 4 if seed is None else seed)
    rows = set()
    for p in range(cfg.n_qparts):
        base = p * cfg.Sp
        for r in (base, base + 1, base + cfg.Sp - 2, base + cfg.Sp - 1):
            rows.add((int(g.integers(cfg.B)), int(g.integers(cfg.Hq)), r))
    for p in {0, cfg.n_qparts - 1}:
        base = p * cfg.Sp
        for t in range(tile, cfg.Sp, tile * 7):
            for r in (base + t - 1, base + t):
                rows.add((int(g.integers(cfg.B)), int(g.integers(cfg.Hq)), r))
    while len(rows) < n:
        rows.add((int(g.integers(cfg.B)), int(g.integers(cfg.Hq)), int(g.integers(Sq))))
    return sorted(rows)
