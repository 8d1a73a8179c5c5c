"""Byte and FLOP accounting from the pages' own formulas (test infrastructure).

Each helper is pinned against a table the pages print (tests/golden/).
"""
from __future__ import annotations


def kv_cache_bytes(layers: int, h_kv: int, d_h: int, n: int, bytes_per_value: int, batch: int = 1) -> int:
    """KV cache size M = 2 * L * H_kv * d_h * n * b, per sequence, times batch; the 2
    counts K and V ([CH] §挑战 2, eq. lc-ch-kv-memory and the symbol table below it)."""
    return 2 * layers * h_kv * d_h * n * bytes_per_value * batch


def decode_lower_bound_s(kv_bytes: float, hbm_bytes_per_s: float) -> float:
    """Per-token decode attention time if it only has to stream the KV cache once:
    KV bytes / HBM bandwidth ([CH] §KV 是 Decode 阶段的隐性瓶颈 and its table
    tbl-longctx-challenge-decode-bw)."""
    return kv_bytes / hbm_bytes_per_s


def prefill_compute_time_s(B: int, S: int, Dqk: int, Dv: int, cp: int, R: float) -> float:
    """T_comp = 2 B S^2 (D_qk + D_v) / (cp R) ([CPEV] §Prefill：加速来自计算按 cp 均分,
    eq. cpeval-comp). One head, every (query, key) pair counted (no causal mask)."""
    return 2.0 * B * S * S * (Dqk + Dv) / (cp * R)


def visible_pairs_aligned_causal(S: int) -> int:
    """Number of (query, key) pairs with key <= query in one causal sequence of S tokens."""
    return S * (S + 1) // 2


def visible_pairs_partition(Sp: int, P: int, i: int, causal: bool, layout: str = "contiguous") -> int:
    """Visible pairs for query partition i of a ring of P partitions of Sp tokens,
    summed over the ring schedule.

    Contiguous: blocks before i are full (Sp^2), block i is the causal triangle
    with its diagonal, later blocks are skipped. Striped (partition p holds
    positions p, p+P, ...): key c of block j is visible to local query row r iff
    c*P + j <= r*P + i, i.e. c <= r when j <= i and c < r when j > i, so a block
    holds the triangle with its diagonal (Sp(Sp+1)/2 pairs) or without it
    (Sp(Sp-1)/2)."""
    from .exact import ring_schedule
    total = 0
    for j, kind in ring_schedule(P, i, causal, layout):
        if kind == "full":
            total += Sp * Sp
        elif kind == "diag":
            if layout == "striped" and j > i:
                total += Sp * (Sp - 1) // 2
            else:
                total += Sp * (Sp + 1) // 2
    return total


def attention_flops(pairs_per_head: int, heads: int, Dqk: int, Dv: int) -> int:
    """2 (D_qk + D_v) FLOPs per visible (query, key) pair: one multiply-add per
    element of the score dot product and one per element of the PV update
    ([CH] §挑战 1 complexity table: the dominant O(n^2 d) terms are QK^T and PV)."""
    return 2 * (Dqk + Dv) * pairs_per_head * heads
