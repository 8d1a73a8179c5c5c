"""Plain fp64 attention, merge, ring order and split-KV decode (test infrastructure).

Readings of the pages taken here (each listed with its reason in the design notes):
  * Causal visibility: key position <= query position, positions being global
    token indices; the diagonal is visible ([RING] §"KV 在 Ring 中如何流动":
    a query may not read future tokens).
  * Scale 1/sqrt(D_qk) applied to the scores; LSE is the natural log of the sum of
    exp(scaled score) ([CH] §挑战 1 eq. lc-ch-attention; [IMPL] §Ring Attention实现
    代码与通信重叠, where lse is built from the scaled weights).
  * GQA: query head h reads KV head h // (Hq / Hkv).
  * A row with no visible key has O = 0 and LSE = -inf; merging with such a row
    is the identity ([IMPL] code initialises out = 0, lse = -inf).
"""
from __future__ import annotations

import math
from typing import List, Sequence, Tuple

import numpy as np

NEG_INF = -np.inf


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible(q_pos: np.ndarray, k_pos: np.ndarray, causal: bool) -> np.ndarray:
    """Boolean [Sq, Sk]: may query at q_pos[r] read key at k_pos[c]?

    Non-causal: every key. Causal: keys at or before the query's own position
    ([RING] §"KV 在 Ring 中如何流动", causal semantics must survive sharding).
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    if not causal:
        return np.ones((q_pos.size, k_pos.size), dtype=bool)
    return k_pos[None, :] <= q_pos[:, None]


def _softmax_rows(s: np.ndarray, vis: np.ndarray, v: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Given materialised scaled scores s [R, Sk] and visibility, return
    O [R, Dv] = softmax(s) V over visible keys, and LSE [R] = log sum exp(s).

    The row maximum is subtracted before exponentiating only to keep exp() in
    range; LSE = m + log(sum exp(s - m)) is the same number ([CH] §挑战 1 defines
    P = softmax(S / sqrt(d_k)), O = P V)."""
    R = s.shape[0]
    Dv = v.shape[1]
    s = np.where(vis, s, -np.inf)
    any_vis = vis.any(axis=1)
    m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
    e = np.exp(s - m[:, None])                      # exp(-inf) = 0 for hidden keys
    denom = e.sum(axis=1)
    with np.errstate(divide="ignore"):
        lse = np.where(any_vis, m + np.log(np.where(any_vis, denom, 1.0)), -np.inf)
    p = np.where(any_vis[:, None], e / np.where(any_vis, denom, 1.0)[:, None], 0.0)
    o = p @ v if R else np.zeros((0, Dv))
    return o, lse


def attention(q, k, v, *, scale: float, causal: bool,
              q_pos0: int = 0, k_pos0: int = 0, q_pos=None, k_pos=None) -> Tuple[np.ndarray, np.ndarray]:
    """Exact attention of a query block against one KV block, fp64.

    q [B,Hq,Sq,Dqk], k [B,Hkv,Sk,Dqk], v [B,Hkv,Sk,Dv] (any float dtype; upcast
    to fp64 exactly). Query r sits at global position q_pos0 + r and key c at
    k_pos0 + c, unless explicit position arrays q_pos [Sq] / k_pos [Sk] are given.
    Returns O [B,Hq,Sq,Dv] and LSE [B,Hq,Sq], both fp64.

    This is softmax(scale * Q K^T) V with the full score matrix materialised for
    each (batch, head) ([CH] §挑战 1, eq. lc-ch-attention and the complexity table
    naming S = QK^T, P = softmax(S/sqrt(d_k)), O = PV).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Sq, Dqk = q.shape
    Bk, Hkv, Sk, Dk2 = k.shape
    assert Bk == B and Dk2 == Dqk and v.shape[:3] == (B, Hkv, Sk)
    assert Hq % Hkv == 0, "query heads must be a multiple of KV heads (GQA groups)"
    group = Hq // Hkv
    Dv = v.shape[3]
    qp = q_pos0 + np.arange(Sq) if q_pos is None else np.asarray(q_pos)
    kp = k_pos0 + np.arange(Sk) if k_pos is None else np.asarray(k_pos)
    assert qp.shape == (Sq,) and kp.shape == (Sk,)
    vis = visible(qp, kp, causal)
    o = np.zeros((B, Hq, Sq, Dv))
    lse = np.full((B, Hq, Sq), -np.inf)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            s = scale * (q[b, h] @ k[b, g].T)          # [Sq, Sk] materialised
            o[b, h], lse[b, h] = _softmax_rows(s, vis, v[b, g])
    return o, lse


def attention_rows(q_rows, q_pos, k, v, *, scale: float, causal: bool,
                   k_pos0: int = 0) -> Tuple[np.ndarray, np.ndarray]:
    """The same definition for a set of query rows that share one KV head.

    q_rows [R, Dqk] with global positions q_pos [R]; k [Sk, Dqk], v [Sk, Dv] with
    key c at k_pos0 + c. Returns O [R, Dv], LSE [R] in fp64. Used to check
    sampled rows of configurations too large for the full definition.
    """
    q_rows, k, v = _f64(q_rows), _f64(k), _f64(v)
    vis = visible(np.asarray(q_pos), k_pos0 + np.arange(k.shape[0]), causal)
    s = scale * (q_rows @ k.T)
    return _softmax_rows(s, vis, v)


def merge(o_a, lse_a, o_b, lse_b) -> Tuple[np.ndarray, np.ndarray]:
    """Combine two normalised partial results over disjoint key sets.

    With L = log(e^{L_a} + e^{L_b}), the combined output is
    e^{L_a - L} O_a + e^{L_b - L} O_b ([IMPL] §Ring Attention实现代码与通信重叠:
    the new lse and the two weights beta, gamma that rescale the old output and
    the block output; [RING] §最容易被忽略的细节: per-block results cannot simply
    be added, the normalisation must be carried across blocks).

    Written in the max-shifted form so that it stays finite; a side with
    LSE = -inf contributes nothing.
    """
    o_a, lse_a, o_b, lse_b = _f64(o_a), _f64(lse_a), _f64(o_b), _f64(lse_b)
    m = np.maximum(lse_a, lse_b)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    ea = np.exp(lse_a - m_safe)
    eb = np.exp(lse_b - m_safe)
    tot = ea + eb
    with np.errstate(divide="ignore"):
        lse = np.where(both_empty, -np.inf, m_safe + np.log(np.where(both_empty, 1.0, tot)))
    wa = np.where(both_empty, 0.0, ea / np.where(both_empty, 1.0, tot))
    wb = np.where(both_empty, 0.0, eb / np.where(both_empty, 1.0, tot))
    o = wa[..., None] * o_a + wb[..., None] * o_b
    return o, lse


def merge_n(o_parts, lse_parts) -> Tuple[np.ndarray, np.ndarray]:
    """n-way reduction of partials along axis -2 of o_parts [..., n, Dv] and the
    last axis of lse_parts [..., n]: L = log sum_p e^{L_p}, O = sum_p e^{L_p - L} O_p
    ([CPEV] §Decode：cp 只解容量、不省计算: partial attention on every chip, then a
    reduction)."""
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    m = lse_parts.max(axis=-1)
    empty = np.isneginf(m)
    m_safe = np.where(empty, 0.0, m)
    e = np.exp(lse_parts - m_safe[..., None])
    tot = e.sum(axis=-1)
    with np.errstate(divide="ignore"):
        lse = np.where(empty, -np.inf, m_safe + np.log(np.where(empty, 1.0, tot)))
    w = np.where(empty[..., None], 0.0, e / np.where(empty, 1.0, tot)[..., None])
    o = (w[..., None] * o_parts).sum(axis=-2)
    return o, lse


LAYOUTS = ("contiguous", "striped")


def partition_positions(P: int, Sp: int, p: int, layout: str = "contiguous") -> np.ndarray:
    """Global token positions held, in order, by partition p of P partitions of Sp
    tokens each.

    contiguous: p*Sp, ..., p*Sp + Sp - 1 -- each device keeps one consecutive slice
    ([RING] opening example: 128K tokens on 4 GPUs, 32K consecutive tokens each).
    striped: p, p + P, p + 2P, ... -- positions dealt round-robin to the devices,
    the striped variant of ring attention, which interleaves positions so that
    under a causal mask every device has visible keys in every ring step
    ([IMPL] §长文本场景下的性能表现与调优).
    """
    if layout == "contiguous":
        return p * Sp + np.arange(Sp, dtype=np.int64)
    if layout == "striped":
        return p + P * np.arange(Sp, dtype=np.int64)
    raise ValueError(f"unknown layout {layout!r}")


def ring_schedule(P: int, i: int, causal: bool, layout: str = "contiguous") -> List[Tuple[int, str]]:
    """KV block visited by query partition i at each of the P ring steps, with its
    class ('diag', 'full' or 'skip').

    At step 0 every device works on its own block; after each step the blocks move
    one place round the ring, device d receiving from d-1 (device 0 from the last
    one), so at step s device i holds block (i - s) mod P ([RING] §"KV 在 Ring 中
    如何流动" and its flowchart; [IMPL] code sends to rank+1, receives from rank-1).
    Contiguous layout under a causal mask: a block strictly after the query
    partition holds only future keys and is skipped; the own block is the masked
    diagonal ([RING] same section, block-pair skipping by relative position).
    Striped layout under a causal mask: every block holds keys before and after
    each query, so every block is a masked ('diag') one and none is skipped.
    """
    if P <= 0 or not (0 <= i < P):
        raise ValueError("need P > 0 and 0 <= i < P")
    if layout not in LAYOUTS:
        raise ValueError(f"unknown layout {layout!r}")
    out = []
    for s in range(P):
        j = (i - s) % P
        if not causal:
            kind = "full"
        elif layout == "striped":
            kind = "diag"
        elif j > i:
            kind = "skip"
        elif j == i:
            kind = "diag"
        else:
            kind = "full"
        out.append((j, kind))
    return out


def ring_attention(q_part, k_blocks: Sequence, v_blocks: Sequence, *, i: int,
                   scale: float, causal: bool, Sp: int, block_order=None,
                   layout: str = "contiguous"):
    """Blockwise protocol for query partition i: start from O = 0, LSE = -inf,
    visit the KV blocks in ring order and merge each block's exact partial result
    ([RING] §最容易被忽略的细节; [IMPL] §Ring Attention环形注意力机制原理与超长序列处理).

    q_part [B,Hq,Sp,Dqk]; k_blocks[j] [B,Hkv,Sp,Dqk]; v_blocks[j] [B,Hkv,Sp,Dv], the
    tokens of each partition at the global positions partition_positions gives for
    the layout. `block_order` overrides the order (a list of block indices) to show
    the result does not depend on it. Exists to pin the protocol against one-shot
    attention.
    """
    P = len(k_blocks)
    B, Hq, Sq, _ = np.shape(q_part)
    Dv = np.shape(v_blocks[0])[3]
    o = np.zeros((B, Hq, Sq, Dv))
    lse = np.full((B, Hq, Sq), -np.inf)
    sched = dict(ring_schedule(P, i, causal, layout))
    order = block_order if block_order is not None else [j for j, _ in ring_schedule(P, i, causal, layout)]
    q_pos = partition_positions(P, Sp, i, layout)
    for j in order:
        if sched[j] == "skip":
            continue
        ob, lb = attention(q_part, k_blocks[j], v_blocks[j], scale=scale, causal=causal,
                           q_pos=q_pos, k_pos=partition_positions(P, Sp, j, layout))
        o, lse = merge(o, lse, ob, lb)
    return o, lse


def splitkv_decode(q, k, v, *, n_splits: int, scale: float):
    """Split-KV decode: one query token per sequence sees the whole cache (it is the
    newest token, so no key is in its future). The cache of length L is cut into
    n_splits contiguous equal chunks; each chunk yields a partial (O_p, LSE_p) by
    the exact definition, and merge_n reduces them ([CPEV] §名词定义 pass-Q and
    §Decode：cp 只解容量、不省计算).

    q [B,Hq,Dqk], k [B,Hkv,L,Dqk], v [B,Hkv,L,Dv]. Returns
    (o_part [B,Hq,n,Dv], lse_part [B,Hq,n], o [B,Hq,Dv], lse [B,Hq]), fp64.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    B, Hq, Dqk = q.shape
    Hkv, L = k.shape[1], k.shape[2]
    Dv = v.shape[3]
    if L % n_splits:
        raise ValueError("L must divide into n_splits equal chunks")
    Ls = L // n_splits
    group = Hq // Hkv
    o_part = np.zeros((B, Hq, n_splits, Dv))
    lse_part = np.zeros((B, Hq, n_splits))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            for p in range(n_splits):
                sl = slice(p * Ls, (p + 1) * Ls)
                o1, l1 = attention_rows(q[b, h][None, :], np.array([L]), k[b, g, sl], v[b, g, sl],
                                        scale=scale, causal=False, k_pos0=p * Ls)
                o_part[b, h, p], lse_part[b, h, p] = o1[0], l1[0]
    o, lse = merge_n(o_part, lse_part)
    return o_part, lse_part, o, lse
