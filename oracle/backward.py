"""Gradients of exact attention, fp64 (test infrastructure).

The pages use ring attention for training samples too long for one device and
name the backward pass's data dependencies among the things to check when a
distributed result disagrees with the single-device one ([RING] opening example
and §什么时候值得引入 Context Parallelism). They give no gradient formulas, so the
plainest reading is taken: the exact gradients of the definition they compute,
O = softmax(scale * Q K^T) V over the visible keys ([CH] §挑战 1, eq.
lc-ch-attention), with the row LSE saved by the forward pass.

Written out, with P the row-softmax of the scaled scores and dO the incoming
gradient:
    dV = P^T dO,  dP = dO V^T,  delta = rowsum(P o dP) = rowsum(dO o O),
    dS = P o (dP - delta),  dQ = scale dS K,  dK = scale dS^T Q.
A query row with no visible key has O = 0 and contributes nothing. Under GQA the
gradient of a KV head sums over its query heads.

Blockwise: with the full-row LSE and delta fixed, P restricted to one KV block is
exp(scale q k - LSE) on that block, so each (query block, KV block) pair's
contribution can be computed on its own and the contributions summed -- the
backward counterpart of the forward's block merge.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from .exact import _f64, visible


def _positions(n, pos0, pos):
    return pos0 + np.arange(n) if pos is None else np.asarray(pos)


def attention_bwd(q, k, v, dout, *, scale: float, causal: bool, q_pos0: int = 0, k_pos0: int = 0,
                  q_pos=None, k_pos=None) -> Tuple[np.ndarray, ...]:
    """dQ [B,Hq,Sq,Dqk], dK [B,Hkv,Sk,Dqk], dV [B,Hkv,Sk,Dv] of sum(O o dO), and the
    forward's LSE [B,Hq,Sq] and delta = rowsum(dO o O) [B,Hq,Sq], all fp64, with the
    score matrix materialised per (batch, head)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    B, Hq, Sq, Dqk = q.shape
    Hkv, Sk, Dv = k.shape[1], k.shape[2], v.shape[3]
    group = Hq // Hkv
    vis = visible(_positions(Sq, q_pos0, q_pos), _positions(Sk, k_pos0, k_pos), causal)
    any_vis = vis.any(axis=1)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    lse = np.full((B, Hq, Sq), -np.inf)
    delta = np.zeros((B, Hq, Sq))
    for b in range(B):
        for h in range(Hq):
            g = h // group
            s = np.where(vis, scale * (q[b, h] @ k[b, g].T), -np.inf)
            m = np.where(any_vis, s.max(axis=1, initial=-np.inf), 0.0)
            e = np.exp(s - m[:, None])
            den = e.sum(axis=1)
            p = np.where(any_vis[:, None], e / np.where(any_vis, den, 1.0)[:, None], 0.0)
            with np.errstate(divide="ignore"):
                lse[b, h] = np.where(any_vis, m + np.log(np.where(any_vis, den, 1.0)), -np.inf)
            o = p @ v[b, g]
            dp = dout[b, h] @ v[b, g].T
            dlt = (dout[b, h] * o).sum(axis=1)
            ds = p * (dp - dlt[:, None])
            dq[b, h] = scale * ds @ k[b, g]
            dk[b, g] += scale * ds.T @ q[b, h]
            dv[b, g] += p.T @ dout[b, h]
            delta[b, h] = dlt
    return dq, dk, dv, lse, delta


def block_bwd(q, k_blk, v_blk, dout, lse, delta, *, scale: float, causal: bool, q_pos0: int = 0,
              k_pos0: int = 0, q_pos=None, k_pos=None) -> Tuple[np.ndarray, np.ndarray, np.ndarray]:
    """One (query block, KV block) pair's share of dQ, dK, dV given the full-row lse
    and delta of the queries: P = exp(scale q k - lse) on this block's visible
    keys, dS = P o (dO V^T - delta). Summed over all KV blocks (dQ) and all query
    blocks (dK, dV) it gives attention_bwd."""
    q, k_blk, v_blk, dout = _f64(q), _f64(k_blk), _f64(v_blk), _f64(dout)
    lse, delta = _f64(lse), _f64(delta)
    B, Hq, Sq, _ = q.shape
    Hkv, Sk = k_blk.shape[1], k_blk.shape[2]
    group = Hq // Hkv
    vis = visible(_positions(Sq, q_pos0, q_pos), _positions(Sk, k_pos0, k_pos), causal)
    dq = np.zeros_like(q)
    dk = np.zeros_like(k_blk)
    dv = np.zeros_like(v_blk)
    for b in range(B):
        for h in range(Hq):
            g = h // group
            live = np.isfinite(lse[b, h])
            s = scale * (q[b, h] @ k_blk[b, g].T)
            p = np.where(vis & live[:, None], np.exp(s - np.where(live, lse[b, h], 0.0)[:, None]), 0.0)
            dp = dout[b, h] @ v_blk[b, g].T
            ds = p * (dp - delta[b, h][:, None])
            dq[b, h] = scale * ds @ k_blk[b, g]
            dk[b, g] += scale * ds.T @ q[b, h]
            dv[b, g] += p.T @ dout[b, h]
    return dq, dk, dv
