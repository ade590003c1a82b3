"""Brute-force numpy form of sink attention, for tiny inputs only.  TEST INFRASTRUCTURE.

This is the eager form the architecture deep-dive page prints ("MiMo-V2-Flash
模型架构深度拆解", CH 10.1; restated in "MiMo-V2-Flash 架构 QA", Q3.8): materialise the
masked, scaled score matrix [S, S], append the per-head sink as one more column, take a
softmax over the S+1 columns, drop the sink column, multiply by V.  It is written
independently of oracle.c (whole matrices, a different reduction order, a mask built from
index grids) so the two can check each other.  float64 throughout.
"""
from __future__ import annotations

import numpy as np

GLOBAL = 0
SWA = 1


def mask_matrix(L: int, mode: int, window: int) -> np.ndarray:
    """Boolean [L, L]: True where query i may attend key j."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    keep = j <= i
    if mode == SWA:
        keep &= j > i - window
    return keep


def prefill(q, k, v, sink, mode: int, window: int, scale: float, return_lse: bool = False):
    """q [B,Hq,L,dqk], k [B,Hkv,L,dqk], v [B,Hkv,L,dv] (any float dtype), sink [Hq] or None.
    Returns float64 [B,Hq,L,dv]; with return_lse also scipy's logsumexp over each row's
    S+1 columns (the log of the softmax denominator), [B,Hq,L]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, L, _ = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    kx = np.repeat(k, G, axis=1)  # query head h uses KV head h // G
    vx = np.repeat(v, G, axis=1)
    scores = np.einsum("bhid,bhjd->bhij", q, kx) * scale
    scores = np.where(mask_matrix(L, mode, window)[None, None], scores, -np.inf)
    if sink is not None:
        col = np.broadcast_to(np.asarray(sink, np.float64)[None, :, None, None], (B, Hq, L, 1))
        scores = np.concatenate([scores, col], axis=-1)
    if return_lse:
        from scipy.special import logsumexp

        lse = logsumexp(scores, axis=-1)
    mx = scores.max(axis=-1, keepdims=True)
    with np.errstate(invalid="ignore"):
        e = np.exp(scores - mx)
        probs = e / e.sum(axis=-1, keepdims=True)
    if sink is not None:
        probs = probs[..., :-1]
        probs = np.where(np.isposinf(np.asarray(sink, np.float64))[None, :, None, None], 0.0, probs)
    return (probs @ vx, lse) if return_lse else probs @ vx
