"""Brute-force numpy form of sink attention, for tiny inputs only.  TEST INFRASTRUCTURE.

Written from the mathematics of the sink softmax ("MiMo-V2-Flash 架构 QA", Q3.8): the
denominator of row i is exp(sink_h) + the sum of exp(a_ij) over its visible keys, so with
the row's log-sum-exp

    LSE_i = log(exp(sink_h) + sum_{j in J(i)} exp(a_ij))

every visible key gets the weight exp(a_ij - LSE_i) and the output is those weights times V.
The sink has no value, so it only enters LSE_i.  This file works on whole matrices, takes
LSE_i as a pairwise log-add-exp reduction (numpy's logaddexp) and builds the mask from index
grids; oracle.c uses a max-shifted sum over explicit key lists.  The two share nothing, so
they can check each other.  float64 throughout.
"""
from __future__ import annotations

import numpy as np

GLOBAL = 0
SWA = 1


def mask_matrix(L: int, mode: int, window: int) -> np.ndarray:
    """Boolean [L, L]: True where query i may attend key j (causal; sliding: the `window`
    most recent keys, the query's own included)."""
    i = np.arange(L)[:, None]
    j = np.arange(L)[None, :]
    keep = j <= i
    if mode == SWA:
        keep &= j > i - window
    return keep


def prefill(q, k, v, sink, mode: int, window: int, scale: float, return_lse: bool = False):
    """q [B,Hq,L,dqk], k [B,Hkv,L,dqk], v [B,Hkv,L,dv] (any float dtype), sink [Hq] or None.
    Returns float64 [B,Hq,L,dv]; with return_lse also LSE_i, [B,Hq,L]."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, Hq, L, _ = q.shape
    G = Hq // k.shape[1]
    heads = np.arange(Hq) // G                 # query head h reads KV head h // G
    a = scale * (q @ np.swapaxes(k[:, heads], -1, -2))   # [B,Hq,L,L] logits
    a = np.where(mask_matrix(L, mode, window), a, -np.inf)
    lse = np.logaddexp.reduce(a, axis=-1)      # over the visible keys (-inf elsewhere)
    if sink is not None:
        lse = np.logaddexp(lse, np.asarray(sink, np.float64)[None, :, None])
    with np.errstate(invalid="ignore"):
        w = np.exp(a - lse[..., None])         # a = -inf (hidden) or lse = +inf give 0
    w = np.where(np.isnan(w), 0.0, w)          # -inf - (-inf): a row with no mass at all
    out = w @ v[:, heads]
    return (out, lse) if return_lse else out
