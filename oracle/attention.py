"""Textbook attention in float64 (test infrastructure).

The Dendrite article (ainews.cool, "technical deep dive") changes only *where*
keys and values come from: a branch's query attends over the K/V of its shared
ancestor path followed by its own leaf path.  What is computed for each query
head is ordinary scaled dot-product attention over that token sequence:

    out = sum_j softmax_j(q . k_j / sqrt(d)) v_j

Readings where the pages are silent:

* scale 1/sqrt(head_dim), natural exponent, max subtracted before exp (this
  changes nothing mathematically);
* grouped-query attention: query head ``hq`` reads KV head
  ``hq // (q_heads // kv_heads)`` (contiguous groups);
* a decode query sees every token of its branch, its own newest token included;
* a verification query for the draft at absolute position p sees positions
  0..p (the block-parallel verification of the DSpark blog, second layer);
  with one handle per draft path this is the tree-causal mask over prefix plus
  the path's own earlier drafts.

Everything runs in float64 on the exact input values.
"""

from __future__ import annotations

import math

import numpy as np


def attend_one(K: np.ndarray, V: np.ndarray, q: np.ndarray) -> np.ndarray:
    """softmax(K q / sqrt(d)) V for one query head.  K, V: [n][d]; q: [d]."""
    K = np.asarray(K, dtype=np.float64)
    V = np.asarray(V, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    if K.shape[0] == 0:
        raise ValueError("attention over an empty sequence")
    d = q.shape[-1]
    s = (K @ q) / math.sqrt(d)
    m = np.max(s)
    w = np.exp(s - m)
    return (w @ V) / np.sum(w)


def kv_head_of(hq: int, q_heads: int, kv_heads: int) -> int:
    if q_heads % kv_heads:
        raise ValueError("q_heads must be a multiple of kv_heads")
    return hq // (q_heads // kv_heads)


def decode(Kh, Vh, q: np.ndarray, kv_heads: int, heads=None) -> np.ndarray:
    """One decode query.

    Kh, Vh: callables ``g -> [n][d]`` (the branch's full history for KV head g)
    or arrays [n][kv_heads][d].  q: [q_heads][d].  Returns [q_heads][d] (rows
    not in ``heads`` are NaN when a subset is requested).
    """
    q = np.asarray(q, dtype=np.float64)
    hq_n = q.shape[0]
    kf = Kh if callable(Kh) else (lambda g: np.asarray(Kh)[:, g, :])
    vf = Vh if callable(Vh) else (lambda g: np.asarray(Vh)[:, g, :])
    out = np.full(q.shape, np.nan)
    cache = {}
    for hq in (range(hq_n) if heads is None else heads):
        g = kv_head_of(hq, hq_n, kv_heads)
        if g not in cache:
            cache[g] = (kf(g), vf(g))
        K, V = cache[g]
        out[hq] = attend_one(K, V, q[hq])
    return out


def verify(Kh, Vh, qs: np.ndarray, positions, kv_heads: int, heads=None) -> np.ndarray:
    """Verification of a block of queries on one branch.

    qs: [m][q_heads][d]; positions[i] is the absolute position of query i; query
    i attends over tokens 0..positions[i] of the branch.  Returns [m][q_heads][d].
    """
    qs = np.asarray(qs, dtype=np.float64)
    m, hq_n, _ = qs.shape
    kf = Kh if callable(Kh) else (lambda g: np.asarray(Kh)[:, g, :])
    vf = Vh if callable(Vh) else (lambda g: np.asarray(Vh)[:, g, :])
    out = np.full(qs.shape, np.nan)
    cache = {}
    for hq in (range(hq_n) if heads is None else heads):
        g = kv_head_of(hq, hq_n, kv_heads)
        if g not in cache:
            cache[g] = (kf(g), vf(g))
        K, V = cache[g]
        for i in range(m):
            p = int(positions[i])
            if p < 0 or p >= K.shape[0]:
                raise ValueError("query position outside the branch")
            out[i, hq] = attend_one(K[: p + 1], V[: p + 1], qs[i, hq])
    return out
