"""Synthetic workloads: seeded input generation (``gen``) and call recipes (``recipes``).

Shared by the oracle and the HIP path; contains no part of the method itself.
"""

from __future__ import annotations

import numpy as np

from . import gen, recipes  # noqa: F401


def kv_values(wl, call: int, ntok: int, kind: int) -> np.ndarray:
    """All K (kind=gen.KIND_K) or V values of append call ``call``, float32,
    shape [layers][ntok][kv_heads][head_dim]."""
    n = wl.layers * ntok * wl.kv_heads * wl.head_dim
    v = gen.values_range(wl.seed, gen.stream_id(kind, call), 0, n, wl.dtype)
    return v.reshape(wl.layers, ntok, wl.kv_heads, wl.head_dim)


def kv_slice(wl, call: int, ntok: int, kind: int, layer: int, kvh: int, t0: int, t1: int) -> np.ndarray:
    """Values of tokens [t0, t1) of one layer and KV head of an append call: [t1-t0][head_dim]."""
    t = np.arange(t0, t1, dtype=np.uint64)[:, None]
    d = np.arange(wl.head_dim, dtype=np.uint64)[None, :]
    idx = ((np.uint64(layer) * np.uint64(ntok) + t) * np.uint64(wl.kv_heads) + np.uint64(kvh)) \
        * np.uint64(wl.head_dim) + d
    return gen.values(wl.seed, gen.stream_id(kind, call), idx.reshape(-1), wl.dtype).reshape(
        t1 - t0, wl.head_dim)


def q_values(wl, qcall: int, nrows: int) -> np.ndarray:
    """Query values of a decode/verify call: [nrows][q_heads][head_dim], float32."""
    n = nrows * wl.q_heads * wl.head_dim
    v = gen.values_range(wl.seed, gen.stream_id(gen.KIND_Q, qcall), 0, n, wl.dtype) * np.float32(wl.q_scale)
    return v.reshape(nrows, wl.q_heads, wl.head_dim)
