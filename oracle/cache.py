"""Materialised per-branch KV histories (test infrastructure).

Each handle owns its complete token history in order: the full-copy strategy
that the Dendrite article (ainews.cool, "technical deep dive", first option)
sets against its copy-on-write tree.  A fork duplicates the parent's history;
an append extends it; a truncation shortens it.  Block ids never appear here,
so this half of the oracle is independent of the allocator half and of the
library.

A history is a list of segments ``(source, t0, t1)``: tokens [t0, t1) of one
append call's input.  Sources hand out float64 rows on demand, so a handle's
history is materialised only for the layer and KV head a check needs; the
values are the same whether a source holds arrays or regenerates them.
"""

from __future__ import annotations

from typing import Dict, List, Tuple

import numpy as np


class ArraySource:
    """Append input held in memory: K, V arrays [layers][ntok][kv_heads][d]."""

    def __init__(self, K: np.ndarray, V: np.ndarray):
        self.K = np.asarray(K)
        self.V = np.asarray(V)
        self.ntok = self.K.shape[1]

    def rows(self, which: str, layer: int, kvh: int, t0: int, t1: int) -> np.ndarray:
        a = self.K if which == "k" else self.V
        return np.asarray(a[layer, t0:t1, kvh, :], dtype=np.float64)


class FunctionSource:
    """Append input produced on demand by ``fn(which, layer, kvh, t0, t1) -> [t1-t0][d]``."""

    def __init__(self, ntok: int, fn):
        self.ntok = ntok
        self.fn = fn

    def rows(self, which: str, layer: int, kvh: int, t0: int, t1: int) -> np.ndarray:
        return np.asarray(self.fn(which, layer, kvh, t0, t1), dtype=np.float64)


class MaterializedCache:
    def __init__(self):
        self.hist: Dict[int, List[Tuple[object, int, int]]] = {}
        self._next = 1

    def seq_new(self) -> int:
        h = self._next
        self._next += 1
        self.hist[h] = []
        return h

    def fork(self, h: int, n: int) -> List[int]:
        src = self.hist[h]
        kids = []
        for _ in range(n):
            c = self._next
            self._next += 1
            self.hist[c] = list(src)  # the child's own copy of the whole history
            kids.append(c)
        return kids

    def append(self, h: int, source) -> None:
        self.hist[h].append((source, 0, source.ntok))

    def release(self, h: int) -> None:
        del self.hist[h]

    def length(self, h: int) -> int:
        return sum(t1 - t0 for _, t0, t1 in self.hist[h])

    def truncate(self, h: int, new_len: int) -> None:
        out = []
        pos = 0
        for src, t0, t1 in self.hist[h]:
            n = t1 - t0
            if pos >= new_len:
                break
            take = min(n, new_len - pos)
            out.append((src, t0, t0 + take))
            pos += take
        self.hist[h] = out

    def kv(self, h: int, layer: int, kvh: int) -> Tuple[np.ndarray, np.ndarray]:
        """The branch's full K and V history for one layer and KV head: [len][d] each."""
        ks, vs = [], []
        for src, t0, t1 in self.hist[h]:
            ks.append(src.rows("k", layer, kvh, t0, t1))
            vs.append(src.rows("v", layer, kvh, t0, t1))
        if not ks:
            return np.zeros((0, 0)), np.zeros((0, 0))
        return np.concatenate(ks, axis=0), np.concatenate(vs, axis=0)
