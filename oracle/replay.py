"""Replay a workload recipe on the oracle (test infrastructure).

Drives ``FlatAllocator`` (block tables) and ``MaterializedCache`` (values) in
lockstep over the same operation list the library replays, and computes the
reference output of every decode / verify operation, either in full or for a
sample of (query row, head) pairs.
"""

from __future__ import annotations

import threading
from concurrent.futures import ThreadPoolExecutor
from typing import Dict, Iterable, Optional

import numpy as np

import workloads
from workloads import gen

from . import attention
from .allocator import FlatAllocator
from .cache import FunctionSource, MaterializedCache


class _LayerArrays:
    """The values of append calls, one layer at a time: each (call, K | V, layer)
    is generated once, as the contiguous range of the call's stream that holds
    that layer ([layers][ntok][kv_heads][d] order), and kept until a different
    layer is asked for.  The same numbers as ``workloads.kv_slice``, generated
    in bulk (and by several threads) for checks that read whole layers."""

    def __init__(self, wl, threads: int):
        self.wl = wl
        self.threads = max(1, threads)
        self.layer = None
        self.arrays: Dict[tuple, np.ndarray] = {}
        self.lock = threading.Lock()

    def _generate(self, stream: int, start: int, count: int) -> np.ndarray:
        wl = self.wl
        if self.threads == 1 or count < (1 << 20):
            return gen.values_range(wl.seed, stream, start, count, wl.dtype)
        n = self.threads
        bounds = [start + count * i // n for i in range(n + 1)]
        with ThreadPoolExecutor(n) as ex:
            parts = list(ex.map(lambda i: gen.values_range(wl.seed, stream, bounds[i], bounds[i + 1] - bounds[i],
                                                           wl.dtype), range(n)))
        return np.concatenate(parts)

    def get(self, call: int, ntok: int, kind: int, layer: int) -> np.ndarray:
        """[ntok][kv_heads][d] float32 values of one layer of an append call."""
        wl = self.wl
        key = (call, kind, layer)
        with self.lock:
            if self.layer != layer:
                self.arrays.clear()
                self.layer = layer
            a = self.arrays.get(key)
            if a is None:
                per_layer = ntok * wl.kv_heads * wl.head_dim
                a = self._generate(gen.stream_id(kind, call), layer * per_layer, per_layer).reshape(
                    ntok, wl.kv_heads, wl.head_dim)
                self.arrays[key] = a
            return a


class PreloadedArrays:
    """Every append call's values generated up front (on ``threads`` threads), so
    that a timed replay measures the oracle's own work and not the input
    generator; ``get`` answers as ``_LayerArrays.get`` does."""

    def __init__(self, wl, threads: int = 1):
        self.wl = wl
        gen_ = _LayerArrays(wl, threads)
        self.arrays: Dict[tuple, np.ndarray] = {}
        for op in wl.ops:
            if op[0] == "append":
                calls = [(op[3], op[2])]
            elif op[0] in ("append_batch",):
                calls = [(op[3], sum(op[2]))]
            elif op[0] == "reserve_batch":
                calls = [(op[2], sum(op[3]) if len(op) > 3 else len(op[1]))]
            else:
                continue
            for call, total in calls:
                per_layer = total * wl.kv_heads * wl.head_dim
                for kind in (gen.KIND_K, gen.KIND_V):
                    whole = gen_._generate(gen.stream_id(kind, call), 0, wl.layers * per_layer)
                    self.arrays[(call, kind)] = whole.reshape(wl.layers, total, wl.kv_heads, wl.head_dim)

    def get(self, call: int, ntok: int, kind: int, layer: int) -> np.ndarray:
        return self.arrays[(call, kind)][layer]


def _source_for(wl, call: int, ntok: int, arrays: Optional[_LayerArrays] = None):
    return _batch_source_for(wl, call, ntok, 0, ntok, arrays)


def _batch_source_for(wl, call: int, total: int, first: int, ntok: int, arrays: Optional[_LayerArrays] = None):
    """Rows [first, first + ntok) of a batched append's source arrays, which hold
    ``total`` token rows (the handles' tokens one after another)."""
    def fn(which, layer, kvh, t0, t1):
        kind = gen.KIND_K if which == "k" else gen.KIND_V
        if arrays is not None:
            return arrays.get(call, total, kind, layer)[first + t0:first + t1, kvh, :]
        return workloads.kv_slice(wl, call, total, kind, layer, kvh, first + t0, first + t1)
    return FunctionSource(ntok, fn)


class OracleReplay:
    """``threads`` > 1: append values are generated a whole layer of a call at a
    time (the same numbers) and ``attend`` works on several handles at once;
    the arithmetic of each output is unchanged.  ``arrays``: a
    ``PreloadedArrays`` holding every call's values already."""

    def __init__(self, wl, with_alloc: bool = True, threads: int = 1, arrays=None):
        self.wl = wl
        self.alloc = FlatAllocator(wl.num_blocks, wl.block_size) if with_alloc else None
        self.mat = MaterializedCache()
        self.h_alloc: Dict[int, int] = {}
        self.h_mat: Dict[int, int] = {}
        self.threads = max(1, threads)
        self.arrays = arrays if arrays is not None else (_LayerArrays(wl, self.threads) if self.threads > 1 else None)

    # -- structural ops --------------------------------------------------------
    def apply(self, op) -> None:
        kind = op[0]
        if kind == "new":
            if self.alloc is not None:
                self.h_alloc[op[1]] = self.alloc.seq_new()
            self.h_mat[op[1]] = self.mat.seq_new()
        elif kind == "append":
            _, h, ntok, call = op
            if self.alloc is not None:
                self.alloc.append(self.h_alloc[h], ntok)
            self.mat.append(self.h_mat[h], _source_for(self.wl, call, ntok, self.arrays))
        elif kind == "append_batch":
            # by definition, the appends one after another in batch order
            _, hs, ns, call = op
            total, first = sum(ns), 0
            for h, n in zip(hs, ns):
                if self.alloc is not None:
                    self.alloc.append(self.h_alloc[h], n)
                self.mat.append(self.h_mat[h], _batch_source_for(self.wl, call, total, first, n, self.arrays))
                first += n
        elif kind == "reserve_batch":
            # ntok[i] tokens (default one) for handle i whose K/V (every layer)
            # are those of batched append `call`, written later by the
            # decode_new ops
            hs, call = op[1], op[2]
            ns = list(op[3]) if len(op) > 3 else [1] * len(hs)
            self.apply(("append_batch", hs, ns, call))
        elif kind == "fork":
            _, h, n, kids = op
            if self.alloc is not None:
                for k, c in zip(kids, self.alloc.fork(self.h_alloc[h], n)):
                    self.h_alloc[k] = c
            for k, c in zip(kids, self.mat.fork(self.h_mat[h], n)):
                self.h_mat[k] = c
        elif kind == "release":
            if self.alloc is not None:
                self.alloc.release(self.h_alloc.pop(op[1]))
            self.mat.release(self.h_mat.pop(op[1]))
        elif kind == "truncate":
            _, h, L = op
            if self.alloc is not None:
                self.alloc.truncate(self.h_alloc[h], L)
            self.mat.truncate(self.h_mat[h], L)
        elif kind in ("decode", "decode_new", "verify", "verify_new", "time_begin"):
            pass
        else:
            raise ValueError(kind)

    # -- attention ---------------------------------------------------------------
    def query_rows(self, op):
        """(handle name, absolute position) of every query row of a decode/verify op."""
        rows = []
        if op[0] in ("decode", "decode_new"):
            for h in op[2]:
                rows.append((h, self.mat.length(self.h_mat[h]) - 1))
        else:
            for h, nq in zip(op[2], op[3]):
                L = self.mat.length(self.h_mat[h])
                for i in range(nq):
                    rows.append((h, L - nq + i))
        return rows

    def attend(self, op, sample: Optional[Iterable] = None) -> np.ndarray:
        """Reference output of a decode/verify op at the current state.

        ``sample``: iterable of (row, head) pairs; None = every row and head.
        Returns [rows][q_heads][d] float64 with NaN where not computed.
        """
        wl = self.wl
        layer = op[1]
        rows = self.query_rows(op)
        Q = workloads.q_values(wl, op[-1], len(rows)).astype(np.float64)
        out = np.full((len(rows), wl.q_heads, wl.head_dim), np.nan)
        want: Dict[int, list] = {}
        if sample is None:
            for r in range(len(rows)):
                want[r] = list(range(wl.q_heads))
        else:
            for r, hq in sample:
                want.setdefault(int(r), []).append(int(hq))
        by_handle: Dict[int, list] = {}
        for r, heads in want.items():
            by_handle.setdefault(rows[r][0], []).append((r, heads))
        def one_handle(h):
            items = by_handle[h]
            mh = self.h_mat[h]
            heads_needed = sorted({hq for _, hs in items for hq in hs})
            kv = {}
            for hq in heads_needed:
                g = attention.kv_head_of(hq, wl.q_heads, wl.kv_heads)
                if g not in kv:
                    kv[g] = self.mat.kv(mh, layer, g)
            for r, heads in items:
                pos = rows[r][1]
                for hq in heads:
                    g = attention.kv_head_of(hq, wl.q_heads, wl.kv_heads)
                    K, V = kv[g]
                    out[r, hq] = attention.attend_one(K[: pos + 1], V[: pos + 1], Q[r, hq])

        if self.threads > 1 and len(by_handle) > 1:
            with ThreadPoolExecutor(self.threads) as ex:
                list(ex.map(one_handle, list(by_handle)))
        else:
            for h in by_handle:
                one_handle(h)
        return out
