"""Replay a workload recipe on the oracle (test infrastructure).

Drives ``FlatAllocator`` (block tables) and ``MaterializedCache`` (values) in
lockstep over the same operation list the library replays, and computes the
reference output of every decode / verify operation, either in full or for a
sample of (query row, head) pairs.
"""

from __future__ import annotations

from typing import Dict, Iterable, Optional

import numpy as np

import workloads
from workloads import gen

from . import attention
from .allocator import FlatAllocator
from .cache import FunctionSource, MaterializedCache


def _source_for(wl, call: int, ntok: int):
    def fn(which, layer, kvh, t0, t1):
        kind = gen.KIND_K if which == "k" else gen.KIND_V
        return workloads.kv_slice(wl, call, ntok, kind, layer, kvh, t0, t1)
    return FunctionSource(ntok, fn)


def _batch_source_for(wl, call: int, total: int, first: int, ntok: int):
    """Rows [first, first + ntok) of a batched append's source arrays, which hold
    ``total`` token rows (the handles' tokens one after another)."""
    def fn(which, layer, kvh, t0, t1):
        kind = gen.KIND_K if which == "k" else gen.KIND_V
        return workloads.kv_slice(wl, call, total, kind, layer, kvh, first + t0, first + t1)
    return FunctionSource(ntok, fn)


class OracleReplay:
    def __init__(self, wl, with_alloc: bool = True):
        self.wl = wl
        self.alloc = FlatAllocator(wl.num_blocks, wl.block_size) if with_alloc else None
        self.mat = MaterializedCache()
        self.h_alloc: Dict[int, int] = {}
        self.h_mat: Dict[int, int] = {}

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
            self.mat.append(self.h_mat[h], _source_for(self.wl, call, ntok))
        elif kind == "append_batch":
            # by definition, the appends one after another in batch order
            _, hs, ns, call = op
            total, first = sum(ns), 0
            for h, n in zip(hs, ns):
                if self.alloc is not None:
                    self.alloc.append(self.h_alloc[h], n)
                self.mat.append(self.h_mat[h], _batch_source_for(self.wl, call, total, first, n))
                first += n
        elif kind == "reserve_batch":
            # one token per handle whose K/V (every layer) are those of batched
            # append `call`, written later by the decode_new ops
            _, hs, call = op
            self.apply(("append_batch", hs, [1] * len(hs), call))
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
        elif kind in ("decode", "decode_new", "verify", "time_begin"):
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
        for h, items in by_handle.items():
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
        return out
