"""Flat reference allocator for the copy-on-write block table (test infrastructure).

Semantics (Dendrite article, ainews.cool, "technical deep dive"; Dendrite demo
tape, "the problem" section, which names a copy-on-write block table):

* The KV of a sequence lives in fixed-size blocks of ``block_size`` token slots.
  A handle's table is the ordered list of ``[block_id, valid]`` entries that
  holds its tokens, root first.
* ``fork(h, n)`` gives n new handles whose tables equal h's.  No block is
  written or allocated: the shared prefix is stored once.  Every block in h's
  table gains n sharers, and a block with two or more sharers becomes frozen.
* ``append(h, m)`` writes m new tokens.  A token goes into the tail entry only
  if that block is not frozen and still has a free slot; otherwise a fresh block
  is taken for it.  So after a fork every branch's new tokens start in blocks
  of their own, and no shared slot is ever written (the article's "new, empty
  leaf nodes for positions >= t").

Readings where the pages are silent (each is a choice, stated):

* Frozen is sticky: a block stays frozen until it is freed, even if its other
  sharers are released.  A forked partial tail block is therefore never
  written again, and the at most ``block_size - 1`` slots it leaves unused are
  the price of never copying.
* The parent handle stays live after a fork.
* A fresh block is always the lowest free block id.
* The sharer count of a block is the number of live handles whose table holds it.
* ``truncate(h, L)`` only removes tokens that sit in blocks that are not
  frozen; otherwise it fails with 'shared'.  ``L == len`` is a no-op.
* ``n < 1`` or ``m < 1`` -> 'inval'.  Appends are all-or-nothing: if the free
  set cannot hold them, 'nomem' and nothing changes.
* A released handle is dead; using it -> 'badseq'.
"""

from __future__ import annotations

import heapq
from typing import Dict, List, Tuple


class OracleError(Exception):
    def __init__(self, code: str):
        super().__init__(code)
        self.code = code


class FlatAllocator:
    def __init__(self, num_blocks: int, block_size: int = 16):
        if num_blocks < 0 or block_size < 1:
            raise ValueError("bad allocator shape")
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.share = [0] * num_blocks
        self.frozen = [False] * num_blocks
        self._free = list(range(num_blocks))
        heapq.heapify(self._free)
        self.tables: Dict[int, List[List[int]]] = {}
        self._next_handle = 1

    # -- helpers -------------------------------------------------------------
    def _table(self, h: int) -> List[List[int]]:
        t = self.tables.get(h)
        if t is None:
            raise OracleError("badseq")
        return t

    def _take_block(self) -> int:
        b = heapq.heappop(self._free)
        self.share[b] = 1
        self.frozen[b] = False
        return b

    def _drop_block(self, b: int) -> None:
        self.share[b] -= 1
        if self.share[b] == 0:
            self.frozen[b] = False
            heapq.heappush(self._free, b)

    # -- operations ----------------------------------------------------------
    def seq_new(self) -> int:
        h = self._next_handle
        self._next_handle += 1
        self.tables[h] = []
        return h

    def fork(self, h: int, n: int) -> List[int]:
        t = self._table(h)
        if n < 1:
            raise OracleError("inval")
        kids = []
        for _ in range(n):
            c = self._next_handle
            self._next_handle += 1
            self.tables[c] = [list(e) for e in t]
            kids.append(c)
        for b, _ in t:
            self.share[b] += n
            if self.share[b] >= 2:
                self.frozen[b] = True
        return kids

    def _blocks_needed(self, t: List[List[int]], m: int) -> int:
        bs = self.block_size
        room = 0
        if t:
            b, valid = t[-1]
            if not self.frozen[b]:
                room = bs - valid
        rest = max(0, m - room)
        return (rest + bs - 1) // bs

    def append(self, h: int, m: int) -> List[Tuple[int, int]]:
        """Append m tokens.  Returns the (block, slot) each token was written to."""
        t = self._table(h)
        if m < 1:
            raise OracleError("inval")
        if self._blocks_needed(t, m) > len(self._free):
            raise OracleError("nomem")
        where = []
        for _ in range(m):
            if not t or t[-1][1] == self.block_size or self.frozen[t[-1][0]]:
                t.append([self._take_block(), 0])
            b, valid = t[-1]
            where.append((b, valid))
            t[-1][1] = valid + 1
        return where

    def release(self, h: int) -> None:
        t = self._table(h)
        for b, _ in t:
            self._drop_block(b)
        del self.tables[h]

    def truncate(self, h: int, new_len: int) -> None:
        t = self._table(h)
        cur = self.length(h)
        if new_len < 0 or new_len > cur:
            raise OracleError("range")
        if new_len == cur:
            return
        start = 0
        starts = []
        for b, valid in t:
            starts.append(start)
            start += valid
        # any frozen block that holds a position in [new_len, cur) -> refuse
        for (b, valid), s in zip(t, starts):
            if s + valid > new_len and self.frozen[b]:
                raise OracleError("shared")
        keep = []
        for (b, valid), s in zip(t, starts):
            if s >= new_len:
                self._drop_block(b)
            else:
                keep.append([b, min(valid, new_len - s)])
        self.tables[h] = keep

    # -- observables ---------------------------------------------------------
    def length(self, h: int) -> int:
        return sum(v for _, v in self._table(h))

    def table(self, h: int) -> List[Tuple[int, int]]:
        return [(b, v) for b, v in self._table(h)]

    def sharers(self, b: int) -> int:
        return self.share[b]

    def num_free(self) -> int:
        return len(self._free)

    def live_handles(self) -> List[int]:
        return sorted(self.tables)
