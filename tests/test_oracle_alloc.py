"""Pins for the oracle's allocator half (CPU only).

The flat allocator is tied to: a hand-derived walkthrough fixture, closed forms
of the block ids each standard workload must produce, invariants that follow
from the copy-on-write description (fork writes and allocates nothing; every
handle's table addresses exactly its own token history; memory grows only with
divergent tokens), and exhaustive enumeration of short operation sequences on
a tiny pool.  Planted mistakes at the end must each be caught.
"""

import itertools
import json
import os
import random

import pytest

from oracle import allocator as A
from workloads import recipes

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _apply(al, names, op):
    kind = op[0]
    if kind == "new":
        names[op[1]] = al.seq_new()
    elif kind == "append":
        al.append(names[op[1]], op[2])
    elif kind == "fork":
        kids = al.fork(names[op[1]], op[2])
        for k, c in zip(op[3], kids):
            names[k] = c
    elif kind == "release":
        al.release(names.pop(op[1]))
    elif kind == "truncate":
        al.truncate(names[op[1]], op[2])
    elif kind in ("decode", "verify"):
        pass
    else:
        raise ValueError(kind)


def _lookup(names, h):
    return names.get(h, -1)


def pin_walkthrough(cls=A.FlatAllocator):
    g = json.load(open(os.path.join(GOLD, "alloc_walkthrough.json")))
    al = cls(g["num_blocks"], g["block_size"])
    names = {}
    for st in g["steps"]:
        op = st["op"]
        err = None
        try:
            if op[0] in ("fork", "append", "release", "truncate") and op[1] not in names:
                # a handle that was released: use a dead id
                tmp = dict(names); tmp[op[1]] = 10 ** 9
                _apply(al, tmp, op)
            else:
                _apply(al, names, op)
        except A.OracleError as e:
            err = e.code
        assert err == st.get("error"), (op, err)
        live = {k: al.table(v) for k, v in names.items()}
        assert {k: [list(e) for e in v] for k, v in live.items()} == st["tables"], op
        assert al.num_free() == st["free"], op
        assert [al.sharers(b) for b in range(g["num_blocks"])] == st["sharers"], op


def test_walkthrough():
    pin_walkthrough()


# ---------------------------------------------------------------------------
# closed forms at the standard workloads

def _replay(wl):
    al = A.FlatAllocator(wl.num_blocks, wl.block_size)
    names = {}
    for op in wl.ops:
        _apply(al, names, op)
    return al, names


def pin_fork_workload_ids(cls=A.FlatAllocator):
    """Request r of a (prefix P, width W, branch T) fork workload holds blocks
    r*S + [0, P/16) as its prefix and branch b holds r*S + P/16 + b*T/16 + [0, T/16),
    S = P/16 + W*T/16; prefix blocks have W sharers, branch blocks 1; nothing is free."""
    for wl, (P, W, T) in [(recipes.tiny_fork(), (256, 4, 32)), (recipes.llama_fork(), (4096, 4, 64)),
                          (recipes.full_depth(), (8192, 16, 256))]:
        al = cls(wl.num_blocks, wl.block_size)
        names = {}
        for op in wl.ops:
            _apply(al, names, op)
        pb, tb = P // 16, T // 16
        S = pb + W * tb
        leaves = wl.attend_ops()[0][2]
        assert al.num_free() == 0
        for i, h in enumerate(leaves):
            r, b = divmod(i, W)
            want = [(r * S + k, 16) for k in range(pb)] + [(r * S + pb + b * tb + k, 16) for k in range(tb)]
            assert al.table(names[h]) == want
        for r in range(wl.num_blocks // S):
            assert all(al.sharers(r * S + k) == W for k in range(pb))
            assert all(al.sharers(r * S + pb + k) == 1 for k in range(W * tb))


def test_fork_workload_ids():
    pin_fork_workload_ids()


def pin_verify_workload_accept(cls=A.FlatAllocator):
    """Speculative verify: request r's prefix is blocks 131r + [0,128), path b's drafts
    are block 131r + 128 + b with 8 valid.  After accepting path a with k drafts, the
    accepted path keeps its draft block with k valid (freed if k = 0), the other two
    draft blocks are freed, and the prefix has one sharer."""
    from workloads import gen
    wl = recipes.spec_verify()
    al = cls(wl.num_blocks, wl.block_size)
    names = {}
    verify_seen = False
    for op in wl.ops:
        _apply(al, names, op)
        if op[0] == "verify":
            verify_seen = True
            for i, h in enumerate(op[2]):
                r, b = divmod(i, 3)
                assert al.table(names[h]) == [(131 * r + k, 16) for k in range(128)] + [(131 * r + 128 + b, 8)]
    assert verify_seen
    free = 0
    for r in range(64):
        st = gen.stream_id(gen.KIND_ACCEPT, r)
        a = gen.uniform_int(0, st, 0, 3)
        k = gen.uniform_int(0, st, 1, 9)
        h = 4 * r + 1 + a  # symbolic names: request r's parent is 4r, its paths 4r+1..4r+3
        tail = [(131 * r + 128 + a, k)] if k else []
        assert al.table(names[h]) == [(131 * r + j, 16) for j in range(128)] + tail
        assert all(al.sharers(131 * r + j) == 1 for j in range(128))
        free += 2 + (k == 0)
    assert al.num_free() == free


def test_verify_workload_accept():
    pin_verify_workload_accept()


def test_mcts_tree_blocks():
    """The MCTS tree: the root holds 128 blocks shared by all 256 leaves; each leaf
    holds 1 + 12 blocks; the union of tables covers every allocated block once."""
    wl = recipes.mcts_tree()
    al, names = _replay(wl)
    leaves = wl.attend_ops()[0][2]
    tabs = [al.table(names[h]) for h in leaves]
    assert all(t[:128] == [(k, 16) for k in range(128)] for t in tabs)
    assert all(len(t) == 140 and all(v == 16 for _, v in t) for t in tabs)
    assert all(al.sharers(k) == 256 for k in range(128))
    used = set(b for t in tabs for b, _ in t)
    assert used == set(range(wl.num_blocks)) and al.num_free() == 0


# ---------------------------------------------------------------------------
# invariants on random operation sequences

class Shadow:
    """Token-level model: each handle's history as a list of token uids."""

    def __init__(self, al):
        self.al = al
        self.hist = {}
        self.slots = {}  # (block, slot) -> uid written there
        self.uid = 0


def _check_invariants(al, sh, names):
    # every live handle's table addresses exactly its own history
    for name, h in names.items():
        tab = al.table(h)
        got = [sh.slots[(b, s)] for b, v in tab for s in range(v)]
        assert got == sh.hist[name], name
        assert al.length(h) == len(sh.hist[name])
    # sharer counts = number of live tables holding the block
    count = {}
    for h in names.values():
        for b, _ in al.table(h):
            count[b] = count.get(b, 0) + 1
    for b in range(al.num_blocks):
        assert al.sharers(b) == count.get(b, 0)
    assert al.num_free() == al.num_blocks - len(count)


def _random_session(seed, num_blocks=24, bs=4, steps=200, cls=A.FlatAllocator):
    rnd = random.Random(seed)
    al = cls(num_blocks, bs)
    sh = Shadow(al)
    names = {}
    nxt = 0
    for _ in range(steps):
        live = sorted(names)
        r = rnd.random()
        if not live or r < 0.08:
            names[nxt] = al.seq_new(); sh.hist[nxt] = []; nxt += 1
        elif r < 0.30:
            p = rnd.choice(live)
            n = rnd.randint(1, 3)
            before_free = al.num_free()
            kids = al.fork(names[p], n)
            assert al.num_free() == before_free
            for c in kids:
                names[nxt] = c; sh.hist[nxt] = list(sh.hist[p]); nxt += 1
                assert al.table(c) == al.table(names[p])
        elif r < 0.65:
            h = rnd.choice(live)
            m = rnd.randint(1, 9)
            snap = (al.table(names[h]), al.num_free())
            try:
                where = al.append(names[h], m)
            except A.OracleError as e:
                assert e.code == "nomem"
                assert (al.table(names[h]), al.num_free()) == snap
                continue
            for b, s in where:
                # a written slot is never one that another live table can see
                for other, oh in names.items():
                    if other != h:
                        assert all(not (bb == b and s < v) for bb, v in al.table(oh))
                sh.slots[(b, s)] = sh.uid
                sh.hist[h].append(sh.uid)
                sh.uid += 1
        elif r < 0.85:
            h = rnd.choice(live)
            al.release(names.pop(h)); del sh.hist[h]
        else:
            h = rnd.choice(live)
            L = rnd.randint(0, len(sh.hist[h]))
            try:
                al.truncate(names[h], L)
                sh.hist[h] = sh.hist[h][:L]
            except A.OracleError as e:
                assert e.code == "shared"
        _check_invariants(al, sh, names)
    for h in list(names):
        al.release(names.pop(h))
    assert al.num_free() == num_blocks


@pytest.mark.parametrize("seed", range(12))
def test_random_sessions_keep_invariants(seed):
    _random_session(seed)


def test_fork_memory_is_divergent_tokens_only():
    """b branches of a long prefix cost only their own new blocks (article: memory
    overhead proportional to the divergent tokens, not to the history)."""
    al = A.FlatAllocator(1000, 16)
    p = al.seq_new()
    al.append(p, 16 * 40)
    used0 = 1000 - al.num_free()
    kids = al.fork(p, 8)
    assert 1000 - al.num_free() == used0
    for c in kids:
        al.append(c, 20)
    assert 1000 - al.num_free() == used0 + 8 * 2


def _exhaustive(cls=A.FlatAllocator, max_len=5):
    """Every sequence of up to max_len ops over a 4-block, block-size-2 pool."""
    moves = []
    for h in range(3):
        moves += [("append", h, 1), ("append", h, 3), ("fork", h, 1), ("fork", h, 2),
                  ("release", h), ("truncate", h, 1), ("truncate", h, 0)]
    count = 0
    for length in range(1, max_len + 1):
        for seq in itertools.product(moves, repeat=length):
            al = cls(4, 2)
            sh = Shadow(al)
            names = {0: al.seq_new()}
            sh.hist[0] = []
            nxt = 1
            for mv in seq:
                kind, h = mv[0], mv[1]
                if h not in names:
                    continue
                try:
                    if kind == "append":
                        where = al.append(names[h], mv[2])
                        for b, s in where:
                            sh.slots[(b, s)] = sh.uid; sh.hist[h].append(sh.uid); sh.uid += 1
                    elif kind == "fork":
                        for c in al.fork(names[h], mv[2]):
                            if nxt < 3:
                                names[nxt] = c; sh.hist[nxt] = list(sh.hist[h]); nxt += 1
                            else:
                                al.release(c)
                    elif kind == "release":
                        al.release(names.pop(h)); del sh.hist[h]
                    else:
                        L = min(mv[2], len(sh.hist[h]))
                        al.truncate(names[h], L); sh.hist[h] = sh.hist[h][:L]
                except A.OracleError as e:
                    assert e.code in ("nomem", "shared")
                _check_invariants(al, sh, names)
            count += 1
    return count


def test_exhaustive_short_sequences():
    assert _exhaustive(max_len=4) > 100000


# ---------------------------------------------------------------------------
# planted mistakes

class _NonStickyFreeze(A.FlatAllocator):
    def _drop_block(self, b):
        super()._drop_block(b)
        if self.share[b] == 1:
            self.frozen[b] = False


class _HighestFree(A.FlatAllocator):
    def _take_block(self):
        b = max(self._free)
        self._free.remove(b)
        import heapq
        heapq.heapify(self._free)
        self.share[b] = 1
        self.frozen[b] = False
        return b


class _NoFreezeOnFork(A.FlatAllocator):
    def fork(self, h, n):
        kids = super().fork(h, n)
        for b, _ in self._table(h):
            self.frozen[b] = False
        return kids


class _TruncateIgnoresFrozen(A.FlatAllocator):
    def truncate(self, h, new_len):
        saved = list(self.frozen)
        self.frozen = [False] * self.num_blocks
        try:
            super().truncate(h, new_len)
        finally:
            self.frozen = saved


class _ForkCountsOnce(A.FlatAllocator):
    def fork(self, h, n):
        kids = super().fork(h, n)
        for b, _ in self._table(h):
            self.share[b] -= n - 1
        return kids


@pytest.mark.parametrize("mutant", [_NonStickyFreeze, _HighestFree, _NoFreezeOnFork,
                                    _TruncateIgnoresFrozen, _ForkCountsOnce],
                         ids=lambda c: c.__name__)
def test_pins_catch_planted_allocator_mistakes(mutant):
    caught = 0
    for pin in (pin_walkthrough, pin_fork_workload_ids, pin_verify_workload_accept,
                lambda cls: _random_session(3, cls=cls)):
        try:
            pin(mutant)
        except (AssertionError, A.OracleError, KeyError, ValueError, IndexError):
            caught += 1
    assert caught > 0
