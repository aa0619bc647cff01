"""The library's host core (C ABI, no GPU) against the oracle's flat allocator.

A host-only cache (no pools) runs the real tree, allocator and planner;
``tkv_append`` without K/V reserves slots only.  Block tables, lengths, sharer
counts, free counts and error codes must equal the oracle's after every step.
"""

import itertools
import json
import os
import random
import re
import time

import pytest

from oracle import allocator as A
from workloads import recipes

tkv = pytest.importorskip("tree_structured_copy_amd.tkv")

GOLD = os.path.join(os.path.dirname(__file__), "golden")
ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

ERR = {"inval": tkv.TKV_E_INVAL, "nomem": tkv.TKV_E_NOMEM, "badseq": tkv.TKV_E_BADSEQ,
       "shared": tkv.TKV_E_SHARED, "range": tkv.TKV_E_RANGE}


def test_library_exports_every_declared_symbol():
    header = open(os.path.join(ROOT, "include", "tkv.h")).read()
    declared = set(re.findall(r"^\s*(?:int|const char\*|size_t)\s+(tkv_\w+)\s*\(", header, re.M))
    assert declared, "no declarations parsed"
    assert declared == set(tkv.EXPORTED)
    for name in declared:
        assert hasattr(tkv._lib, name)


def host_cache(num_blocks, layers=1, hq=4, hkv=4, d=64, dtype=None):
    return tkv.tkv_create(layers, hq, hkv, d, num_blocks, tkv.TKV_F32 if dtype is None else dtype)


class Pair:
    """Library and oracle driven in lockstep over symbolic handle names."""

    def __init__(self, num_blocks):
        self.nb = num_blocks
        self.c = host_cache(num_blocks)
        self.o = A.FlatAllocator(num_blocks, 16)
        self.lh, self.oh = {}, {}

    def close(self):
        tkv.tkv_destroy(self.c)

    def step(self, op):
        """Apply op to both; return (lib error name or None, oracle error name or None)."""
        kind, name = op[0], op[1]
        le = oe = None
        try:
            if kind == "new":
                self.lh[name] = tkv.tkv_seq_new(self.c)
            elif kind == "append":
                tkv.tkv_append(self.c, self.lh.get(name, 0), op[2])
            elif kind == "fork":
                kids = tkv.tkv_fork(self.c, self.lh.get(name, 0), op[2])
                for k, s in zip(op[3], kids):
                    self.lh[k] = s
            elif kind == "release":
                tkv.tkv_release(self.c, self.lh.get(name, 0))
                self.lh.pop(name, None)
            elif kind == "truncate":
                tkv.tkv_truncate(self.c, self.lh.get(name, 0), op[2])
        except tkv.TkvError as e:
            le = e.name
        try:
            if kind == "new":
                self.oh[name] = self.o.seq_new()
            elif kind == "append":
                self.o.append(self.oh.get(name, -1), op[2])
            elif kind == "fork":
                kids = self.o.fork(self.oh.get(name, -1), op[2])
                for k, s in zip(op[3], kids):
                    self.oh[k] = s
            elif kind == "release":
                self.o.release(self.oh.get(name, -1))
                self.oh.pop(name, None)
            elif kind == "truncate":
                self.o.truncate(self.oh.get(name, -1), op[2])
        except A.OracleError as e:
            oe = e.code
        return le, oe

    def compare(self):
        assert set(self.lh) == set(self.oh)
        for name in self.lh:
            assert tkv.tkv_block_table(self.c, self.lh[name]) == self.o.table(self.oh[name]), name
            assert tkv.tkv_seq_len(self.c, self.lh[name]) == self.o.length(self.oh[name])
        assert tkv.tkv_num_free(self.c) == self.o.num_free()
        assert tkv.tkv_block_refcounts(self.c, self.nb) == [self.o.sharers(b) for b in range(self.nb)]


def test_walkthrough_scaled_to_block_16():
    """The hand-derived block-size-4 walkthrough with every token count x4 runs
    unchanged at block size 16."""
    g = json.load(open(os.path.join(GOLD, "alloc_walkthrough.json")))
    p = Pair(g["num_blocks"])
    try:
        for st in g["steps"]:
            op = list(st["op"])
            if op[0] in ("append", "truncate"):
                op[2] *= 4
            le, oe = p.step(op)
            assert le == oe == st.get("error"), (op, le, oe)
            want = {k: [(b, 4 * v) for b, v in t] for k, t in st["tables"].items()}
            got = {k: tkv.tkv_block_table(p.c, s) for k, s in p.lh.items()}
            assert got == want, op
            assert tkv.tkv_num_free(p.c) == st["free"]
            assert tkv.tkv_block_refcounts(p.c, g["num_blocks"]) == st["sharers"]
            p.compare()
    finally:
        p.close()


def _random_ops(seed, n_ops, nb):
    rnd = random.Random(seed)
    live, nxt, ops = [], 0, []
    for _ in range(n_ops):
        r = rnd.random()
        if not live or r < 0.07:
            ops.append(("new", nxt)); live.append(nxt); nxt += 1
        elif r < 0.27:
            h = rnd.choice(live); n = rnd.randint(1, 3)
            kids = list(range(nxt, nxt + n)); nxt += n
            ops.append(("fork", h, n, kids)); live += kids
        elif r < 0.62:
            ops.append(("append", rnd.choice(live), rnd.choice([1, 2, 5, 15, 16, 17, 31, 40, 64])))
        elif r < 0.78:
            h = rnd.choice(live); ops.append(("release", h)); live.remove(h)
        elif r < 0.95:
            ops.append(("truncate", rnd.choice(live), rnd.randint(0, 300)))
        else:  # stale / bad arguments
            ops.append(rnd.choice([("append", rnd.choice(live), 0), ("fork", rnd.choice(live), 0, []),
                                   ("truncate", rnd.choice(live), -1), ("release", 10 ** 6)]))
    return ops


@pytest.mark.parametrize("seed", range(16))
def test_random_differential(seed):
    nb = 40
    p = Pair(nb)
    try:
        for op in _random_ops(seed, 300, nb):
            if op[0] == "truncate" and op[1] in p.oh:
                L = p.o.length(p.oh[op[1]])
                if op[2] > L and op[2] != -1:
                    op = ("truncate", op[1], L if random.Random(op[2]).random() < 0.3 else op[2] % (L + 1))
            le, oe = p.step(op)
            assert le == oe, (op, le, oe)
            p.compare()
    finally:
        p.close()


def test_exhaustive_short_sequences():
    """Every sequence of up to 4 moves over 3 handle names on a 4-block pool."""
    moves = []
    for h in range(3):
        moves += [("append", h, 4), ("append", h, 20), ("fork", h, 1, None), ("fork", h, 2, None),
                  ("release", h), ("truncate", h, 4), ("truncate", h, 0)]
    count = 0
    for length in range(1, 5):
        for seq in itertools.product(moves, repeat=length):
            p = Pair(4)
            try:
                p.step(("new", 0))
                nxt = 1
                for mv in seq:
                    if mv[1] not in p.lh:
                        continue
                    if mv[0] == "fork":
                        kids = list(range(nxt, nxt + mv[2])); nxt += mv[2]
                        mv = ("fork", mv[1], mv[2], kids)
                    if mv[0] == "truncate":
                        L = p.o.length(p.oh[mv[1]])
                        mv = ("truncate", mv[1], min(mv[2], L))
                    le, oe = p.step(mv)
                    assert le == oe, (seq, mv, le, oe)
                p.compare()
            finally:
                p.close()
            count += 1
    assert count == sum(21 ** k for k in range(1, 5))


@pytest.mark.parametrize("name", ["tiny_fork", "llama_fork", "mcts_tree", "spec_verify", "full_depth"])
def test_standard_recipes_match_oracle(name):
    wl = recipes.STANDARD[name]()
    c = host_cache(wl.num_blocks, wl.layers, wl.q_heads, wl.kv_heads, wl.head_dim)
    o = A.FlatAllocator(wl.num_blocks, 16)
    lh, oh = {}, {}
    try:
        for op in wl.ops:
            k = op[0]
            if k == "new":
                lh[op[1]] = tkv.tkv_seq_new(c); oh[op[1]] = o.seq_new()
            elif k == "append":
                tkv.tkv_append(c, lh[op[1]], op[2]); o.append(oh[op[1]], op[2])
            elif k == "fork":
                for n, s, t in zip(op[3], tkv.tkv_fork(c, lh[op[1]], op[2]), o.fork(oh[op[1]], op[2])):
                    lh[n], oh[n] = s, t
            elif k == "release":
                tkv.tkv_release(c, lh.pop(op[1])); o.release(oh.pop(op[1]))
            elif k == "truncate":
                tkv.tkv_truncate(c, lh[op[1]], op[2]); o.truncate(oh[op[1]], op[2])
            else:
                for h in op[2]:
                    assert tkv.tkv_block_table(c, lh[h]) == o.table(oh[h])
                info = tkv.tkv_plan_info_get(c, [lh[h] for h in op[2]], op[3] if k == "verify" else None)
                tabs = {b: v for h in op[2] for b, v in o.table(oh[h])}
                assert info["unique_blocks"] == len(tabs)
                assert info["unique_tokens"] == sum(tabs.values())
        assert tkv.tkv_num_free(c) == o.num_free()
        assert tkv.tkv_block_refcounts(c, wl.num_blocks) == [o.sharers(b) for b in range(wl.num_blocks)]
    finally:
        tkv.tkv_destroy(c)


# ---------------------------------------------------------------------------
# fork cost: O(1) in prefix length and depth

def test_fork_touches_no_block():
    c = host_cache(5000)
    try:
        s = tkv.tkv_seq_new(c)
        tkv.tkv_append(c, s, 16 * 4000 + 5)
        before = tkv.tkv_get_counters(c)
        free = tkv.tkv_num_free(c)
        kids = tkv.tkv_fork(c, s, 16)
        after = tkv.tkv_get_counters(c)
        assert tkv.tkv_num_free(c) == free
        for k in ("blocks_taken", "blocks_freed", "block_ids_copied", "nodes_created"):
            assert after[k] == before[k], k
        assert all(tkv.tkv_block_table(c, k) == tkv.tkv_block_table(c, s) for k in kids[:2])
    finally:
        tkv.tkv_destroy(c)


def _median_fork_ns(prefix_tokens, depth, reps=3000):
    c = host_cache(prefix_tokens // 16 + depth + 8)
    try:
        s = tkv.tkv_seq_new(c)
        tkv.tkv_append(c, s, prefix_tokens)
        for _ in range(depth - 1):  # a chain of depth nodes
            s2 = tkv.tkv_fork(c, s, 1)[0]
            tkv.tkv_release(c, s)
            s = s2
            tkv.tkv_append(c, s, 1)
        f = tkv._lib.tkv_fork
        out = (tkv._U64 * 1)()
        times = []
        for _ in range(reps):
            t0 = time.perf_counter_ns()
            f(c, s, 1, out)
            times.append(time.perf_counter_ns() - t0)
            tkv._lib.tkv_release(c, out[0])
        times.sort()
        return times[len(times) // 2]
    finally:
        tkv.tkv_destroy(c)


def test_fork_bench_flat_over_prefix_and_depth():
    """The C++ fork benchmark: per n, the slowest (prefix, depth) point is within
    3x (+50 ns) of the fastest, over prefix 16..65536 tokens and depth 1..500."""
    import json
    import subprocess
    exe = os.path.join(ROOT, "tree_structured_copy_amd", "fork_bench")
    if not os.path.exists(exe):
        pytest.skip("fork_bench not built")
    grid = json.loads(subprocess.run([exe, "100"], capture_output=True, text=True, timeout=120, check=True).stdout)
    assert len(grid) >= 40
    for n in (1, 4, 16):
        vals = [v for k, v in grid.items() if k.endswith(":%d" % n)]
        assert max(vals) < 3 * min(vals) + 50, (n, min(vals), max(vals))


def _host_check(tmp_path, src, sanitize):
    """Compile a host checker against the library's host sources (tree.cpp,
    plan.cpp), with g++ alone, optionally under AddressSanitizer and
    UndefinedBehaviorSanitizer (any report aborts)."""
    import shutil
    import subprocess
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    csrc = os.path.join(ROOT, "tree_structured_copy_amd", "csrc")
    exe = str(tmp_path / (os.path.splitext(src)[0] + ("_san" if sanitize else "")))
    flags = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-fno-omit-frame-pointer"] if sanitize else ["-O1"]
    subprocess.run([cxx] + flags + ["-std=c++17", "-I" + csrc, "-I" + os.path.join(ROOT, "include"),
                                    os.path.join(ROOT, "tests", src), os.path.join(csrc, "tree.cpp"),
                                    os.path.join(csrc, "plan.cpp"), "-o", exe], check=True, timeout=300)
    return exe


@pytest.mark.parametrize("sanitize", [False, True])
def test_plan_update_in_place_equals_rebuild(tmp_path, sanitize):
    """The planner's in-place update after appends that fit in tip blocks
    (patch_plan): over 60 seeded random fork/append/truncate/release sessions
    with random planner options, 12 rounds each of such appends, the updated
    plan equals a fresh build byte for byte, and its list of changed words,
    written over the previous bytes (what the device copy receives), gives the
    same bytes (tests/plan_patch_check.cpp); also built with ASan + UBSan."""
    import subprocess
    exe = _host_check(tmp_path, "plan_patch_check.cpp", sanitize)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "60"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "all sessions ok: 720 rounds" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    words = int(re.search(r"(\d+) changed words", r.stdout).group(1))
    assert words > 1000


@pytest.mark.parametrize("sanitize", [False, True])
def test_plan_means_what_the_tree_says(tmp_path, sanitize):
    """What the planner's output means, checked from the tree alone over 120
    seeded random sessions with random planner options (row limit 16..256,
    one-tile subgroups on or off, 1..16 query heads per KV head, chunk floors,
    workgroup targets): every query sees exactly its own path's (block, slot)
    pairs up to its position once; items cover their groups' lists; each
    query's output is written directly once or merged from one record per
    item at that item's slot, no slot shared; the layout's sections are
    disjoint (tests/plan_semantics_check.cpp); also built with ASan + UBSan."""
    import subprocess
    exe = _host_check(tmp_path, "plan_semantics_check.cpp", sanitize)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe, "120"], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-3000:])
    assert "all sessions ok" in r.stdout
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr
    assert sum("cascade 1 ok" in line for line in r.stdout.splitlines()) > 20


_PLANTED_PLANNER_MISTAKES = [
    # a block's first position off by one
    ("out[b].pos = pos0 + 16 * b;", "out[b].pos = pos0 + 16 * b + 1;"),
    # a tip block counted full
    ("out[nb - 1].valid = nd.tail_valid();", "out[nb - 1].valid = 16;"),
    # a merge record's slot without the KV-head stride
    ("P.parts.push_back({P.items[item].part_base + j * q_per_kv * num_kv_heads, item});",
     "P.parts.push_back({P.items[item].part_base + j * q_per_kv, item});"),
    # a visibility bit given to the wrong query of a pair
    ("bits |= 1ull << j1;", "bits |= 1ull << (j1 / 2 * 2);"),
]


@pytest.mark.parametrize("planted", range(len(_PLANTED_PLANNER_MISTAKES)))
def test_plan_checker_catches_planted_mistakes(tmp_path, planted):
    """The planner checker has the power to fail: each mistake planted in a
    copy of plan.cpp (a block position off by one, a tip block counted full,
    a merge slot without the KV-head stride, a visibility bit on the wrong
    query) makes tests/plan_semantics_check.cpp report a failure."""
    import shutil
    import subprocess
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    csrc = os.path.join(ROOT, "tree_structured_copy_amd", "csrc")
    src = open(os.path.join(csrc, "plan.cpp")).read()
    old, new = _PLANTED_PLANNER_MISTAKES[planted]
    assert src.count(old) == 1, old
    mutated = tmp_path / "plan_planted.cpp"
    mutated.write_text(src.replace(old, new))
    exe = str(tmp_path / "psc_planted")
    subprocess.run([cxx, "-O1", "-std=c++17", "-I" + csrc, "-I" + os.path.join(ROOT, "include"),
                    os.path.join(ROOT, "tests", "plan_semantics_check.cpp"), os.path.join(csrc, "tree.cpp"),
                    str(mutated), "-o", exe], check=True, timeout=300)
    r = subprocess.run([exe, "100"], capture_output=True, text=True, timeout=300)
    assert r.returncode != 0 or "all sessions ok" not in r.stdout, r.stdout[-1000:]


def test_shape_epoch_only_moves_on_structural_change():
    """Appends that fit in the tip node's last block leave the tree's shape
    unchanged, so a cached plan is updated rather than rebuilt; a new block, a
    fork, a truncation or a release changes it (observed through the plan
    counters of a host-only cache: tkv_plan_info_get goes through the cache)."""
    from tree_structured_copy_amd import tkv
    c = host_cache(64)
    try:
        p = tkv.tkv_seq_new(c)
        tkv.tkv_append(c, p, 20)
        kids = tkv.tkv_fork(c, p, 2)
        tkv.tkv_release(c, p)
        for k in kids:
            tkv.tkv_append(c, k, 3)

        def info():
            tkv.tkv_plan_info_get(c, kids)
            return tkv.tkv_get_counters(c)

        base = info()
        tkv.tkv_append(c, kids[0], 5)      # 8 of 16: same block
        tkv.tkv_append(c, kids[1], 13)     # 16 of 16: same block
        a = info()
        assert a["plans_built"] == base["plans_built"] and a["plans_patched"] == base["plans_patched"] + 1
        assert tkv.tkv_plan_info_get(c, kids)["unique_tokens"] == 20 + 8 + 16
        tkv.tkv_append(c, kids[1], 1)      # opens a block
        b = info()
        assert b["plans_built"] == a["plans_built"] + 1 and b["plans_patched"] == a["plans_patched"]
        tkv.tkv_set_option(c, tkv.TKV_OPT_PLAN_PATCH, 0)
        tkv.tkv_append(c, kids[0], 1)
        d = info()
        assert d["plans_built"] == b["plans_built"] + 1 and d["plans_patched"] == b["plans_patched"]
        assert tkv.tkv_get_option(c, tkv.TKV_OPT_PLAN_PATCH) == 0
        with pytest.raises(tkv.TkvError):
            tkv.tkv_set_option(c, tkv.TKV_OPT_PLAN_PATCH, 2)
    finally:
        tkv.tkv_destroy(c)


@pytest.mark.parametrize("seed", range(12))
def test_append_batch_is_the_appends_in_order(seed):
    """tkv_append_batch over distinct handles gives the tables, lengths, sharer
    counts and free set of the oracle allocator appending to each handle in
    batch order (seeded random sessions; a batch over a random subset of live
    handles with random counts, some opening blocks and nodes)."""
    rng = random.Random(7000 + seed)
    p = Pair(400)
    try:
        names = [0]
        p.step(("new", 0))
        nxt = 1
        for _ in range(40):
            h = rng.choice(names)
            c = rng.random()
            if c < 0.4:
                p.step(("append", h, rng.randint(1, 40)))
            elif c < 0.7 and len(names) < 16:
                kids = list(range(nxt, nxt + rng.randint(1, 3)))
                nxt += len(kids)
                p.step(("fork", h, len(kids), kids))
                names += kids
            elif len(names) > 3:
                p.step(("release", h))
                names.remove(h)
            for _ in range(2):
                sub = rng.sample(names, rng.randint(1, len(names)))
                ns = [rng.choice([1, 1, 2, 7, 16, 23]) for _ in sub]
                tkv.tkv_append_batch(p.c, [p.lh[x] for x in sub], ns)
                for x, n in zip(sub, ns):
                    p.o.append(p.oh[x], n)
                p.compare()
    finally:
        p.close()


def test_append_batch_refusals_change_nothing():
    """A repeated handle or a zero count (TKV_E_INVAL), a stale handle
    (TKV_E_BADSEQ) and a batch the free blocks cannot hold (TKV_E_NOMEM) are
    refused before any handle changes, even when the failing handle comes
    last."""
    c = host_cache(10)
    try:
        a = tkv.tkv_seq_new(c)
        b = tkv.tkv_seq_new(c)
        tkv.tkv_append(c, a, 5)
        dead = tkv.tkv_seq_new(c)
        tkv.tkv_release(c, dead)

        def state():
            return (tkv.tkv_block_table(c, a), tkv.tkv_block_table(c, b), tkv.tkv_num_free(c))

        before = state()
        for seqs, ns, err in [([a, b, a], [1, 1, 1], "inval"), ([a, b], [3, 0], "inval"),
                              ([a, b, dead], [1, 1, 1], "badseq"), ([a, b], [11, 16 * 9 + 1], "nomem")]:
            with pytest.raises(tkv.TkvError) as ei:
                tkv.tkv_append_batch(c, seqs, ns)
            assert ei.value.name == err
            assert state() == before
        tkv.tkv_append_batch(c, [b, a], [16 * 9, 11])   # exactly fits: b takes the 9 free blocks, a's tail holds 11
        assert tkv.tkv_num_free(c) == 0
        assert tkv.tkv_seq_len(c, a) == 16 and tkv.tkv_seq_len(c, b) == 144
    finally:
        tkv.tkv_destroy(c)


@pytest.mark.parametrize("kind", ["spec_loop", "spec_loop_one_launch", "mcts_loop", "mcts_loop_one_launch"])
def test_replay_bench_host_mode_matches_the_oracle(kind, tmp_path):
    """The native replayer (replay_bench), run host-only on the loop recipes
    (with the new tokens appended before the attention calls, or reserved and
    written by them):
    its block high-water mark after time_begin equals the oracle allocator's
    over the same operations, its call, query, token and fork counts equal the
    recipe's, and its full-copy figure is the sum over forks of n x the
    parent's length (oracle lengths) x bytes per token."""
    import subprocess
    exe = os.path.join(ROOT, "tree_structured_copy_amd", "replay_bench")
    if not os.path.exists(exe):
        pytest.skip("replay_bench not built")
    one = kind.endswith("one_launch")
    if kind.startswith("spec_loop"):
        wl = recipes.spec_loop_workload("s", requests=5, prefix=40, paths=3, drafts=5, rounds=6, seed=3,
                                        one_launch=one)
    else:
        wl = recipes.mcts_loop_workload("m", root_tokens=40, branching=3, depth=4, iterations=60,
                                        node_tokens=5, seed=4, one_launch=one)
    path = tmp_path / "ops.txt"
    path.write_text(recipes.ops_text(wl))
    r = subprocess.run([exe, str(path), "--host"], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    got = json.loads(r.stdout)
    o = A.FlatAllocator(wl.num_blocks, 16)
    names = {}
    timed = False
    peak = 0
    full_copy = forks = queries = vtokens = calls = appended = 0
    for op in wl.ops:
        k = op[0]
        if k == "time_begin":
            timed = True
            peak = wl.num_blocks - o.num_free()
            continue
        if k == "new":
            names[op[1]] = o.seq_new()
        elif k == "append":
            o.append(names[op[1]], op[2])
            appended += op[2] if timed else 0
        elif k in ("append_batch", "reserve_batch"):
            ns = op[2] if k == "append_batch" else (op[3] if len(op) > 3 else [1] * len(op[1]))
            for h, n in zip(op[1], ns):
                o.append(names[h], n)
            appended += sum(ns) if timed else 0
        elif k == "fork":
            if timed:
                full_copy += op[2] * o.length(names[op[1]])
                forks += 1
            for c, s in zip(op[3], o.fork(names[op[1]], op[2])):
                names[c] = s
        elif k == "release":
            o.release(names.pop(op[1]))
        elif k == "truncate":
            o.truncate(names[op[1]], op[2])
        elif k in ("decode", "decode_new"):
            calls += 1
            queries += len(op[2])
        elif k in ("verify", "verify_new"):
            calls += 1
            vtokens += sum(op[3])
        if timed:
            peak = max(peak, wl.num_blocks - o.num_free())
    token_bytes = wl.layers * wl.kv_heads * wl.head_dim * wl.elem_bytes * 2
    assert got["peak_blocks"] == peak
    assert got["attend_calls"] == calls and got["decode_queries"] == queries and got["verify_tokens"] == vtokens
    assert got["forks"] == forks and got["appended_tokens"] == appended
    assert got["full_copy_bytes"] == full_copy * token_bytes
    # host mode runs no attention call but plans each one (a cached plan may serve one)
    assert 0 < got["plans_built"] <= calls and got["plans_uploaded"] == 0


def test_fork_and_node_creation_do_not_scale_with_tree_size():
    """fork and a node-creating append cost about the same beside 20 000 live
    handles and nodes as beside a handful (each handle or node added must not
    move every existing one: growth is geometric)."""
    def per_step_us(live):
        c = host_cache(live + 2600)
        try:
            root = tkv.tkv_seq_new(c)
            tkv.tkv_append(c, root, 16)
            if live > 1:
                many = tkv.tkv_fork(c, root, live)
                tkv.tkv_append_batch(c, many, [1] * live)   # one node each
            h = tkv.tkv_fork(c, root, 1)[0]
            ones = tkv.i32_array([1] * 4)
            # the children are kept, so the handle and node tables grow as in a search
            best = float("inf")
            for _ in range(3):
                t0 = time.perf_counter()
                for _ in range(200):
                    kids = tkv.tkv_fork(c, h, 4)
                    tkv.tkv_append_batch(c, kids, ones)
                best = min(best, (time.perf_counter() - t0) / 200 * 1e6)
            return best
        finally:
            tkv.tkv_destroy(c)
    small, large = per_step_us(4), per_step_us(20000)
    assert large < 3 * small + 5, (small, large)


def test_fork_latency_flat_in_prefix_and_depth():
    base = _median_fork_ns(16, 1)
    for prefix, depth in [(65536, 1), (16, 500), (65536, 500)]:
        assert _median_fork_ns(prefix, depth) < 3 * base + 2000


# ---------------------------------------------------------------------------
# errors

def test_error_codes_and_strong_guarantee():
    c = host_cache(4)
    try:
        s = tkv.tkv_seq_new(c)
        tkv.tkv_append(c, s, 40)  # 3 blocks
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_append(c, s, 9 + 16)  # 8 slots left in the tail + needs 2 blocks, 1 free
        assert e.value.code == tkv.TKV_E_NOMEM
        assert tkv.tkv_seq_len(c, s) == 40 and tkv.tkv_num_free(c) == 1
        for bad, code in [(lambda: tkv.tkv_fork(c, s, 0), tkv.TKV_E_INVAL),
                          (lambda: tkv.tkv_append(c, s, 0), tkv.TKV_E_INVAL),
                          (lambda: tkv.tkv_truncate(c, s, 41), tkv.TKV_E_RANGE),
                          (lambda: tkv.tkv_release(c, s + 1), tkv.TKV_E_BADSEQ),
                          (lambda: tkv.tkv_release(c, 0), tkv.TKV_E_BADSEQ),
                          (lambda: tkv.tkv_attend_decode(c, 0, [s], 1, 1), tkv.TKV_E_NODEVICE),
                          (lambda: tkv.tkv_gather(c, s, 0, 1, 1), tkv.TKV_E_NODEVICE),
                          (lambda: tkv.tkv_set_option(c, tkv.TKV_OPT_MAX_ROWS, 8), tkv.TKV_E_RANGE),
                          (lambda: tkv.tkv_set_option(c, tkv.TKV_OPT_CASCADE, 2), tkv.TKV_E_RANGE),
                          (lambda: tkv.tkv_set_option(c, tkv.TKV_OPT_CONCURRENT, 2), tkv.TKV_E_RANGE),
                          (lambda: tkv.tkv_set_option(c, tkv.TKV_OPT_CONCURRENT, -1), tkv.TKV_E_RANGE),
                          (lambda: tkv.tkv_set_option(c, 99, 1), tkv.TKV_E_INVAL)]:
            with pytest.raises(tkv.TkvError) as e:
                bad()
            assert e.value.code == code
        k = tkv.tkv_fork(c, s, 1)[0]
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_truncate(c, k, 39)
        assert e.value.code == tkv.TKV_E_SHARED
        tkv.tkv_release(c, s)
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_seq_len(c, s)
        assert e.value.code == tkv.TKV_E_BADSEQ
        e0 = tkv.tkv_seq_new(c)
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_workspace_size(c, [e0])
        assert e.value.code == tkv.TKV_E_EMPTY
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_workspace_size(c, [k], [41])
        assert e.value.code == tkv.TKV_E_RANGE
    finally:
        tkv.tkv_destroy(c)


def test_bad_configs_rejected():
    # block ids must fit 27 bits: 2^27 blocks is the largest pool
    for args in [(0, 4, 4, 64, 10), (1, 4, 3, 64, 10), (1, 4, 4, 96, 10), (1, 4, 4, 64, 0), (1, 4, 4, 64, (1 << 27) + 1)]:
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_create(*args, tkv.TKV_F32)
        assert e.value.code == tkv.TKV_E_INVAL
    with pytest.raises(tkv.TkvError):
        tkv.tkv_create(1, 4, 4, 64, 10, tkv.TKV_F32, k_pool=256, v_pool=None)


def test_plan_shapes():
    """Groups never mix independent trees and hold <= 64 rows; every query is in one group."""
    wl = recipes.llama_fork()
    c = host_cache(wl.num_blocks, 1, 32, 8, 128)
    try:
        h = {}
        for op in wl.ops:
            if op[0] == "new":
                h[op[1]] = tkv.tkv_seq_new(c)
            elif op[0] == "append":
                tkv.tkv_append(c, h[op[1]], op[2])
            elif op[0] == "fork":
                for n, s in zip(op[3], tkv.tkv_fork(c, h[op[1]], op[2])):
                    h[n] = s
            elif op[0] == "release":
                tkv.tkv_release(c, h.pop(op[1]))
        seqs = [h[x] for x in wl.attend_ops()[0][2]]
        info = tkv.tkv_plan_info_get(c, seqs)
        assert info["groups"] == 32
        assert info["unique_blocks"] == 32 * 272
        assert info["block_entries"] == 32 * 272  # each block listed once
        assert info["items_per_kernel"][0] == info["items"]  # 16 rows per group -> 1 tile
        before = tkv.tkv_get_counters(c)["plans_built"]
        tkv.tkv_plan_info_get(c, seqs)
        assert tkv.tkv_get_counters(c)["plans_built"] == before  # cached
    finally:
        tkv.tkv_destroy(c)


def _host_plan(wl, opts=()):
    """The plan summary of the workload's first attention call, planned by a
    host-only cache of the workload's dtype (the planner sizes its LDS-staged
    classes by the kernels' workgroups per CU, which depend on it)."""
    c = host_cache(wl.num_blocks, wl.layers, wl.q_heads, wl.kv_heads, wl.head_dim,
                   tkv.TKV_BF16 if wl.dtype == "bf16" else tkv.TKV_F32)
    try:
        for k, v in opts:
            tkv.tkv_set_option(c, k, v)
        h = {}
        for op in wl.ops:
            if op[0] == "new":
                h[op[1]] = tkv.tkv_seq_new(c)
            elif op[0] == "append":
                tkv.tkv_append(c, h[op[1]], op[2])
            elif op[0] == "fork":
                for n, s in zip(op[3], tkv.tkv_fork(c, h[op[1]], op[2])):
                    h[n] = s
            elif op[0] == "release":
                tkv.tkv_release(c, h.pop(op[1]))
            elif op[0] == "truncate":
                tkv.tkv_truncate(c, h[op[1]], op[2])
            elif op[0] in ("decode", "verify"):
                nq = op[3] if op[0] == "verify" else None
                return tkv.tkv_plan_info_get(c, [h[x] for x in op[2]], nq)
    finally:
        tkv.tkv_destroy(c)


def test_plan_cascade_shapes():
    """The search tree's large groups hand their private (one-leaf) nodes to
    one-tile subgroups: more groups, the same block entries (nothing is listed
    twice more than before), one-tile items; the fork and verify workloads,
    whose groups are small or whose blocks are all wide, are unchanged."""
    wl = recipes.mcts_tree()
    big = [(tkv.TKV_OPT_TARGET_WGS, 256), (tkv.TKV_OPT_MAX_ROWS, 256)]
    on = _host_plan(wl, big + [(tkv.TKV_OPT_CASCADE, 1)])
    off = _host_plan(wl, big + [(tkv.TKV_OPT_CASCADE, 0)])
    assert on["block_entries"] == off["block_entries"]
    assert on["unique_blocks"] == off["unique_blocks"]
    assert on["groups"] > off["groups"]
    assert on["items_per_kernel"][0] > 0 and off["items_per_kernel"][0] == 0
    for name in ("llama_fork", "spec_verify"):
        w = recipes.STANDARD[name]()
        a = _host_plan(w, big + [(tkv.TKV_OPT_CASCADE, 1)])
        b = _host_plan(w, big + [(tkv.TKV_OPT_CASCADE, 0)])
        assert a == b, name
        assert a["partial_slots"] == 0


def test_plan_classes_fill_one_round():
    """Each kernel class is cut to fill the GPU on its own, in exactly one
    round of workgroups where its groups can be cut that fine (two per CU for
    the 4- and 8-tile shapes): the search tree's 10 groups become 64 items
    (512 workgroups for 256 CUs; shared by cost, the leftovers of rounding
    down going to the largest remainders); with 16-tile groups, 32 shared items
    (256 workgroups); groups that already give one workgroup per CU, or that
    cannot be cut below the chunk floor, are left whole (the 32-layer
    workload's 768-block lists fit one item each)."""
    expect = {"llama_fork": [32, 0, 0, 0, 0, 0], "spec_verify": [0, 0, 0, 64, 0, 0],
              "full_depth": [0, 0, 64, 0, 0, 0]}
    for name, ipk in expect.items():
        info = _host_plan(recipes.STANDARD[name](), [(tkv.TKV_OPT_TARGET_WGS, 256)])
        assert info["items_per_kernel"] == ipk, (name, info)
    # the search tree with the defaults: groups of 32 leaves (8 row tiles), one
    # launch of the 8-tile shape, cut to two workgroups per CU
    info = _host_plan(recipes.mcts_tree(), [(tkv.TKV_OPT_TARGET_WGS, 256)])
    ipk = info["items_per_kernel"]
    assert ipk == [0, 0, 0, 0, 64, 0], info
    assert ipk[4] * 8 == 2 * 256
    # with 16-tile groups and the cascade: 32 shared items (256 workgroups) plus
    # the one-tile subgroups
    big = [(tkv.TKV_OPT_MAX_ROWS, 256), (tkv.TKV_OPT_CASCADE, 1)]
    info = _host_plan(recipes.mcts_tree(), [(tkv.TKV_OPT_TARGET_WGS, 256)] + big)
    ipk = info["items_per_kernel"]
    assert ipk[0] > 0 and ipk[5] == 32 and sum(ipk[1:5]) == 0, info
    assert ipk[5] * 8 == 256
    # twice the workgroups asked for: the shared groups are cut about twice as
    # fine, still within one round
    info2 = _host_plan(recipes.mcts_tree(), [(tkv.TKV_OPT_TARGET_WGS, 512)] + big)
    assert 2 * ipk[5] <= info2["items_per_kernel"][5] and info2["items_per_kernel"][5] * 8 <= 512, info2


def test_plan_lds_classes_join_the_largest():
    """With groups of up to 8 row tiles (the default 128 rows), every LDS-staged
    class runs in the largest one's kernel: a search tree whose groups come
    out of 6 and 8 tiles is one launch of the 8-tile shape.  Below a 16-tile
    class only a class with less work joins: the search tree's one 8-tile
    group (30 queries) joins its 16-tile groups with 256-row groups; a
    workload with only 8-tile groups keeps them."""
    # 64 random leaves: the depth-first packing into 32-query groups gives
    # groups of 5-6 and of 7-8 row tiles
    mixed = recipes.mcts_workload("mixed", leaves=64, node_tokens=64)
    info = _host_plan(mixed, [(tkv.TKV_OPT_TARGET_WGS, 256)])
    ipk = info["items_per_kernel"]
    assert ipk[:4] == [0, 0, 0, 0] and ipk[4] == 64 and ipk[5] == 0, info
    on = _host_plan(recipes.mcts_tree(), [(tkv.TKV_OPT_TARGET_WGS, 256), (tkv.TKV_OPT_MAX_ROWS, 256),
                                          (tkv.TKV_OPT_CASCADE, 1)])
    assert on["items_per_kernel"][4] == 0 and on["items_per_kernel"][5] > 0
    wl = recipes.fork_workload("eight", dtype="bf16", layers=1, q_heads=32, kv_heads=8, head_dim=128,
                               requests=2, prefix=300, width=30, branch_tokens=5, seed=3)
    info = _host_plan(wl, [(tkv.TKV_OPT_TARGET_WGS, 256)])
    assert info["items_per_kernel"][4] > 0 and info["items_per_kernel"][5] == 0, info


def test_plan_last_groups_of_a_tree_are_balanced():
    """A tree's queries are packed into groups of at most 32 (128 rows at GQA
    4) in depth-first order, and its last two groups share their queries as
    evenly as a unit boundary allows: a 40-way fork makes two groups of 20
    queries (5 row tiles each, one kernel class), not 32 and 8 (an 8-tile and
    a 2-tile class, two launches)."""
    wl = recipes.fork_workload("fork40", dtype="bf16", layers=1, q_heads=32, kv_heads=8, head_dim=128,
                               requests=8, prefix=4096, width=40, branch_tokens=64)
    info = _host_plan(wl, [(tkv.TKV_OPT_TARGET_WGS, 256)])
    assert info["groups"] == 16, info
    ipk = info["items_per_kernel"]
    assert ipk[3] > 0 and ipk[3] == sum(ipk), info


def test_plan_six_tile_class_fills_one_round():
    """The 6-tile shape's workgroups pair two KV heads, so one round of them is
    twice target_wgs / Hkv items in bf16: a 24-branch fork (96 rows per
    request, 16 requests) is cut into 64 items, 256 workgroups.  fp32 at
    d = 128 runs one KV head per workgroup and one workgroup per CU: 32 items."""
    def fork24(dtype):
        return recipes.fork_workload("fork24", dtype=dtype, layers=1, q_heads=32, kv_heads=8, head_dim=128,
                                     requests=16, prefix=4096, width=24, branch_tokens=64)
    info = _host_plan(fork24("bf16"), [(tkv.TKV_OPT_TARGET_WGS, 256)])
    assert info["items_per_kernel"] == [0, 0, 0, 64, 0, 0], info
    info = _host_plan(fork24("f32"), [(tkv.TKV_OPT_TARGET_WGS, 256)])
    assert info["items_per_kernel"] == [0, 0, 0, 32, 0, 0], info


def test_empty_batch_and_query_counts_rejected():
    """An attention call over no handles is TKV_E_INVAL; a verify query count of
    0 or above the handle's length is TKV_E_RANGE (checked when the plan is
    built, before anything could be launched)."""
    c = host_cache(64, 1, 8, 2, 64)
    try:
        s = tkv.tkv_seq_new(c)
        tkv.tkv_append(c, s, 20)
        for bad, code in [(lambda: tkv.tkv_workspace_size(c, []), tkv.TKV_E_INVAL),
                          (lambda: tkv.tkv_plan_info_get(c, [], None), tkv.TKV_E_INVAL),
                          (lambda: tkv.tkv_workspace_size(c, [s], [0]), tkv.TKV_E_RANGE),
                          (lambda: tkv.tkv_workspace_size(c, [s], [21]), tkv.TKV_E_RANGE)]:
            with pytest.raises(tkv.TkvError) as e:
                bad()
            assert e.value.code == code
        assert tkv.tkv_workspace_size(c, [s], [20]) >= 0  # all 20 positions as queries is fine
    finally:
        tkv.tkv_destroy(c)


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits non-zero with a message, before
    touching a device."""
    import subprocess
    import sys
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
    assert r.stdout.strip() == "" or not r.stdout.strip().startswith("{")


def test_binding_fails_loudly_without_the_library():
    """With libtkv.so absent, importing the binding raises ImportError naming the
    library: there is no fallback path."""
    import subprocess
    import sys
    code = ("import os, sys\n"
            "real = os.path.exists\n"
            "os.path.exists = lambda p: False if str(p).endswith('libtkv.so') else real(p)\n"
            "try:\n"
            "    import tree_structured_copy_amd.tkv\n"
            "except ImportError as e:\n"
            "    print('refused:', e); sys.exit(0)\n"
            "sys.exit(3)\n")
    r = subprocess.run([sys.executable, "-c", code], capture_output=True, text=True, timeout=300, cwd=ROOT)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "libtkv.so is not built" in r.stdout


def test_search_loop_host_work_per_simulation():
    """The host work of a tree-search simulation (descend, fork, release,
    batched append of 4 nodes, and the plan of the decode of the 4 new leaves)
    stays a few microseconds: replay_bench --host over the 500-simulation
    search loop (2048-token root, branching 4, depth 12) builds every call's
    plan, and the median of three passes stays under 15 us per simulation.
    (A per-build rebuild of the planner's tile table once made it 22-34 us.)"""
    import subprocess
    exe = os.path.join(ROOT, "tree_structured_copy_amd", "replay_bench")
    if not os.path.exists(exe):
        pytest.skip("replay_bench not built")
    import tempfile
    wl = recipes.mcts_loop_workload("search_loop")
    with tempfile.NamedTemporaryFile("w", suffix=".ops", delete=False) as f:
        f.write(recipes.ops_text(wl))
        path = f.name
    try:
        walls = []
        for _ in range(3):
            r = subprocess.run([exe, path, "--host"], capture_output=True, text=True, timeout=120)
            assert r.returncode == 0, r.stderr
            d = json.loads(r.stdout)
            assert d["plans_built"] == 500
            walls.append(d["wall_ms"] * 1e3 / 500)
    finally:
        os.unlink(path)
    assert sorted(walls)[1] < 15.0, walls
