"""Workload recipes: the exact sequence of cache calls for each synthetic workload.

A recipe is data: a list of operations over symbolic handle names.  The oracle
and the HIP library each replay the same list with their own implementation.
Every append, decode and verify draws its numbers from ``workloads.gen`` with a
stream of its own.

Operations:

* ``("new", h)``                          -- empty root sequence named ``h``
* ``("append", h, ntok, call)``           -- append ``ntok`` tokens; K values come from
  stream ``(KIND_K, call)`` and V values from ``(KIND_V, call)``, each laid out
  ``[layers][ntok][kv_heads][head_dim]``
* ``("append_batch", [h...], [ntok...], call)`` -- append ``ntok[i]`` tokens to each
  (distinct) ``h[i]`` in one call; the source arrays from stream ``(KIND_K, call)``
  / ``(KIND_V, call)`` are laid out ``[layers][sum ntok][kv_heads][head_dim]``, the
  handles' tokens one after another in list order
* ``("fork", h, n, [c0, ..., c(n-1)])``   -- n children of ``h``; ``h`` stays live
* ``("release", h)``
* ``("truncate", h, new_len)``
* ``("reserve_batch", [h...], call[, [ntok...]])`` -- ``ntok[i]`` tokens (default 1)
  per (distinct) handle, slots only; their K/V are those of a batched append
  ``call`` of those counts, written layer by layer by the ``decode_new`` ops that
  follow
* ``("decode_new", layer, [h...], call, qcall)`` or
  ``("decode_new", layer, [h...], call, [ntok...], qcall)`` -- write layer
  ``layer`` of those tokens' K/V and decode, in one call
  (``tkv_attend_decode_new_token``, or ``tkv_attend_decode_new_tokens`` with counts)
* ``("time_begin",)``                     -- no effect on the cache: where a timed
  replay of a loop starts (after its set-up)
* ``("decode", layer, [h...], qcall)``    -- one query per handle; Q from stream
  ``(KIND_Q, qcall)``, laid out ``[n][q_heads][head_dim]``
* ``("verify", layer, [h...], [nq...], qcall)`` -- the last ``nq[i]`` positions of each
  handle are queries; Q laid out ``[sum nq][q_heads][head_dim]``
* ``("verify_new", layer, [h...], [nq...], call, qcall)`` -- as ``verify``, where the
  queried tokens are the ones ``reserve_batch`` ``call`` reserved with counts ``nq``:
  the call writes layer ``layer`` of their K/V and verifies them
  (``tkv_attend_verify_new_tokens``)

The tree shapes follow the fork-based decoding strategies of the Dendrite
article (ainews.cool, "technical deep dive" and its Table 1: width-4 fork
search, multi-draft speculative decoding), the MCTS run of the Dendrite demo
tape (branching 4, depth 12, head_dim 128) and the predict / verify /
accept-or-rollback loop of the DSpark blog (second layer).  The KV shape of the
bf16 workloads is Llama 3 8B's (32 query heads, 8 KV heads, head_dim 128), the
model the article benchmarks.
"""

from __future__ import annotations

import dataclasses
import itertools
from typing import List, Tuple

from . import gen


@dataclasses.dataclass
class Workload:
    name: str
    dtype: str  # 'f32' | 'bf16'
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    num_blocks: int
    ops: List[tuple]
    seed: int = 0
    block_size: int = 16
    # every query value is multiplied by this power of two (exact in bf16 and
    # fp32): 2 or 4 give score spreads 2 or 4 times wider, weights gathered on
    # fewer keys
    q_scale: int = 1
    # descriptive fields (no effect on replay)
    description: str = ""

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def attend_ops(self):
        return [op for op in self.ops if op[0] in ("decode", "decode_new", "verify", "verify_new")]


class _Names:
    def __init__(self):
        self._c = itertools.count()

    def __call__(self) -> int:
        return next(self._c)


def _blocks_for(ntok: int, bs: int) -> int:
    return (ntok + bs - 1) // bs


def fork_workload(name: str, *, dtype: str, layers: int, q_heads: int, kv_heads: int,
                  head_dim: int, requests: int, prefix: int, width: int, branch_tokens: int,
                  seed: int = 0, extra_blocks: int = 0, description: str = "") -> Workload:
    """Per request: P = new; append(P, prefix); C = fork(P, width); release(P);
    append(C[b], branch_tokens) for each b.  Then one decode over all branches."""
    nm = _Names()
    ops: List[tuple] = []
    call = 0
    leaves = []
    for _ in range(requests):
        p = nm()
        ops.append(("new", p))
        ops.append(("append", p, prefix, call)); call += 1
        kids = [nm() for _ in range(width)]
        ops.append(("fork", p, width, kids))
        ops.append(("release", p))
        for c in kids:
            if branch_tokens > 0:
                ops.append(("append", c, branch_tokens, call)); call += 1
        leaves.extend(kids)
    for layer in range(layers):
        ops.append(("decode", layer, list(leaves), layer))
    bs = 16
    need = requests * (_blocks_for(prefix, bs) + width * _blocks_for(branch_tokens, bs))
    return Workload(name, dtype, layers, q_heads, kv_heads, head_dim, need + extra_blocks, ops,
                    seed=seed, description=description)


def mcts_paths(seed: int, leaves: int, branching: int, depth: int) -> List[Tuple[int, ...]]:
    """``leaves`` distinct uniformly random root-to-leaf paths (``depth`` draws from
    ``[0, branching)`` each; a duplicate path is redrawn), in lexicographic order."""
    if leaves > branching ** depth:
        raise ValueError("more leaves than distinct paths")
    stream = gen.stream_id(gen.KIND_SHAPE, 0)
    seen = set()
    counter = 0
    while len(seen) < leaves:
        path = []
        for _ in range(depth):
            path.append(gen.uniform_int(seed, stream, counter, branching))
            counter += 1
        seen.add(tuple(path))
    return sorted(seen)


def mcts_workload(name: str, *, dtype: str = "bf16", q_heads: int = 32, kv_heads: int = 8,
                  head_dim: int = 128, root_tokens: int = 2048, branching: int = 4,
                  depth: int = 12, leaves: int = 256, node_tokens: int = 16, seed: int = 0,
                  extra_blocks: int = 0, description: str = "") -> Workload:
    """Root: append root_tokens.  Breadth-first by depth: each present node (in
    lexicographic order) is forked into its present children and released, then
    every child gets node_tokens appended (lexicographic order).  Every leaf then
    decodes one query, leaves in lexicographic order."""
    paths = mcts_paths(seed, leaves, branching, depth)
    nm = _Names()
    ops: List[tuple] = []
    call = 0
    root = nm()
    ops.append(("new", root))
    ops.append(("append", root, root_tokens, call)); call += 1
    level = {(): root}
    nodes = 0
    for dpt in range(depth):
        prefixes = sorted({p[: dpt + 1] for p in paths})
        children_of = {}
        for pre in prefixes:
            children_of.setdefault(pre[:-1], []).append(pre)
        nxt = {}
        for parent in sorted(level):
            kids = children_of.get(parent, [])
            if not kids:
                continue
            names = [nm() for _ in kids]
            ops.append(("fork", level[parent], len(kids), names))
            ops.append(("release", level[parent]))
            for pre, h in zip(kids, names):
                nxt[pre] = h
        for pre in sorted(nxt):
            ops.append(("append", nxt[pre], node_tokens, call)); call += 1
            nodes += 1
        level = nxt
    leaf_handles = [level[p] for p in paths]
    ops.append(("decode", 0, leaf_handles, 0))
    bs = 16
    need = _blocks_for(root_tokens, bs) + nodes * _blocks_for(node_tokens, bs)
    return Workload(name, dtype, 1, q_heads, kv_heads, head_dim, need + extra_blocks, ops,
                    seed=seed, description=description)


def verify_workload(name: str, *, dtype: str = "bf16", q_heads: int = 32, kv_heads: int = 8,
                    head_dim: int = 128, requests: int = 64, prefix: int = 2048, paths: int = 3,
                    drafts: int = 8, seed: int = 0, accept: bool = True, extra_blocks: int = 0,
                    description: str = "") -> Workload:
    """Per request: P = new; append(P, prefix); C = fork(P, paths); release(P);
    append(C[b], drafts).  One verify over every path with nq = drafts.  Then,
    per request, path a ~ U{0..paths-1} and k ~ U{0..drafts} are drawn: the
    accepted path is truncated to prefix + k and the others are released."""
    nm = _Names()
    ops: List[tuple] = []
    call = 0
    per_req = []
    for _ in range(requests):
        p = nm()
        ops.append(("new", p))
        ops.append(("append", p, prefix, call)); call += 1
        kids = [nm() for _ in range(paths)]
        ops.append(("fork", p, paths, kids))
        ops.append(("release", p))
        for c in kids:
            ops.append(("append", c, drafts, call)); call += 1
        per_req.append(kids)
    allh = [h for kids in per_req for h in kids]
    ops.append(("verify", 0, allh, [drafts] * len(allh), 0))
    if accept:
        for r, kids in enumerate(per_req):
            st = gen.stream_id(gen.KIND_ACCEPT, r)
            a = gen.uniform_int(seed, st, 0, paths)
            k = gen.uniform_int(seed, st, 1, drafts + 1)
            ops.append(("truncate", kids[a], prefix + k))
            for b, c in enumerate(kids):
                if b != a:
                    ops.append(("release", c))
    bs = 16
    need = requests * (_blocks_for(prefix, bs) + paths * _blocks_for(drafts, bs))
    return Workload(name, dtype, 1, q_heads, kv_heads, head_dim, need + extra_blocks, ops,
                    seed=seed, description=description)


def decode_loop_workload(name: str, *, dtype: str = "bf16", layers: int = 1, q_heads: int = 8,
                         kv_heads: int = 2, head_dim: int = 128, requests: int = 3, prefix: int = 40,
                         width: int = 3, branch_tokens: int = 5, rounds: int = 20, verify_nq: int = 0,
                         batched: bool = True, fused: bool = False, seed: int = 0,
                         description: str = "") -> Workload:
    """A generation loop over the fork workload's tree: per request, P = new;
    append(P, prefix); C = fork(P, width); release(P); append(C[b],
    branch_tokens).  Then ``rounds`` rounds of: append one token to each branch
    except those with (round + branch index) % 3 == 2, then one attention call
    over all branches and every layer -- a decode, or with ``verify_nq`` > 0 a
    verify of each branch's last ``verify_nq`` tokens.  Most rounds' tokens fit
    in the branches' last blocks; now and then one opens a block.  A round's
    appends are one ``append_batch`` (``batched``) or one ``append`` each.
    With ``fused`` (decode only) every branch gets a token each round, reserved
    by one ``reserve_batch`` and written layer by layer by ``decode_new``."""
    nm = _Names()
    ops: List[tuple] = []
    call = 0
    leaves = []
    for _ in range(requests):
        p = nm()
        ops.append(("new", p))
        ops.append(("append", p, prefix, call)); call += 1
        kids = [nm() for _ in range(width)]
        ops.append(("fork", p, width, kids))
        ops.append(("release", p))
        for c in kids:
            ops.append(("append", c, branch_tokens, call)); call += 1
        leaves.extend(kids)
    qcall = 0
    for r in range(rounds):
        if fused:
            ops.append(("reserve_batch", list(leaves), call))
            for layer in range(layers):
                ops.append(("decode_new", layer, list(leaves), call, qcall))
                qcall += 1
            call += 1
            continue
        grow = [c for b, c in enumerate(leaves) if (r + b) % 3 != 2]
        if batched:
            ops.append(("append_batch", grow, [1] * len(grow), call)); call += 1
        else:
            for c in grow:
                ops.append(("append", c, 1, call)); call += 1
        for layer in range(layers):
            if verify_nq > 0:
                ops.append(("verify", layer, list(leaves), [verify_nq] * len(leaves), qcall))
            else:
                ops.append(("decode", layer, list(leaves), qcall))
            qcall += 1
    bs = 16
    need = requests * (_blocks_for(prefix, bs) + width * _blocks_for(branch_tokens + rounds, bs))
    return Workload(name, dtype, layers, q_heads, kv_heads, head_dim, need, ops, seed=seed,
                    description=description or "fork tree, then %d rounds of one-token appends and "
                                               "attention over every branch" % rounds)


def spec_loop_workload(name: str, *, dtype: str = "bf16", q_heads: int = 32, kv_heads: int = 8,
                       head_dim: int = 128, requests: int = 64, prefix: int = 2048, paths: int = 3,
                       drafts: int = 8, rounds: int = 8, seed: int = 0, one_launch: bool = False,
                       description: str = "") -> Workload:
    """The multi-round speculative loop: per request, P = new; append(P, prefix).
    Each round: every request forks P into ``paths`` draft paths and releases P;
    one append_batch gives every path ``drafts`` tokens; one verify covers every
    path's last ``drafts`` tokens; then per request a path a ~ U{0..paths-1}
    and an accepted count k ~ U{0..drafts} are drawn (stream (KIND_ACCEPT,
    100000 * (round + 1) + request)), path a is truncated to len(P) + k, the
    other paths are released, and one append_batch gives every request the
    token the target model emits after its accepted drafts.  Path a is the next
    round's P.  From the second round on the forks fall at unaligned lengths,
    so a fork point's partial block is shared, frozen, and each path's drafts
    start a fresh block.  With ``one_launch`` the drafts are reserved instead
    (``reserve_batch``) and written by the verify call itself (``verify_new``),
    as a target model computes the drafts' K/V in the pass that verifies them."""
    nm = _Names()
    ops: List[tuple] = []
    call = 0
    cur = []
    for _ in range(requests):
        p = nm()
        ops.append(("new", p))
        ops.append(("append", p, prefix, call)); call += 1
        cur.append(p)
    lens = [prefix] * requests
    ops.append(("time_begin",))
    qcall = 0
    for rnd in range(rounds):
        kids = []
        for p in cur:
            ks = [nm() for _ in range(paths)]
            ops.append(("fork", p, paths, ks))
            ops.append(("release", p))
            kids.append(ks)
        allk = [h for ks in kids for h in ks]
        if one_launch:
            ops.append(("reserve_batch", allk, call, [drafts] * len(allk)))
            ops.append(("verify_new", 0, allk, [drafts] * len(allk), call, qcall)); call += 1; qcall += 1
        else:
            ops.append(("append_batch", allk, [drafts] * len(allk), call)); call += 1
            ops.append(("verify", 0, allk, [drafts] * len(allk), qcall)); qcall += 1
        nxt = []
        for r, ks in enumerate(kids):
            st = gen.stream_id(gen.KIND_ACCEPT, 100000 * (rnd + 1) + r)
            a = gen.uniform_int(seed, st, 0, paths)
            k = gen.uniform_int(seed, st, 1, drafts + 1)
            ops.append(("truncate", ks[a], lens[r] + k))
            lens[r] += k + 1
            for b, c in enumerate(ks):
                if b != a:
                    ops.append(("release", c))
            nxt.append(ks[a])
        ops.append(("append_batch", list(nxt), [1] * len(nxt), call)); call += 1
        cur = nxt
    bs = 16
    per_req = _blocks_for(prefix, bs) + 1 + rounds * (paths * (_blocks_for(drafts + 1, bs) + 1) + 1)
    return Workload(name, dtype, 1, q_heads, kv_heads, head_dim, requests * per_req, ops, seed=seed,
                    description=description or "%d rounds of fork, draft, verify, accept or roll back" % rounds)


def mcts_loop_workload(name: str, *, dtype: str = "bf16", q_heads: int = 32, kv_heads: int = 8,
                       head_dim: int = 128, root_tokens: int = 2048, branching: int = 4, depth: int = 12,
                       iterations: int = 500, node_tokens: int = 16, seed: int = 0,
                       one_launch: bool = False, description: str = "") -> Workload:
    """A tree search run as ``iterations`` simulations (the Dendrite demo tape's
    MCTS run: 500 simulations, branching 4, depth 12, head_dim 128): root = new;
    append(root, root_tokens).  A simulation descends from the root, taking at
    every expanded node a child drawn uniformly (stream (KIND_SHAPE, 2)), to
    the first node not yet expanded.  A node at depth ``depth`` is terminal: its
    handle decodes one query.  Any other is expanded: forked into ``branching``
    children and released (the children keep its path), one append_batch gives
    every child ``node_tokens`` tokens, and one decode evaluates the new
    children.  With ``one_launch`` the children's tokens are reserved instead
    (``reserve_batch``) and written by the decode call itself (``decode_new``):
    the same cache contents and outputs, one launch fewer."""
    nm = _Names()
    ops: List[tuple] = []
    call = 0
    qcall = 0
    root = nm()
    ops.append(("new", root))
    ops.append(("append", root, root_tokens, call)); call += 1
    ops.append(("time_begin",))
    children = {}          # expanded node -> its children
    level = {root: 0}      # node -> depth
    stream = gen.stream_id(gen.KIND_SHAPE, 2)
    counter = 0
    expansions = 0
    for _ in range(iterations):
        h = root
        while h in children:
            h = children[h][gen.uniform_int(seed, stream, counter, branching)]
            counter += 1
        if level[h] >= depth:
            ops.append(("decode", 0, [h], qcall)); qcall += 1
            continue
        kids = [nm() for _ in range(branching)]
        ops.append(("fork", h, branching, kids))
        ops.append(("release", h))
        if one_launch:
            ns = [node_tokens] * branching
            ops.append(("reserve_batch", list(kids), call, ns))
            ops.append(("decode_new", 0, list(kids), call, ns, qcall)); call += 1; qcall += 1
        else:
            ops.append(("append_batch", list(kids), [node_tokens] * branching, call)); call += 1
            ops.append(("decode", 0, list(kids), qcall)); qcall += 1
        children[h] = kids
        for c in kids:
            level[c] = level[h] + 1
        expansions += 1
    bs = 16
    need = _blocks_for(root_tokens, bs) + expansions * branching * _blocks_for(node_tokens, bs)
    return Workload(name, dtype, 1, q_heads, kv_heads, head_dim, need, ops, seed=seed,
                    description=description or "%d tree-search simulations, branching %d, depth %d"
                    % (iterations, branching, depth))


def ops_text(wl: Workload) -> str:
    """The recipe as the text the native replayer (replay_bench) reads: a config
    line, then one operation per line, handle names as integers:
    ``config layers q_heads kv_heads head_dim num_blocks dtype(0 f32, 1 bf16)``,
    ``new h``, ``append h ntok``, ``append_batch n h1 n1 ... hn nn``,
    ``fork h n c1 ... cn``, ``release h``, ``truncate h len``, ``time_begin``,
    ``decode layer n h1 ... hn``, ``verify layer n h1 q1 ... hn qn``,
    ``reserve_batch n h1 n1 ... hn nn``, ``decode_new layer n h1 n1 ... hn nn``,
    ``verify_new layer n h1 q1 ... hn qn``.  K/V/Q
    values are not carried: the replayer measures time and memory, while the
    parity tests replay the same recipe against the oracle."""
    if wl.q_scale != 1:
        raise ValueError("the native replayer generates unscaled queries")
    out = ["config %d %d %d %d %d %d" % (wl.layers, wl.q_heads, wl.kv_heads, wl.head_dim, wl.num_blocks,
                                         1 if wl.dtype == "bf16" else 0)]
    for op in wl.ops:
        k = op[0]
        if k == "new":
            out.append("new %d" % op[1])
        elif k == "append":
            out.append("append %d %d" % (op[1], op[2]))
        elif k == "append_batch":
            out.append("append_batch %d %s" % (len(op[1]), " ".join("%d %d" % x for x in zip(op[1], op[2]))))
        elif k == "fork":
            out.append("fork %d %d %s" % (op[1], op[2], " ".join(str(c) for c in op[3])))
        elif k == "release":
            out.append("release %d" % op[1])
        elif k == "truncate":
            out.append("truncate %d %d" % (op[1], op[2]))
        elif k == "time_begin":
            out.append("time_begin")
        elif k == "decode":
            out.append("decode %d %d %s" % (op[1], len(op[2]), " ".join(str(h) for h in op[2])))
        elif k == "verify":
            out.append("verify %d %d %s" % (op[1], len(op[2]), " ".join("%d %d" % x for x in zip(op[2], op[3]))))
        elif k == "reserve_batch":
            ns = op[3] if len(op) > 3 else [1] * len(op[1])
            out.append("reserve_batch %d %s" % (len(op[1]), " ".join("%d %d" % x for x in zip(op[1], ns))))
        elif k == "decode_new":
            ns = op[4] if len(op) > 5 else [1] * len(op[2])
            out.append("decode_new %d %d %s" % (op[1], len(op[2]), " ".join("%d %d" % x for x in zip(op[2], ns))))
        elif k == "verify_new":
            out.append("verify_new %d %d %s" % (op[1], len(op[2]), " ".join("%d %d" % x for x in zip(op[2], op[3]))))
        else:
            raise ValueError(k)
    return "\n".join(out) + "\n"


# ---------------------------------------------------------------------------
# The five standard workloads.

def tiny_fork(seed: int = 0) -> Workload:
    return fork_workload("tiny_fork", dtype="f32", layers=1, q_heads=4, kv_heads=4, head_dim=64,
                         requests=1, prefix=256, width=4, branch_tokens=32, seed=seed,
                         description="fp32, 1 layer, MHA 4/4, d=64; 256-token prefix forked "
                                     "into 4 branches of 32 tokens; 4 decode queries")


def llama_fork(seed: int = 0) -> Workload:
    return fork_workload("llama_fork", dtype="bf16", layers=1, q_heads=32, kv_heads=8, head_dim=128,
                         requests=32, prefix=4096, width=4, branch_tokens=64, seed=seed,
                         description="bf16 GQA 32/8, d=128; 32 requests x (4096-token prefix "
                                     "forked into 4 branches of 64 tokens); 128 decode queries")


def mcts_tree(seed: int = 0) -> Workload:
    return mcts_workload("mcts_tree", seed=seed,
                         description="bf16 GQA 32/8, d=128; 2048-token root; union of 256 random "
                                     "depth-12 paths of a branching-4 tree, 16 tokens per node; "
                                     "256 leaf decode queries")


def spec_verify(seed: int = 0) -> Workload:
    return verify_workload("spec_verify", seed=seed,
                           description="bf16 GQA 32/8, d=128; 64 requests x (2048-token prefix "
                                       "forked into 3 draft paths of 8 tokens); verify 1536 draft "
                                       "queries; accept/rollback by truncation")


def full_depth(seed: int = 0) -> Workload:
    return fork_workload("full_depth", dtype="bf16", layers=32, q_heads=32, kv_heads=8, head_dim=128,
                         requests=64, prefix=8192, width=16, branch_tokens=256, seed=seed,
                         description="bf16, 32 layers of Llama-3-8B KV shape; 64 requests x "
                                     "(8192-token prefix forked into 16 branches of 256 tokens); "
                                     "one decode step per branch over all layers")


STANDARD = {
    "tiny_fork": tiny_fork,
    "llama_fork": llama_fork,
    "mcts_tree": mcts_tree,
    "spec_verify": spec_verify,
    "full_depth": full_depth,
}


def random_tree_workload(name: str, *, seed: int, dtype: str = "bf16", q_heads: int = 8,
                         kv_heads: int = 2, head_dim: int = 128, layers: int = 1, steps: int = 60,
                         num_blocks: int = 400, max_append: int = 40, verify: bool = True) -> Workload:
    """A random session of forks (at unaligned lengths), appends, truncations and
    releases, ending with one decode over every live non-empty handle and, if
    ``verify``, one verify over a subset.  Random choices come from stream
    (KIND_SHAPE, 1000 + seed) so the recipe is reproducible.  Appends that would
    not fit in ``num_blocks`` are skipped, so the recipe never fails."""
    st = gen.stream_id(gen.KIND_SHAPE, 1000 + seed)
    ctr = itertools.count()

    def rnd(n):
        return gen.uniform_int(seed, st, next(ctr), n)

    nm = _Names()
    ops: List[tuple] = []
    call = 0
    live = {}      # name -> length
    frozen_at = {}  # name -> length below which its tokens are shared
    own_blocks = {}  # name -> blocks held by its own node (rough bound for the budget)
    used = 0
    r = nm()
    ops.append(("new", r)); live[r] = 0; frozen_at[r] = 0
    for _ in range(steps):
        names = sorted(live)
        choice = rnd(10)
        h = names[rnd(len(names))]
        if choice < 4:
            n = 1 + rnd(max_append)
            need = (n + 15) // 16 + 1
            if used + need > num_blocks - 2:
                continue
            ops.append(("append", h, n, call)); call += 1
            live[h] += n
            used += need
        elif choice < 6 and len(live) < 24:
            k = 1 + rnd(3)
            kids = [nm() for _ in range(k)]
            ops.append(("fork", h, k, kids))
            frozen_at[h] = live[h]
            for c in kids:
                live[c] = live[h]; frozen_at[c] = live[h]
        elif choice < 8 and live[h] > frozen_at[h]:
            L = frozen_at[h] + rnd(live[h] - frozen_at[h] + 1)
            ops.append(("truncate", h, L)); live[h] = L
        elif len(live) > 2:
            ops.append(("release", h)); del live[h]
    nonempty = [h for h in sorted(live) if live[h] > 0]
    if not nonempty:
        ops.append(("append", r if r in live else sorted(live)[0], 5, call)); call += 1
        nonempty = [r if r in live else sorted(live)[0]]
    for layer in range(layers):
        ops.append(("decode", layer, nonempty, 100 + layer))
    if verify:
        vs = nonempty[::2]
        nqs = [1 + rnd(min(8, live[h])) for h in vs]
        ops.append(("verify", 0, vs, nqs, 200))
    return Workload(name, dtype, layers, q_heads, kv_heads, head_dim, num_blocks, ops, seed=seed,
                    description="random fork/append/truncate/release session")
