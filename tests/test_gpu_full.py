"""GPU parity at the full workload sizes, in the launch configuration bench.py times.

The fork, search-tree and verify workloads are compared in full: every query
row and head of the call against the float64 oracle (run on several host
threads, its arithmetic unchanged).  The 32-layer workload is compared in full
on its first layer call and sampled on the other 31 (rows of a few requests
per layer, every head drawn); block tables are compared in full everywhere.
Loops and extreme shapes are sampled; the sample always includes the first and
last rows.
"""

import dataclasses

import numpy as np
import pytest

from workloads import recipes

from _gpu_common import assert_close, oracle_threads, run_both

pytestmark = pytest.mark.gpu


def _sampler(per_op, seed=0):
    def sample(op, nrows):
        rng = np.random.default_rng(seed + op[1])
        wl_heads = sample.heads
        rows = rng.integers(0, nrows, per_op)
        heads = rng.integers(0, wl_heads, per_op)
        pts = list(zip(rows.tolist(), heads.tolist()))
        pts += [(0, 0), (nrows - 1, wl_heads - 1)]
        return sorted(set(pts))
    return sample


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama_fork", "mcts_tree", "spec_verify"])
def test_standard_workload_every_output(name):
    """Every (query row, head) output of the call at full size against the oracle."""
    wl = recipes.STANDARD[name]()
    res = run_both(wl, threads=oracle_threads())
    op = wl.attend_ops()[0]
    rows = sum(op[3]) if op[0] == "verify" else len(op[2])
    assert [n for _, _, n in res] == [rows * wl.q_heads * wl.head_dim]
    assert_close(res, wl.dtype)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,q_scale", [("spec_verify", 2), ("spec_verify", 4), ("llama_fork", 2), ("llama_fork", 4)])
def test_standard_workload_sharp_scores_every_output(name, q_scale):
    """The same at full size with the queries scaled by a power of two: wider
    score spreads, weights gathered on fewer keys, so the P.V step keeps the
    low parts of its bf16 weights on more of the super-blocks."""
    wl = dataclasses.replace(recipes.STANDARD[name](), q_scale=q_scale)
    res = run_both(wl, threads=oracle_threads())
    assert_close(res, wl.dtype)


@pytest.mark.timeout(600)
@pytest.mark.parametrize("part", ["first_layer_whole", "every_layer_sampled"])
def test_full_depth(part):
    """The 32-layer workload (64 requests, 8192-token prefixes forked 16 ways, 256
    tokens per branch; 103 GB of K/V), one decode step of 32 layer calls.
    first_layer_whole: layer 0's call on every one of its 1024 rows x 32 heads.
    every_layer_sampled: each layer's call on 128 (row, head) pairs drawn from
    the rows of 4 requests chosen per layer, every head drawn."""
    wl = recipes.STANDARD["full_depth"]()

    def sample(op, nrows):
        if part == "first_layer_whole":
            return None if op[1] == 0 else []
        rng = np.random.default_rng(100 + op[1])
        reqs = rng.choice(nrows // 16, 4, replace=False)
        rows = (reqs[:, None] * 16 + np.arange(16)[None, :]).reshape(-1)
        pts = [(int(r), int(h)) for r in rows for h in rng.choice(wl.q_heads, 2, replace=False)]
        return sorted(set(pts + [(0, 0), (nrows - 1, wl.q_heads - 1)]))
    res = run_both(wl, sample=sample, threads=oracle_threads())
    if part == "first_layer_whole":
        assert [n for _, _, n in res] == [1024 * 32 * 128]
    else:
        assert len(res) == 32
    assert_close(res, wl.dtype)


@pytest.mark.parametrize("case", ["long_decode", "long_verify", "wide_batch", "gqa8_tree", "wide_batch_f32",
                                  "wide_batch_d64"])
def test_extreme_shapes_sampled(case):
    """Shapes beyond the standard workloads, sampled against the oracle:
    a 40 000-token shared prefix (2500 blocks, cut into many split-K chunks
    and merged); verification over a 30 000-token prefix; 1500 independent
    sequences in one call (1500 groups, 12 000 workgroups); a search tree at
    8 query heads per KV head (cascade subgroups of 2 queries); wide batches
    at fp32 and at d = 64."""
    if case == "long_decode":
        wl = recipes.fork_workload("long_decode", dtype="bf16", layers=1, q_heads=8, kv_heads=2, head_dim=128,
                                   requests=1, prefix=40000, width=3, branch_tokens=17, seed=51)
    elif case == "long_verify":
        wl = recipes.verify_workload("long_verify", dtype="bf16", q_heads=8, kv_heads=2, head_dim=128,
                                     requests=2, prefix=30000, paths=3, drafts=8, seed=52)
    elif case == "wide_batch":
        wl = recipes.fork_workload("wide_batch", dtype="bf16", layers=1, q_heads=32, kv_heads=8, head_dim=128,
                                   requests=1500, prefix=40, width=1, branch_tokens=3, seed=53)
    elif case == "wide_batch_f32":
        # one-tile groups, more workgroups than CUs, short items: the LDS-staged
        # kernel's 4-tile shape at fp32
        wl = recipes.fork_workload("wide_batch_f32", dtype="f32", layers=1, q_heads=16, kv_heads=4, head_dim=128,
                                   requests=600, prefix=70, width=1, branch_tokens=5, seed=55)
    elif case == "wide_batch_d64":
        wl = recipes.fork_workload("wide_batch_d64", dtype="bf16", layers=1, q_heads=16, kv_heads=4, head_dim=64,
                                   requests=600, prefix=70, width=1, branch_tokens=5, seed=56)
    else:
        wl = recipes.mcts_workload("gqa8_tree", dtype="bf16", q_heads=32, kv_heads=4, head_dim=128,
                                   root_tokens=300, branching=4, depth=5, leaves=128, node_tokens=16, seed=54)
    s = _sampler(64, seed=3)
    s.heads = wl.q_heads
    # the search tree at GQA 8 runs with 16-tile groups and the cascade on (subgroups of 2 queries)
    opts = {3: 256, 6: 1} if case == "gqa8_tree" else None
    assert_close(run_both(wl, sample=s, options=opts), wl.dtype)


@pytest.mark.parametrize("kind", ["decode", "verify"])
def test_longest_lds_staged_item(kind):
    """One LDS-staged work item of about 1000 blocks (the block list kernel B
    stages is at most 1024 entries, 16 KiB): with a workgroup target of 2 the
    planner leaves each group whole.  Sampled against the oracle."""
    from tree_structured_copy_amd import tkv
    if kind == "decode":
        wl = recipes.fork_workload("long_item", dtype="bf16", layers=1, q_heads=8, kv_heads=2, head_dim=128,
                                   requests=1, prefix=16000, width=12, branch_tokens=9, seed=61)
    else:
        wl = recipes.verify_workload("long_item_v", dtype="bf16", q_heads=8, kv_heads=2, head_dim=128,
                                     requests=1, prefix=16000, paths=3, drafts=8, seed=62)
    s = _sampler(64, seed=5)
    s.heads = wl.q_heads
    assert_close(run_both(wl, sample=s, options={tkv.TKV_OPT_TARGET_WGS: 2}), wl.dtype)


@pytest.mark.parametrize("fused", [False, True])
def test_fork_workload_decode_loop_sampled(fused):
    """The decode loop bench.py times, at the fork workload's full size (32
    requests x 4096-token prefix forked 4 ways, 64 tokens per branch; GQA 32/8,
    d = 128, bf16), for 3 rounds of one token per branch -- appended in a batch
    then decoded, or reserved and written inside the decode call -- with plans
    updated in place between rounds.  Sampled against the oracle."""
    wl = recipes.decode_loop_workload("llama_loop", layers=1, q_heads=32, kv_heads=8, head_dim=128, requests=32,
                                      prefix=4096, width=4, branch_tokens=64, rounds=3, fused=fused, seed=91)
    s = _sampler(24, seed=7)
    s.heads = wl.q_heads
    res = run_both(wl, sample=s)
    assert len(res) == 3
    assert_close(res, wl.dtype)


@pytest.mark.parametrize("kind", ["spec_loop", "spec_loop_one_launch", "search_loop", "search_loop_one_launch"])
def test_loops_at_full_shape_sampled(kind):
    """The loops bench.py times, at their full shapes: the speculative loop on
    the verify workload's 64 requests (2048-token prefixes, 3 paths of 8
    drafts) for 2 rounds, with the drafts appended then verified or reserved
    and written by the verify call, and 40 tree-search simulations
    (2048-token root, branching 4, depth 12, 16 tokens per node), with each
    expansion's nodes appended then decoded or reserved and written by the
    decode call.
    Sampled against the oracle; tables bit-exact."""
    if kind.startswith("spec_loop"):
        wl = recipes.spec_loop_workload("spec_loop_full", rounds=2, seed=5, one_launch=kind == "spec_loop_one_launch")
        per_op = 64
    else:
        wl = recipes.mcts_loop_workload("search_loop_full", iterations=40, seed=6,
                                        one_launch=kind == "search_loop_one_launch")
        per_op = 16
    s = _sampler(per_op, seed=9)
    s.heads = wl.q_heads
    res = run_both(wl, sample=s)
    assert len(res) == len(wl.attend_ops())
    assert_close(res, wl.dtype)


def test_queued_plan_copies_wait_for_the_launches_before_them():
    """Six verify calls on the verify workload's handles (64 requests x
    2048-token prefix, 3 draft paths of 8 tokens), each over the handles in
    another order, so each builds its own plan of about 200 KB.  All six are
    queued behind a spin kernel, so the host queues them before the first runs:
    the four plan slots are reused (the fifth and sixth plans are copied into
    slots whose earlier plans are still to be read) and the ring of pinned
    staging buffers wraps.  Every output must be bit-identical to that of the
    same call made on an idle GPU."""
    import torch
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    from workloads import device as wdev

    wl = recipes.STANDARD["spec_verify"]()
    lib = LibReplay(wl)
    try:
        op = wl.ops[lib.build()]
        hs = lib.handles(op)
        nq = list(op[3])
        rows = sum(nq)
        q = wdev.q_tensor(wl, op[-1], rows, "cuda")
        batches = [hs[24 * k:] + hs[:24 * k] for k in range(6)]
        outs = [torch.full((rows, wl.q_heads, wl.head_dim), float("nan"), device="cuda") for _ in batches]
        refs = [torch.full((rows, wl.q_heads, wl.head_dim), float("nan"), device="cuda") for _ in batches]
        sizes = [tkv.tkv_workspace_size(lib.c, b, nq) for b in batches]
        ws = [torch.empty(max(n, 1), dtype=torch.uint8, device="cuda") for n in sizes]
        stream = torch.cuda.current_stream()
        torch.cuda.synchronize()
        before = tkv.tkv_get_counters(lib.c)["plans_uploaded"]
        torch.cuda._sleep(20_000_000)
        for b, o, w, n in zip(batches, outs, ws, sizes):
            tkv.tkv_attend_verify(lib.c, 0, b, nq, q, o, w, n, stream)
        torch.cuda.synchronize()
        assert tkv.tkv_get_counters(lib.c)["plans_uploaded"] - before == 6
        for b, o, w, n in zip(batches, refs, ws, sizes):
            tkv.tkv_attend_verify(lib.c, 0, b, nq, q, o, w, n, stream)
            torch.cuda.synchronize()
        for k in range(6):
            assert not torch.isnan(outs[k]).any(), k
            assert torch.equal(outs[k], refs[k]), k
    finally:
        lib.close()
