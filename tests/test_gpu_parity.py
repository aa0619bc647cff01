"""GPU parity: the HIP path against the oracle, element by element (small sizes).

Sizes are small enough for the float64 oracle to finish in seconds, yet span
several 16-token blocks, several work items, ragged tails, unaligned forks,
truncations, block reuse and both dtypes.  Tolerances: max-abs 1e-5 (fp32) and
2e-3 (bf16 inputs, fp32 accumulation).
"""

import dataclasses

import numpy as np
import pytest

from workloads import gen, recipes

from _gpu_common import TOL, assert_close, need_gpu, run_both, say

pytestmark = pytest.mark.gpu


def test_tiny_fork_fp32_full():
    wl = recipes.tiny_fork()
    assert_close(run_both(wl), "f32")


@pytest.mark.parametrize("dtype,hq,hkv,d", [("bf16", 32, 8, 128), ("bf16", 8, 2, 64), ("f32", 4, 4, 64),
                                            ("f32", 16, 2, 128)])
def test_small_fork_ragged(dtype, hq, hkv, d):
    wl = recipes.fork_workload("small_fork", dtype=dtype, layers=2, q_heads=hq, kv_heads=hkv, head_dim=d,
                               requests=3, prefix=100, width=4, branch_tokens=7, seed=3)
    assert_close(run_both(wl), dtype)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_small_verify(dtype):
    wl = recipes.verify_workload("small_verify", dtype=dtype, q_heads=8, kv_heads=2, head_dim=128,
                                 requests=3, prefix=37, paths=3, drafts=5, seed=5)
    assert_close(run_both(wl), dtype)


@pytest.mark.parametrize("q_scale", [2, 4])
@pytest.mark.parametrize("kind,prefix", [("decode", 37), ("decode", 1100), ("verify", 300), ("verify", 1100)])
def test_sharp_scores(kind, prefix, q_scale):
    """Queries scaled by 2 and 4: score spreads 2 and 4 times wider, so weights
    gather on a few keys, the case in which the P.V step must keep the low
    parts of its bf16 weights; short and long contexts, every output against
    the oracle."""
    if kind == "decode":
        wl = recipes.fork_workload("sharp_fork", dtype="bf16", layers=1, q_heads=16, kv_heads=4, head_dim=128,
                                   requests=3, prefix=prefix, width=4, branch_tokens=21, seed=60 + q_scale)
    else:
        wl = recipes.verify_workload("sharp_verify", dtype="bf16", q_heads=16, kv_heads=4, head_dim=128,
                                     requests=3, prefix=prefix, paths=3, drafts=8, seed=70 + q_scale)
    wl = dataclasses.replace(wl, q_scale=q_scale)
    assert_close(run_both(wl), "bf16")


def test_small_mcts():
    wl = recipes.mcts_workload("small_mcts", q_heads=32, kv_heads=8, head_dim=128, root_tokens=50,
                               branching=3, depth=4, leaves=20, node_tokens=5, seed=7)
    assert_close(run_both(wl), "bf16")


@pytest.mark.parametrize("cascade,dtype,hq,hkv,d", [(1, "bf16", 8, 2, 128), (0, "bf16", 8, 2, 128),
                                                      (1, "f32", 4, 1, 64), (1, "bf16", 16, 8, 64)])
def test_mcts_cascade(cascade, dtype, hq, hkv, d):
    """64 leaves of a branching-4 tree: groups of 16 row tiles whose deep nodes
    are private to one leaf.  With the cascade on, those nodes go to one-tile
    subgroups and every query merges its records from both; off, one group
    reads everything.  Both against the oracle on every row."""
    wl = recipes.mcts_workload("mcts_cascade", dtype=dtype, q_heads=hq, kv_heads=hkv, head_dim=d, root_tokens=70,
                               branching=4, depth=5, leaves=64, node_tokens=9, seed=41 + cascade)
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    need_gpu()
    lib = LibReplay(wl)
    try:
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_MAX_ROWS, 256)
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_CASCADE, cascade)
        i = lib.build()
        op = wl.ops[i]
        info = tkv.tkv_plan_info_get(lib.c, lib.handles(op), None)
        say("plan %s" % info)
        ipk = info["items_per_kernel"]
        if cascade:
            assert ipk[0] > 0 and sum(ipk[4:]) > 0, info
        else:
            assert ipk[0] == 0, info
    finally:
        lib.close()
    assert_close(run_both(wl, options={3: 256, 6: cascade}), dtype)


@pytest.mark.parametrize("mode", [0, 1])
def test_concurrent_modes(mode):
    """The kernel classes of one call run one after another (0) or on side
    streams (1): the same outputs against the oracle in both modes, on a plan
    with one-tile and 16-tile items and a merge (256-row groups with the
    cascade)."""
    from tree_structured_copy_amd import tkv
    wl = recipes.mcts_workload("mcts_modes", dtype="bf16", q_heads=8, kv_heads=2, head_dim=128, root_tokens=70,
                               branching=4, depth=5, leaves=64, node_tokens=9, seed=43)
    opts = {tkv.TKV_OPT_MAX_ROWS: 256, tkv.TKV_OPT_CASCADE: 1, tkv.TKV_OPT_CONCURRENT: mode}
    from tree_structured_copy_amd.replay import LibReplay
    need_gpu()
    lib = LibReplay(wl)
    try:
        for k, v in opts.items():
            tkv.tkv_set_option(lib.c, k, v)
        op = wl.ops[lib.build()]
        ipk = tkv.tkv_plan_info_get(lib.c, lib.handles(op), None)["items_per_kernel"]
        assert ipk[0] > 0 and ipk[5] > 0, ipk
    finally:
        lib.close()
    assert_close(run_both(wl, options=opts), "bf16")


@pytest.mark.parametrize("waves", [2, 4, 8])
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_register_kernel_waves(waves, dtype, d):
    """The one- and two-tile kernel with 2, 4 or 8 waves splitting a group's
    super-blocks (the library keeps 4 where a shape has no 2- or 8-wave form):
    the same results against the oracle."""
    from tree_structured_copy_amd import tkv
    wl = recipes.fork_workload("waves", dtype=dtype, layers=1, q_heads=8, kv_heads=2, head_dim=d,
                               requests=3, prefix=333, width=5, branch_tokens=21, seed=47)
    assert_close(run_both(wl, options={tkv.TKV_OPT_WAVES: waves}), dtype)


@pytest.mark.parametrize("seed", range(8))
def test_random_sessions(seed):
    dtype = "bf16" if seed % 2 == 0 else "f32"
    hq, hkv, d = [(8, 2, 128), (4, 4, 64), (32, 8, 128), (16, 1, 64)][seed % 4]
    wl = recipes.random_tree_workload("rand", seed=seed, dtype=dtype, q_heads=hq, kv_heads=hkv, head_dim=d,
                                      layers=1 + seed % 2)
    assert_close(run_both(wl), dtype)


@pytest.mark.parametrize("opts", [{1: 1}, {1: 100000, 2: 1}, {3: 16}, {3: 32, 2: 2}])
def test_chunking_and_grouping_options(opts):
    """Split-K granularity and group size change only rounding."""
    wl = recipes.fork_workload("opt_fork", dtype="bf16", layers=1, q_heads=32, kv_heads=8, head_dim=128,
                               requests=2, prefix=300, width=6, branch_tokens=20, seed=11)
    assert_close(run_both(wl, options=opts), "bf16")


@pytest.mark.parametrize("max_rows,cls", [(16, 0), (32, 1), (64, 2), (96, 3), (128, 4), (256, 5)])
@pytest.mark.parametrize("kind", ["decode", "verify"])
def test_every_kernel_class(max_rows, cls, kind):
    """Group size decides the kernel: 1-2 row tiles in registers (attn.hip), 3-16
    row tiles with K/V staged in LDS (attn_rows.hip).  Each class against the oracle."""
    if kind == "decode":
        # 64 branches per request: groups of 4, 8, 16, 24 (24, 20, 20 after the
        # last two are balanced), 32 and 64 queries for the six row limits
        wl = recipes.fork_workload("classes", dtype="bf16", layers=1, q_heads=16, kv_heads=4, head_dim=128,
                                   requests=2, prefix=333, width=64, branch_tokens=5, seed=17)
    else:
        wl = recipes.verify_workload("classes_v", dtype="bf16", q_heads=16, kv_heads=4, head_dim=128,
                                     requests=2, prefix=333, paths=8, drafts=7, seed=19)
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    need_gpu()
    lib = LibReplay(wl)
    try:
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_MAX_ROWS, max_rows)
        i = lib.build()
        op = wl.ops[i]
        info = tkv.tkv_plan_info_get(lib.c, lib.handles(op), op[3] if op[0] == "verify" else None)
        assert info["items_per_kernel"][cls] > 0, info
    finally:
        lib.close()
    assert_close(run_both(wl, options={3: max_rows}), "bf16")


@pytest.mark.parametrize("hq,hkv", [(16, 8), (16, 2), (8, 8)])
@pytest.mark.parametrize("kind", ["decode", "verify"])
def test_query_heads_per_kv_head(hq, hkv, kind):
    """GQA ratios 2, 8 and 1 (the other tests use 4, and 16 in random
    sessions): a fork of 12 branches per request and a verify batch of 3
    draft paths x 6 tokens per request, against the oracle on every output."""
    if kind == "decode":
        wl = recipes.fork_workload("gqa_fork", dtype="bf16", layers=1, q_heads=hq, kv_heads=hkv, head_dim=128,
                                   requests=3, prefix=300, width=12, branch_tokens=21, seed=71 + hq + hkv)
    else:
        wl = recipes.verify_workload("gqa_verify", dtype="bf16", q_heads=hq, kv_heads=hkv, head_dim=128,
                                     requests=3, prefix=300, paths=3, drafts=6, seed=73 + hq + hkv)
    assert_close(run_both(wl), "bf16")


@pytest.mark.parametrize("case", ["tree_deep_nodes", "tree_short_nodes", "fork24"])
def test_promoted_classes_and_six_tile_items(case):
    """Groups of different sizes in one launch, and the 6-tile class cut to
    twice the items: a search tree's 64 leaves packed into three groups of
    4-8 row tiles all run in the 8-tile kernel (the smaller groups with idle
    waves); a 24-branch fork's 6-tile groups are cut into 64 items (16 per
    group, merged).  Every output against the oracle."""
    if case == "fork24":
        wl = recipes.fork_workload("fork24", dtype="bf16", layers=1, q_heads=32, kv_heads=8, head_dim=128,
                                   requests=4, prefix=1024, width=24, branch_tokens=40, seed=61)
        want = [0, 0, 0, 64, 0, 0]
    else:
        node = 64 if case == "tree_deep_nodes" else 16
        wl = recipes.mcts_workload(case, leaves=64, node_tokens=node, root_tokens=512,
                                   depth=6 if node == 64 else 12, seed=0 if node == 64 else 2)
        want = [0, 0, 0, 0, 64, 0]
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    need_gpu()
    lib = LibReplay(wl)
    try:
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_TARGET_WGS, 256)
        op = wl.ops[lib.build()]
        info = tkv.tkv_plan_info_get(lib.c, lib.handles(op), None)
        say("plan %s" % info)
        assert info["items_per_kernel"] == want and info["groups"] >= 3, info
    finally:
        lib.close()
    assert_close(run_both(wl, options={tkv.TKV_OPT_TARGET_WGS: 256}), "bf16")


@pytest.mark.parametrize("dtype,hkv,d", [("bf16", 3, 128), ("bf16", 2, 64), ("f32", 2, 64), ("f32", 2, 128)])
def test_six_tile_shapes(dtype, hkv, d):
    """Groups of 6 row tiles run two KV heads per workgroup where the head count
    is even (and fp32 fragments fit), else one: each variant against the oracle."""
    wl = recipes.verify_workload("six", dtype=dtype, q_heads=4 * hkv, kv_heads=hkv, head_dim=d,
                                 requests=3, prefix=200, paths=3, drafts=8, seed=31 + hkv + d)
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    need_gpu()
    lib = LibReplay(wl)
    try:
        i = lib.build()
        op = wl.ops[i]
        info = tkv.tkv_plan_info_get(lib.c, lib.handles(op), op[3])
        assert info["items_per_kernel"][3] > 0, info
    finally:
        lib.close()
    assert_close(run_both(wl), dtype)


def test_many_queries_per_group_mha():
    """MHA with 64 branches: one group of 64 rows (4 row tiles)."""
    wl = recipes.fork_workload("mha64", dtype="bf16", layers=1, q_heads=4, kv_heads=4, head_dim=64,
                               requests=1, prefix=70, width=64, branch_tokens=3, seed=13, extra_blocks=4)
    assert_close(run_both(wl), "bf16")


def test_gather_returns_appended_kv_exactly():
    """tkv_gather reads back, in token order, exactly what the oracle's history holds."""
    torch = need_gpu()
    from oracle.replay import OracleReplay
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    for seed, dtype, hkv, d in [(21, "bf16", 2, 128), (22, "f32", 4, 64), (23, "bf16", 8, 64)]:
        wl = recipes.random_tree_workload("gather", seed=seed, dtype=dtype, q_heads=hkv * 2, kv_heads=hkv,
                                          head_dim=d, layers=2, verify=False)
        say("gather seed %d %s" % (seed, dtype))
        lib, orc = LibReplay(wl), OracleReplay(wl)
        try:
            for op in wl.ops:
                lib.apply(op)
                orc.apply(op)
            for name in lib.h:
                L = tkv.tkv_seq_len(lib.c, lib.h[name])
                if L == 0:
                    continue
                for layer in range(wl.layers):
                    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
                    ko = torch.empty((L, hkv, d), dtype=dt, device="cuda")
                    vo = torch.empty_like(ko)
                    tkv.tkv_gather(lib.c, lib.h[name], layer, ko, vo, torch.cuda.current_stream())
                    torch.cuda.synchronize()
                    for g in range(hkv):
                        K, V = orc.mat.kv(orc.h_mat[name], layer, g)
                        np.testing.assert_array_equal(ko[:, g].float().cpu().numpy(), K)
                        np.testing.assert_array_equal(vo[:, g].float().cpu().numpy(), V)
        finally:
            lib.close()


def test_append_batch_writes_what_the_appends_write():
    """tkv_append_batch over a random session's live handles (1 to 40 tokens
    each, three times, then one batch of more than 240 blocks, which takes two
    launches) leaves in the pool exactly the K/V of the oracle's history, which
    appends to each handle in batch order."""
    import dataclasses
    torch = need_gpu()
    from oracle.replay import OracleReplay
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    for seed, dtype, hkv, d in [(31, "bf16", 2, 128), (32, "f32", 4, 64)]:
        base = recipes.random_tree_workload("abatch", seed=seed, dtype=dtype, q_heads=hkv * 2, kv_heads=hkv,
                                            head_dim=d, layers=2, verify=False)
        live = [op for op in base.ops if op[0] == "decode"][0][2]
        ops = [op for op in base.ops if op[0] != "decode"]
        rng = np.random.default_rng(seed)
        for r in range(3):
            ops.append(("append_batch", list(live), [int(x) for x in rng.integers(1, 41, len(live))], 9000 + r))
        big = -(-250 // len(live)) * 16 + 5
        ops.append(("append_batch", list(live), [big] * len(live), 9003))
        wl = dataclasses.replace(base, ops=ops, num_blocks=base.num_blocks + 700 + 3 * 4 * len(live))
        say("append_batch seed %d %s: %d handles, last batch %d tokens each" % (seed, dtype, len(live), big))
        lib, orc = LibReplay(wl), OracleReplay(wl)
        try:
            for op in wl.ops:
                lib.apply(op)
                orc.apply(op)
            for name in live:
                L = tkv.tkv_seq_len(lib.c, lib.h[name])
                assert tkv.tkv_block_table(lib.c, lib.h[name]) == orc.alloc.table(orc.h_alloc[name])
                for layer in range(wl.layers):
                    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
                    ko = torch.empty((L, hkv, d), dtype=dt, device="cuda")
                    vo = torch.empty_like(ko)
                    tkv.tkv_gather(lib.c, lib.h[name], layer, ko, vo, torch.cuda.current_stream())
                    torch.cuda.synchronize()
                    for g in range(hkv):
                        K, V = orc.mat.kv(orc.h_mat[name], layer, g)
                        np.testing.assert_array_equal(ko[:, g].float().cpu().numpy(), K)
                        np.testing.assert_array_equal(vo[:, g].float().cpu().numpy(), V)
        finally:
            lib.close()


@pytest.mark.parametrize("requests,kv_heads,waves", [(5, 2, 0), (300, 8, 0), (300, 8, 2)])
def test_single_token_is_exact_v(requests, kv_heads, waves):
    """One key: softmax weight 1, so the output is the value itself -- in the
    register kernel (5 sequences; 300 sequences with its wave count forced) and
    in the LDS-staged kernel (300 sequences x 8 KV heads: more workgroups than
    CUs).  9600 rows give scaled scores well above 1, where a weight formed as
    exp2(s * c - m * c) would be off by the rounding of m * c."""
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    from workloads import device as wdev
    wl = recipes.fork_workload("one", dtype="bf16", layers=1, q_heads=4 * kv_heads, kv_heads=kv_heads,
                               head_dim=128, requests=requests, prefix=1, width=1, branch_tokens=0, seed=2)
    lib = LibReplay(wl)
    try:
        lib.build()
        if waves:
            tkv.tkv_set_option(lib.c, tkv.TKV_OPT_WAVES, waves)
        op = wl.attend_ops()[0]
        out = lib.attend(op)
        for i, hname in enumerate(op[2]):
            ko = torch.empty((1, kv_heads, 128), dtype=torch.bfloat16, device="cuda")
            vo = torch.empty_like(ko)
            tkv.tkv_gather(lib.c, lib.h[hname], 0, ko, vo, torch.cuda.current_stream())
            for h in range(4 * kv_heads):
                assert torch.equal(out[i, h], vo[0, h // 4].float())
    finally:
        lib.close()


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_fork_and_identical_siblings_invariance(dtype):
    """Forking a branch does not change its output; siblings with identical K/V
    give identical outputs; permuting the batch permutes the outputs.  Work is
    regrouped between the calls, so only rounding may differ: fp32 within 1e-6,
    bf16 within the bf16 tolerance (the softmax weights are rounded to bf16
    relative to a running max that depends on the processing order)."""
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    from workloads import device as wdev
    tol = 1e-6 if dtype == "f32" else TOL["bf16"]
    hq, hkv, d = 32, 8, 128
    nb = 200
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kp = torch.empty(nb * hkv * 16 * d, dtype=tdt, device="cuda")
    vp = torch.empty_like(kp)
    c = tkv.tkv_create(1, hq, hkv, d, nb, tkv.TKV_BF16 if dtype == "bf16" else tkv.TKV_F32, kp, vp)
    try:
        wl = recipes.fork_workload("inv", dtype=dtype, layers=1, q_heads=hq, kv_heads=hkv, head_dim=d,
                                   requests=1, prefix=1, width=1, branch_tokens=0)
        s = tkv.tkv_seq_new(c)
        k = wdev.kv_tensor(wl, 0, 517, gen.KIND_K)
        v = wdev.kv_tensor(wl, 0, 517, gen.KIND_V)
        tkv.tkv_append(c, s, 517, k, v, torch.cuda.current_stream())
        q = wdev.q_tensor(wl, 0, 4)
        out = torch.empty((1, hq, d), dtype=torch.float32, device="cuda")
        ws = torch.empty(1 << 24, dtype=torch.uint8, device="cuda")
        tkv.tkv_attend_decode(c, 0, [s], q[:1], out, ws, ws.numel(), None)
        before = out.clone()
        kids = tkv.tkv_fork(c, s, 3)
        k2 = wdev.kv_tensor(wl, 1, 9, gen.KIND_K)
        v2 = wdev.kv_tensor(wl, 1, 9, gen.KIND_V)
        for kid in kids[:2]:  # two siblings get identical tokens
            tkv.tkv_append(c, kid, 9, k2, v2, torch.cuda.current_stream())
        tkv.tkv_append(c, kids[2], 3, k2, v2, torch.cuda.current_stream())
        qq = torch.cat([q[:1], q[1:2], q[1:2], q[2:3]])
        out4 = torch.empty((4, hq, d), dtype=torch.float32, device="cuda")
        seqs = [s] + kids
        tkv.tkv_attend_decode(c, 0, seqs, qq, out4, ws, ws.numel(), None)
        torch.cuda.synchronize()
        assert float((out4[0] - before[0]).abs().max()) <= tol
        assert float((out4[1] - out4[2]).abs().max()) <= tol
        perm = [3, 1, 0, 2]
        outp = torch.empty_like(out4)
        tkv.tkv_attend_decode(c, 0, [seqs[i] for i in perm], qq[perm], outp, ws, ws.numel(), None)
        torch.cuda.synchronize()
        assert float((outp - out4[perm]).abs().max()) <= tol
    finally:
        tkv.tkv_destroy(c)


def test_release_then_reuse_same_stream():
    """A released block reused by a later append on the same stream: outputs still
    match the oracle (the stream orders the reads and the overwrite)."""
    wl = recipes.Workload("reuse", "bf16", 1, 8, 2, 128, 12, [
        ("new", 0), ("append", 0, 100, 0), ("fork", 0, 2, [1, 2]), ("append", 1, 40, 1),
        ("decode", 0, [1, 2], 0), ("release", 1), ("append", 2, 45, 2), ("decode", 0, [2, 0], 1),
        ("release", 2), ("release", 0), ("new", 3), ("append", 3, 150, 3), ("decode", 0, [3], 2)])
    assert_close(run_both(wl), "bf16")


def test_workspace_and_argument_errors():
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    kp = torch.empty(64 * 2 * 16 * 128, dtype=torch.bfloat16, device="cuda")
    vp = torch.empty_like(kp)
    c = tkv.tkv_create(1, 8, 2, 128, 64, tkv.TKV_BF16, kp, vp)
    try:
        s = tkv.tkv_seq_new(c)
        k = torch.zeros((1, 700, 2, 128), dtype=torch.bfloat16, device="cuda")
        tkv.tkv_append(c, s, 700, k, k, None)
        kids = tkv.tkv_fork(c, s, 8)
        q = torch.zeros((8, 8, 128), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((8, 8, 128), dtype=torch.float32, device="cuda")
        tkv.tkv_set_option(c, tkv.TKV_OPT_TARGET_WGS, 100000)
        tkv.tkv_set_option(c, tkv.TKV_OPT_MIN_CHUNK, 1)
        need = tkv.tkv_workspace_size(c, kids)
        assert need > 0
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_attend_decode(c, 0, kids, q, out, None, 0, None)
        assert e.value.code == tkv.TKV_E_WORKSPACE
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_attend_decode(c, 1, kids, q, out, None, 0, None)
        assert e.value.code == tkv.TKV_E_RANGE
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_attend_decode(c, 0, kids, q.data_ptr() + 2, out, None, 0, None)
        assert e.value.code == tkv.TKV_E_INVAL
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        tkv.tkv_attend_decode(c, 0, kids, q, out, ws, need, None)
        torch.cuda.synchronize()
        # q = 0 and K = V = 0: every output is exactly 0
        assert float(out.abs().max()) == 0.0
    finally:
        tkv.tkv_destroy(c)


@pytest.mark.parametrize("kind,layers", [("decode", 1), ("verify", 1), ("decode", 2)])
def test_generation_loop_plan_update(kind, layers):
    """A generation loop: 20 rounds of one-token appends to most branches, each
    followed by attention over every branch (and layer).  Every call matches
    the oracle.  Most rounds' appends fit in the branches' last blocks, so the
    cached plan is updated in place (block counts, query positions, their
    minima) rather than rebuilt: the outputs must equal, bit for bit, those of
    a library that rebuilds every such plan, and the counters must show both
    paths taken."""
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    wl = recipes.decode_loop_workload("loop_%s_%d" % (kind, layers), layers=layers,
                                      verify_nq=4 if kind == "verify" else 0, seed=71)
    assert_close(run_both(wl), wl.dtype)
    outs, counters = {}, {}
    for patch in (1, 0):
        lib = LibReplay(wl)
        try:
            tkv.tkv_set_option(lib.c, tkv.TKV_OPT_PLAN_PATCH, patch)
            got = []
            for op in wl.ops:
                if op[0] in ("decode", "verify"):
                    got.append(lib.attend(op).cpu())
                lib.apply(op)
            torch.cuda.synchronize()
            outs[patch] = got
            counters[patch] = tkv.tkv_get_counters(lib.c)
        finally:
            lib.close()
    assert len(outs[1]) == 20 * layers
    for a, b in zip(outs[1], outs[0]):
        assert torch.equal(a, b)
    say("counters with updates %s, without %s" % (counters[1], counters[0]))
    assert counters[0]["plans_patched"] == 0
    assert counters[1]["plans_patched"] >= 10
    assert counters[1]["plans_built"] + counters[1]["plans_patched"] >= 20
    assert counters[1]["plans_built"] < counters[0]["plans_built"]


@pytest.mark.parametrize("kind", ["spec_loop", "spec_loop_one_launch", "mcts_loop", "mcts_loop_one_launch"])
def test_loop_recipes_match_oracle(kind):
    """The multi-round speculative loop (6 rounds of forking at unaligned
    lengths, drafts in fresh blocks, verify, rollback by truncation, a bonus
    token; also with the drafts reserved and written by the verify call) and
    the tree-search loop (60 simulations with terminal re-evaluations; also
    with each expansion's new nodes reserved and written by the decode call),
    replayed through the library: every attention call matches the oracle;
    tables and free blocks are bit-exact."""
    if kind.startswith("spec_loop"):
        wl = recipes.spec_loop_workload("spec_loop_small", q_heads=8, kv_heads=2, requests=5, prefix=40, paths=3,
                                        drafts=5, rounds=6, seed=3, one_launch=kind == "spec_loop_one_launch")
    else:
        wl = recipes.mcts_loop_workload("mcts_loop_small", q_heads=8, kv_heads=2, root_tokens=40, branching=3,
                                        depth=4, iterations=60, node_tokens=5, seed=4,
                                        one_launch=kind == "mcts_loop_one_launch")
    res = run_both(wl)
    assert len(res) == len(wl.attend_ops())
    assert_close(res, wl.dtype)


@pytest.mark.parametrize("route", ["register_kernel", "lds_kernel", "off"])
def test_search_loop_reuses_device_plans_of_the_same_shape(route):
    """A tree-search loop (60 simulations: descend, fork into 3, append a
    node to each child, decode the new leaves): each decode is a new batch,
    and a plan whose device copy differs from a cached one of the same shape
    only in block ids takes that copy over; the ids are rewritten by the
    attention launch (register kernel) or by the patch kernel with the other
    changed words (when the call runs the LDS-staged kernel).  Every call
    matches the oracle, tables bit-exact; with TKV_OPT_PLAN_PATCH = 0 no plan
    is reused."""
    from tree_structured_copy_amd import tkv
    wl = recipes.mcts_loop_workload("mcts_loop_reuse", q_heads=8, kv_heads=2, root_tokens=40, branching=3,
                                    depth=4, iterations=60, node_tokens=5, seed=4)
    opts = {"register_kernel": {}, "lds_kernel": {tkv.TKV_OPT_TARGET_WGS: 4096},
            "off": {tkv.TKV_OPT_PLAN_PATCH: 0}}[route]
    counters = {}
    res = run_both(wl, options=opts, counters=counters)
    assert len(res) == len(wl.attend_ops())
    assert_close(res, wl.dtype)
    if route == "off":
        assert counters["plans_reused"] == 0
    else:
        assert counters["plans_reused"] > 10, counters
        assert counters["plans_uploaded"] + counters["plans_reused"] >= counters["plans_built"]


@pytest.mark.parametrize("one_launch", [1, 0])
@pytest.mark.parametrize("dtype,layers,head_dim", [("bf16", 1, 128), ("bf16", 2, 128), ("f32", 1, 64),
                                                   ("bf16", 1, 64), ("f32", 2, 128)])
def test_decode_with_new_token_written_in_the_call(dtype, layers, head_dim, one_launch):
    """The fused decode step: each round reserves one token per branch
    (tkv_append_batch without K/V), then per layer tkv_attend_decode_new_token
    writes that layer's K/V of the token and decodes -- from the attention
    launch itself (one_launch = 1: TKV_OPT_FUSED_NEW_TOKEN, every call launches
    only attention kernels) or from a preparation launch first.  Every call
    matches the oracle; outputs and pool contents equal, bit for bit, those of
    the same loop run as a batched append with K/V followed by
    tkv_attend_decode."""
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    import dataclasses
    wl = recipes.decode_loop_workload("fused_%s_%d_%d" % (dtype, layers, head_dim), dtype=dtype, layers=layers,
                                      head_dim=head_dim, rounds=14, fused=True, seed=81)
    assert_close(run_both(wl, options={tkv.TKV_OPT_FUSED_NEW_TOKEN: one_launch}), wl.dtype)
    plain_ops = []
    for op in wl.ops:
        if op[0] == "reserve_batch":
            plain_ops.append(("append_batch", op[1], [1] * len(op[1]), op[2]))
        elif op[0] == "decode_new":
            plain_ops.append(("decode", op[1], op[2], op[4]))
        else:
            plain_ops.append(op)
    plain = dataclasses.replace(wl, ops=plain_ops)
    outs, pools = {}, {}
    for key, w in (("fused", wl), ("plain", plain)):
        lib = LibReplay(w)
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_FUSED_NEW_TOKEN, one_launch)
        try:
            got = []
            for op in w.ops:
                if op[0] in ("decode", "decode_new"):
                    got.append(lib.attend(op).cpu())
                    if op[0] == "decode_new":
                        names = tkv.tkv_last_kernels(lib.c)
                        attn = [n for n in names if n.startswith(("attn_partial_kernel", "attn_rows_kernel"))]
                        prep = [n for n in names if n.startswith(("decode_prep_kernel", "plan_patch"))]
                        assert attn, names
                        if one_launch:
                            assert not prep and all("NewTokens" in n for n in attn), names
                        else:
                            assert prep and not any("NewTokens" in n for n in attn), names
                lib.apply(op)
            torch.cuda.synchronize()
            outs[key] = got
            views = {}
            for name in sorted(lib.h):
                L = tkv.tkv_seq_len(lib.c, lib.h[name])
                for layer in range(w.layers):
                    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
                    ko = torch.empty((L, w.kv_heads, w.head_dim), dtype=dt, device="cuda")
                    vo = torch.empty_like(ko)
                    tkv.tkv_gather(lib.c, lib.h[name], layer, ko, vo, torch.cuda.current_stream())
                    views[(name, layer)] = (ko.cpu(), vo.cpu())
            torch.cuda.synchronize()
            pools[key] = views
        finally:
            lib.close()
    assert len(outs["fused"]) == 14 * layers
    for a, b in zip(outs["fused"], outs["plain"]):
        assert torch.equal(a, b)
    assert pools["fused"].keys() == pools["plain"].keys()
    for k in pools["fused"]:
        assert torch.equal(pools["fused"][k][0], pools["plain"][k][0])
        assert torch.equal(pools["fused"][k][1], pools["plain"][k][1])


def _multi_new_token_workload(name, dtype, layers, head_dim, rounds, seed):
    """3 requests (a 37-token prefix forked 3 ways, 6 tokens per branch), then
    ``rounds`` rounds of: every third round the first leaf forks into two
    (their tokens open blocks in new nodes); every leaf reserves n tokens, n
    cycling over 1, 2, 3, 5, 16 but at most what its last block still holds (16
    when its next token opens a block); then per layer one decode_new with
    those counts."""
    ops, nxt, call = [], [0], 0

    def nm():
        nxt[0] += 1
        return nxt[0] - 1
    leaves, free = [], {}
    for _ in range(3):
        p = nm()
        ops += [("new", p), ("append", p, 37, call)]
        call += 1
        kids = [nm() for _ in range(3)]
        ops += [("fork", p, 3, kids), ("release", p)]
        for c in kids:
            ops.append(("append", c, 6, call))
            call += 1
            free[c] = 10
        leaves += kids
    cycle, qcall = [1, 2, 3, 5, 16], 0
    for rnd in range(rounds):
        if rnd % 3 == 1:
            h, kids = leaves[0], [nm(), nm()]
            ops += [("fork", h, 2, kids), ("release", h)]
            leaves = kids + leaves[1:]
            for c in kids:
                free[c] = 16
        ns = []
        for i, h in enumerate(leaves):
            n = min(cycle[(rnd + i) % len(cycle)], free[h])
            ns.append(n)
            free[h] = free[h] - n or 16
        ops.append(("reserve_batch", list(leaves), call, ns))
        for layer in range(layers):
            ops.append(("decode_new", layer, list(leaves), call, ns, qcall))
            qcall += 1
        call += 1
    return recipes.Workload(name=name, dtype=dtype, layers=layers, q_heads=8, kv_heads=2, head_dim=head_dim,
                            num_blocks=1024, ops=ops, seed=seed)


@pytest.mark.parametrize("one_launch", [1, 0])
@pytest.mark.parametrize("dtype,layers,head_dim", [("bf16", 1, 128), ("bf16", 2, 64), ("f32", 2, 128), ("f32", 1, 64)])
def test_decode_with_several_new_tokens_written_in_the_call(dtype, layers, head_dim, one_launch):
    """tkv_attend_decode_new_tokens: each round every branch reserves 1 to 16
    tokens (a partly filled block, a block they fill, or a new node's block
    after a fork), and per layer the decode call writes them -- from the
    attention launch itself (one_launch = 1) or from a preparation launch.
    Every call matches the oracle; outputs and pool contents equal, bit for
    bit, those of the same rounds run as a batched append with K/V followed by
    tkv_attend_decode."""
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    import dataclasses
    wl = _multi_new_token_workload("multi_%s_%d_%d" % (dtype, layers, head_dim), dtype, layers, head_dim, 12, 82)
    assert_close(run_both(wl, options={tkv.TKV_OPT_FUSED_NEW_TOKEN: one_launch}), wl.dtype)
    plain_ops = []
    for op in wl.ops:
        if op[0] == "reserve_batch":
            plain_ops.append(("append_batch", op[1], op[3], op[2]))
        elif op[0] == "decode_new":
            plain_ops.append(("decode", op[1], op[2], op[-1]))
        else:
            plain_ops.append(op)
    plain = dataclasses.replace(wl, ops=plain_ops)
    outs, pools = {}, {}
    for key, w in (("fused", wl), ("plain", plain)):
        lib = LibReplay(w)
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_FUSED_NEW_TOKEN, one_launch)
        try:
            got = []
            for op in w.ops:
                if op[0] in ("decode", "decode_new"):
                    got.append(lib.attend(op).cpu())
                    if op[0] == "decode_new":
                        names = tkv.tkv_last_kernels(lib.c)
                        attn = [n for n in names if n.startswith(("attn_partial_kernel", "attn_rows_kernel"))]
                        prep = [n for n in names if n.startswith(("decode_prep_kernel", "plan_patch"))]
                        assert attn, names
                        if one_launch:
                            assert not prep and all("NewTokens" in n for n in attn), names
                        else:
                            assert prep and not any("NewTokens" in n for n in attn), names
                lib.apply(op)
            torch.cuda.synchronize()
            outs[key] = got
            views = {}
            for name in sorted(lib.h):
                L = tkv.tkv_seq_len(lib.c, lib.h[name])
                for layer in range(w.layers):
                    dt = torch.bfloat16 if dtype == "bf16" else torch.float32
                    ko = torch.empty((L, w.kv_heads, w.head_dim), dtype=dt, device="cuda")
                    vo = torch.empty_like(ko)
                    tkv.tkv_gather(lib.c, lib.h[name], layer, ko, vo, torch.cuda.current_stream())
                    views[(name, layer)] = (ko.cpu(), vo.cpu())
            torch.cuda.synchronize()
            pools[key] = views
        finally:
            lib.close()
    assert len(outs["fused"]) == 12 * layers
    for a, b in zip(outs["fused"], outs["plain"]):
        assert torch.equal(a, b)
    assert pools["fused"].keys() == pools["plain"].keys()
    for k in pools["fused"]:
        assert torch.equal(pools["fused"][k][0], pools["plain"][k][0])
        assert torch.equal(pools["fused"][k][1], pools["plain"][k][1])


def _draft_verify_workload(name, dtype, layers, head_dim, rounds, seed):
    """3 requests (prefixes of 37, 50 and 70 tokens); each round every request's
    head forks into 2 or 3 draft paths (alternating by request and round), each
    path reserves n drafts (n cycling over 1, 3, 8, 16, 5; a path's drafts open
    a block of its new node) and per layer one verify_new verifies them; then
    each request keeps its first path truncated to its head's length plus
    n // 2 + 1 drafts, releases the others and appends one bonus token (with
    K/V)."""
    ops, nxt, call, qcall = [], [0], 0, 0

    def nm():
        nxt[0] += 1
        return nxt[0] - 1
    heads, lens = [], []
    for L in (37, 50, 70):
        h = nm()
        ops += [("new", h), ("append", h, L, call)]
        call += 1
        heads.append(h)
        lens.append(L)
    cycle = [1, 3, 8, 16, 5]
    for rnd in range(rounds):
        paths, ns, kids_of = [], [], []
        for r, h in enumerate(heads):
            kids = [nm() for _ in range(2 + (rnd + r) % 2)]
            ops += [("fork", h, len(kids), kids), ("release", h)]
            kids_of.append(kids)
            for i, c in enumerate(kids):
                paths.append(c)
                ns.append(cycle[(rnd + r + i) % len(cycle)])
        ops.append(("reserve_batch", list(paths), call, list(ns)))
        for layer in range(layers):
            ops.append(("verify_new", layer, list(paths), list(ns), call, qcall))
            qcall += 1
        call += 1
        at = 0
        for r, kids in enumerate(kids_of):
            keep = ns[at] // 2 + 1
            ops.append(("truncate", kids[0], lens[r] + keep))
            lens[r] += keep + 1
            for c in kids[1:]:
                ops.append(("release", c))
            heads[r] = kids[0]
            at += len(kids)
        ops.append(("append_batch", list(heads), [1] * len(heads), call))
        call += 1
    return recipes.Workload(name=name, dtype=dtype, layers=layers, q_heads=8, kv_heads=2, head_dim=head_dim,
                            num_blocks=1024, ops=ops, seed=seed)


@pytest.mark.parametrize("one_launch", [1, 0])
@pytest.mark.parametrize("dtype,layers,head_dim", [("bf16", 1, 128), ("bf16", 2, 64), ("f32", 2, 128), ("f32", 1, 64)])
def test_verify_with_new_tokens_written_in_the_call(dtype, layers, head_dim, one_launch):
    """tkv_attend_verify_new_tokens: each round the draft paths reserve 1 to 16
    tokens and per layer the verify call writes their K/V -- from the attention
    launch itself (one_launch = 1) or from a preparation launch -- and verifies
    them; then accept or roll back by truncation and a bonus token.  Every
    call matches the oracle; outputs and pool contents equal, bit for bit,
    those of the same rounds run as a batched append with K/V followed by
    tkv_attend_verify."""
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    import dataclasses
    wl = _draft_verify_workload("drafts_%s_%d_%d" % (dtype, layers, head_dim), dtype, layers, head_dim, 8, 86)
    assert_close(run_both(wl, options={tkv.TKV_OPT_FUSED_NEW_TOKEN: one_launch}), wl.dtype)
    plain_ops = []
    for op in wl.ops:
        if op[0] == "reserve_batch":
            plain_ops.append(("append_batch", op[1], op[3], op[2]))
        elif op[0] == "verify_new":
            plain_ops.append(("verify", op[1], op[2], op[3], op[-1]))
        else:
            plain_ops.append(op)
    plain = dataclasses.replace(wl, ops=plain_ops)
    outs, pools = {}, {}
    for key, w in (("fused", wl), ("plain", plain)):
        lib = LibReplay(w)
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_FUSED_NEW_TOKEN, one_launch)
        try:
            got = []
            for op in w.ops:
                if op[0] in ("verify", "verify_new"):
                    got.append(lib.attend(op).cpu())
                    if op[0] == "verify_new":
                        names = tkv.tkv_last_kernels(lib.c)
                        attn = [n for n in names if n.startswith(("attn_partial_kernel", "attn_rows_kernel"))]
                        prep = [n for n in names if n.startswith(("decode_prep_kernel", "plan_patch"))]
                        assert attn, names
                        if one_launch:
                            assert not prep and all("NewTokens" in n for n in attn), names
                        else:
                            assert prep and not any("NewTokens" in n for n in attn), names
                lib.apply(op)
            torch.cuda.synchronize()
            outs[key] = got
            views = {}
            for name in sorted(lib.h):
                L = tkv.tkv_seq_len(lib.c, lib.h[name])
                for layer in range(w.layers):
                    ko = torch.empty((L, w.kv_heads, w.head_dim), dtype=torch.bfloat16 if w.dtype == "bf16"
                                     else torch.float32, device="cuda")
                    vo = torch.empty_like(ko)
                    tkv.tkv_gather(lib.c, lib.h[name], layer, ko, vo, torch.cuda.current_stream())
                    views[(name, layer)] = (ko.cpu(), vo.cpu())
            torch.cuda.synchronize()
            pools[key] = views
        finally:
            lib.close()
    assert len(outs["fused"]) == 8 * layers
    for a, b in zip(outs["fused"], outs["plain"]):
        assert torch.equal(a, b)
    assert pools["fused"].keys() == pools["plain"].keys()
    for k in pools["fused"]:
        assert torch.equal(pools["fused"][k][0], pools["plain"][k][0])
        assert torch.equal(pools["fused"][k][1], pools["plain"][k][1])


def test_decode_with_several_new_tokens_refusals():
    """tkv_attend_decode_new_tokens refuses, before any launch, a count outside
    1..16 and tokens that would reach into an earlier block (TKV_E_RANGE)."""
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    n = 1 * 64 * 2 * 16 * 64
    kp = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    c = tkv.tkv_create(1, 8, 2, 64, 64, tkv.TKV_BF16, kp, vp)
    try:
        st = torch.cuda.current_stream()
        root = tkv.tkv_seq_new(c)
        tkv.tkv_append(c, root, 22)  # slots 0..5 of its second block
        k = torch.zeros((20, 2, 64), dtype=torch.bfloat16, device="cuda")
        q = torch.zeros((1, 8, 64), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((1, 8, 64), dtype=torch.float32, device="cuda")
        for cnt in (0, 17, 7):
            with pytest.raises(tkv.TkvError) as e:
                tkv.tkv_attend_decode_new_tokens(c, 0, [root], [cnt], k, k, q, out, None, 0, st)
            assert e.value.code == tkv.TKV_E_RANGE, cnt
        tkv.tkv_attend_decode_new_tokens(c, 0, [root], [6], k, k, q, out, None, 0, st)
        torch.cuda.synchronize()
    finally:
        tkv.tkv_destroy(c)


def test_decode_with_new_token_refusals():
    """tkv_attend_decode_new_token refuses, before any launch: a handle given
    twice or a null K/V (TKV_E_INVAL), a handle whose last token is shared
    with other branches (TKV_E_SHARED: its tip was forked, or a fresh child
    has no token of its own) and an empty handle (TKV_E_EMPTY)."""
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    n = 1 * 64 * 2 * 16 * 128
    kp = torch.zeros(n, dtype=torch.bfloat16, device="cuda")
    vp = torch.zeros_like(kp)
    c = tkv.tkv_create(1, 8, 2, 128, 64, tkv.TKV_BF16, kp, vp)
    try:
        p = tkv.tkv_seq_new(c)
        tkv.tkv_append(c, p, 20)
        kids = tkv.tkv_fork(c, p, 2)
        tkv.tkv_append_batch(c, [kids[0]], [1])
        empty = tkv.tkv_seq_new(c)
        q = torch.zeros((2, 8, 128), dtype=torch.bfloat16, device="cuda")
        kn = torch.zeros((2, 2, 128), dtype=torch.bfloat16, device="cuda")
        out = torch.empty((2, 8, 128), dtype=torch.float32, device="cuda")
        st = torch.cuda.current_stream()
        for seqs, k, err in [([kids[0], kids[0]], kn, "TKV_E_INVAL"), ([kids[1]], kn, "TKV_E_SHARED"),
                             ([p], kn, "TKV_E_SHARED"), ([empty], kn, "TKV_E_EMPTY"), ([kids[0]], None, "TKV_E_INVAL")]:
            with pytest.raises(tkv.TkvError) as ei:
                tkv.tkv_attend_decode_new_token(c, 0, seqs, k, kn, q, out, None, 0, st)
            assert ei.value.code == getattr(tkv, err), (seqs, err)
        tkv.tkv_attend_decode_new_token(c, 0, [kids[0]], kn, kn, q, out, None, 0, st)
        torch.cuda.synchronize()
    finally:
        tkv.tkv_destroy(c)


@pytest.mark.parametrize("requests,one_launch", [(45, 0), (45, 1), (80, 1)])
def test_decode_with_new_token_more_than_128_handles(requests, one_launch):
    """135 branches in one fused decode call: its tokens are written by the
    attention launch (one_launch = 1, up to 192 tokens) or by two preparation
    launches (128 + 7), the first also carrying the plan's changed words; 240
    branches are more than one attention launch carries, so preparation
    launches write them even with one_launch = 1.  Every call matches the
    oracle."""
    from tree_structured_copy_amd import tkv
    wl = recipes.decode_loop_workload("fused_wide_%d" % requests, requests=requests, width=3, branch_tokens=14,
                                      rounds=4, fused=True, seed=83)
    assert len(wl.attend_ops()[0][2]) == 3 * requests
    assert_close(run_both(wl, options={tkv.TKV_OPT_FUSED_NEW_TOKEN: one_launch}), wl.dtype)


@pytest.mark.parametrize("concurrent", [0, 1])
def test_search_tree_decode_loop_with_cascade(concurrent):
    """A search tree (64 leaves, 256-row groups with the cascade: a one-tile
    class and a 16-tile class, run one after another or on side streams),
    then 6 rounds of one token appended to every leaf and a decode of all
    leaves: the plan is updated in place across both classes.  Every call
    matches the oracle."""
    import dataclasses
    from tree_structured_copy_amd import tkv
    base = recipes.mcts_workload("mcts_loop_cascade", q_heads=8, kv_heads=2, root_tokens=70, branching=4, depth=5,
                                 leaves=64, node_tokens=9, seed=47)
    dec = base.ops[-1]
    assert dec[0] == "decode"
    leaves = dec[2]
    ops = list(base.ops)
    for r in range(6):
        ops.append(("append_batch", list(leaves), [1] * len(leaves), 5000 + r))
        ops.append(("decode", 0, list(leaves), 100 + r))
    wl = dataclasses.replace(base, ops=ops, num_blocks=base.num_blocks + len(leaves))
    res = run_both(wl, options={tkv.TKV_OPT_MAX_ROWS: 256, tkv.TKV_OPT_CASCADE: 1,
                                tkv.TKV_OPT_CONCURRENT: concurrent})
    assert len(res) == 7
    assert_close(res, wl.dtype)
