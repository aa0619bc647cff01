#!/usr/bin/env python3
"""Benchmark: tree-attention decode over a forked, copy-on-write KV cache on one MI355X.

A step is one ``tkv_attend_decode`` call (plan lookup, split-K partial
attention kernel, merge kernel) over the Llama-3-8B-shaped fork workload: 32
requests, each a 4096-token prefix forked into 4 branches of 64 tokens, one
decode query per branch (128 queries x 32 heads, GQA 32/8, head_dim 128, bf16).
The tree is built first (fork + append, untimed); K/V are resident in HBM
before the timed region.  Consecutive steps rotate over ``--copies``
independent copies of the workload (disjoint pools) so that no step finds the
previous step's KV in L2 or the 256 MB Infinity Cache.

Printed: one JSON line.  ``value`` is unique-KV GB/s: distinct (block, KV head)
tiles the step must read, counted by valid token slots, K and V, divided by the
wall time per step.  Also reported: branch-queries/s, the speculative-verify
workload's verify tokens/s (64 requests x 3 draft paths x 8 drafts), the
partial-attention kernel's roofline against 8 TB/s measured with HIP events,
fork latency, and the CPU oracle timed on a sample of the same workload.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0

# HBM bytes per launch of the decode kernel on llama_fork, from two rocprofv3
# --pmc passes (FETCH_SIZE, then WRITE_SIZE) over `bench.py --counters`, each
# scaled by the factor that makes the same counter read a plain 1 GiB copy
# right.  Valid only for the kernel sources they were taken on (sha256 below);
# after any change to them the bench line reports traffic as null.
TRAFFIC_RECORD = {
    "sources_sha256": "eeb46a9f0dd7e965c016df17018afb22ccbfcf619efd690b5ae671cebe0c6f48",
    "fetch_kib_per_launch": 281858, "fetch_factor": 1.9999,   # 1 GiB read reads as 524309 KiB
    "write_kib_per_launch": 2048, "write_factor": 1.0,        # 1 GiB written reads as 1048576 KiB
    "hbm_bytes_per_launch": 577221744 + 2097152,
}


def _kernel_sources_sha():
    """sha256 of the decode kernel's sources with // comments and blank lines
    removed, so that an edit of the comments alone keeps the recorded traffic."""
    import hashlib
    import re
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_structured_copy_amd", "csrc")
    for f in ("attn.hip", "attn_common.h", "layout.h", "tkv_types.h"):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def _recorded_traffic():
    rec = TRAFFIC_RECORD
    if not rec or rec.get("sources_sha256") != _kernel_sources_sha():
        return None
    return rec["hbm_bytes_per_launch"]


class _Copy:
    """One independent instance of a workload on the GPU: its tree, and every
    attend call of one step (one per layer for multi-layer workloads) with its
    query, output and workspace buffers."""

    def __init__(self, wl, extra_blocks=0):
        import torch
        from tree_structured_copy_amd import tkv
        from tree_structured_copy_amd.replay import LibReplay
        from workloads import device as wdev
        self.wl = wl
        self.lib = LibReplay(wl, "cuda", extra_blocks=extra_blocks)
        i = self.lib.build()
        self.ops = []
        while i < len(wl.ops) and wl.ops[i][0] in ("decode", "verify"):
            self.ops.append(wl.ops[i])
            i += 1
        self.calls = []
        need = 0
        for op in self.ops:
            rows = self.lib.nrows(op)
            q = wdev.q_tensor(wl, op[-1], rows)
            out = torch.empty((rows, wl.q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
            nq = tkv.i32_array(op[3]) if op[0] == "verify" else None
            seqs = tkv.seq_array(self.lib.handles(op))
            need = max(need, tkv.tkv_workspace_size(self.lib.c, seqs, nq))
            self.calls.append((op[1], seqs, nq, q, out))
        self.ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
        self.need = need

    def step(self, stream):
        from tree_structured_copy_amd import tkv
        c = self.lib.c
        for layer, seqs, nq, q, out in self.calls:
            if nq is None:
                tkv.tkv_attend_decode(c, layer, seqs, q, out, self.ws, self.need, stream)
            else:
                tkv.tkv_attend_verify(c, layer, seqs, nq, q, out, self.ws, self.need, stream)

    def unique_bytes(self):
        from tree_structured_copy_amd import tkv
        wl = self.wl
        total = 0
        infos = []
        for layer, seqs, nq, q, out in self.calls:
            info = tkv.tkv_plan_info_get(self.lib.c, seqs, nq)
            infos.append(info)
            total += info["unique_tokens"] * wl.kv_heads * wl.head_dim * wl.elem_bytes * 2
        return total, infos[0]

    def queries(self):
        return sum(out.shape[0] for _, _, _, _, out in self.calls)

    def close(self):
        self.lib.close()


def _prepare(wl, copies):
    import torch
    items = [_Copy(wl) for _ in range(copies)]
    torch.cuda.synchronize()
    return items


def _time_wall(items, steps, warmup):
    """Wall time per step: K calls back to back, synchronised on both sides, no
    profiling events in the stream."""
    import torch
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(warmup):
        items[i % len(items)].step(stream)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        items[i % len(items)].step(stream)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    return (t1 - t0) / steps * 1e3


def _time_kernels(items, steps):
    """Average device time of the partial-attention and merge kernels per call,
    from HIP events the library records around them on the call's stream."""
    import torch
    from tree_structured_copy_amd import tkv
    stream = torch.cuda.current_stream().cuda_stream
    for it in items:
        tkv.tkv_profile_read(it.lib.c)
        tkv.tkv_profile_enable(it.lib.c, True)
    for i in range(steps):
        items[i % len(items)].step(stream)
    torch.cuda.synchronize()
    part = merge = 0.0
    calls = 0
    for it in items:
        p, m, n = tkv.tkv_profile_read(it.lib.c)
        tkv.tkv_profile_enable(it.lib.c, False)
        part += p
        merge += m
        calls += n
    return part / max(1, calls), merge / max(1, calls)


def _time_rebuild(items, steps):
    """Wall time per step when every call rebuilds and uploads its plan (plan
    cache off): the cost a caller pays when the tree changed since the last call."""
    import torch
    from tree_structured_copy_amd import tkv
    for it in items:
        tkv.tkv_set_option(it.lib.c, tkv.TKV_OPT_PLAN_CACHE, 0)
    ms = _time_wall(items, steps, 2)
    for it in items:
        tkv.tkv_set_option(it.lib.c, tkv.TKV_OPT_PLAN_CACHE, 1)
    torch.cuda.synchronize()
    return ms


def _fork_latency_ns():
    """Median wall time of one tkv_fork(n=1) call through ctypes, for a prefix of
    16 vs 65536 tokens (host-only cache).  ctypes adds its own ~1 us."""
    from tree_structured_copy_amd import tkv
    res = {}
    for prefix in (16, 65536):
        c = tkv.tkv_create(1, 32, 8, 128, prefix // 16 + 8, tkv.TKV_BF16)
        s = tkv.tkv_seq_new(c)
        tkv.tkv_append(c, s, prefix)
        out = (tkv._U64 * 1)()
        ts = []
        for _ in range(20000):
            t0 = time.perf_counter_ns()
            tkv._lib.tkv_fork(c, s, 1, out)
            ts.append(time.perf_counter_ns() - t0)
            tkv._lib.tkv_release(c, out[0])
        ts.sort()
        res[str(prefix)] = ts[len(ts) // 2]
        tkv.tkv_destroy(c)
    return res


def _fork_sweep_ns():
    """Fork latency from the host-only C++ benchmark built beside the library
    (tree_structured_copy_amd/fork_bench): median ns per tkv_fork(n) over
    prefix 16..65536 tokens and path depth 1..500 nodes, no ctypes in between."""
    import subprocess
    exe = os.path.join(ROOT, "tree_structured_copy_amd", "fork_bench")
    if not os.path.exists(exe):
        return None
    out = subprocess.run([exe, "400"], capture_output=True, text=True, timeout=120, check=True).stdout
    grid = json.loads(out)
    summary = {}
    for n in (1, 4, 16):
        vals = [v for k, v in grid.items() if k.endswith(":%d" % n)]
        summary["n=%d" % n] = {"min": min(vals), "max": max(vals), "median": sorted(vals)[len(vals) // 2]}
    return {"summary": summary, "grid_prefix_depth_n": grid}


def _cpu_baseline(requests: int, reps: int):
    """The float64 oracle on the first ``requests`` requests of the fork workload:
    materialise each branch's history and run textbook attention for all heads."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:
        threads = 1
    from oracle import attention
    from oracle.cache import ArraySource, MaterializedCache
    from workloads import gen, recipes
    import workloads
    full = recipes.llama_fork()
    wl = recipes.fork_workload("llama_fork_sample", dtype="bf16", layers=1, q_heads=32, kv_heads=8, head_dim=128,
                               requests=requests, prefix=4096, width=4, branch_tokens=64, seed=full.seed)
    # inputs generated up front (not timed)
    arrays = {}
    for op in wl.ops:
        if op[0] == "append":
            _, h, ntok, call = op
            arrays[call] = (workloads.kv_values(wl, call, ntok, gen.KIND_K),
                            workloads.kv_values(wl, call, ntok, gen.KIND_V))
    dec = wl.attend_ops()[0]
    Q = workloads.q_values(wl, dec[-1], len(dec[2])).astype(np.float64)
    times = []
    for _ in range(reps):
        t0 = time.perf_counter()
        mc = MaterializedCache()
        names = {}
        for op in wl.ops:
            if op[0] == "new":
                names[op[1]] = mc.seq_new()
            elif op[0] == "append":
                mc.append(names[op[1]], ArraySource(*arrays[op[3]]))
            elif op[0] == "fork":
                for n, c in zip(op[3], mc.fork(names[op[1]], op[2])):
                    names[n] = c
            elif op[0] == "release":
                mc.release(names.pop(op[1]))
        for r, h in enumerate(dec[2]):
            kv = [mc.kv(names[h], 0, g) for g in range(wl.kv_heads)]
            for hq in range(wl.q_heads):
                K, V = kv[attention.kv_head_of(hq, wl.q_heads, wl.kv_heads)]
                attention.attend_one(K, V, Q[r, hq])
        times.append(time.perf_counter() - t0)
    t = sorted(times)[len(times) // 2]
    unique = requests * (4096 + 4 * 64) * wl.kv_heads * wl.head_dim * 2 * 2
    return {"value": unique / t / 1e9, "unit": "GB/s", "cores": int(threads), "kind": "oracle",
            "sample": "%d of 32 requests of the fork workload (%d decode queries x 32 heads), median of %d "
                      "runs of %.2f s" % (requests, 4 * requests, reps, t),
            "branch_queries_per_s": 4 * requests / t}


def _native_loops():
    """The speculative loop and the tree-search loop at full size, timed by the
    native replayer (tree_structured_copy_amd/replay_bench) from their recipes:
    * spec_loop: the verify workload's 64 requests (2048-token prefixes, 3 draft
      paths of 8 tokens) through 8 rounds of fork, draft, verify, accept or
      roll back and a bonus token;
    * search_loop: 500 tree-search simulations, branching 4, depth 12, a
      2048-token root and 16 tokens per node (GQA 32/8, d = 128, bf16)."""
    import subprocess
    import tempfile
    from workloads import recipes
    exe = os.path.join(ROOT, "tree_structured_copy_amd", "replay_bench")
    res = {}
    for key, wl in (("spec_loop", recipes.spec_loop_workload("spec_loop", rounds=8)),
                    ("search_loop", recipes.mcts_loop_workload("search_loop"))):
        with tempfile.NamedTemporaryFile("w", suffix=".ops", delete=False) as f:
            f.write(recipes.ops_text(wl))
            path = f.name
        try:
            r = subprocess.run([exe, path], capture_output=True, text=True, timeout=300)
        finally:
            os.unlink(path)
        if r.returncode != 0:
            raise RuntimeError("replay_bench failed on %s: %s" % (key, r.stderr[-2000:]))
        d = json.loads(r.stdout)
        sec = d["wall_ms"] / 1e3
        if key == "spec_loop":
            d["rounds"] = 8
            d["verify_tokens_per_s"] = d["verify_tokens"] / sec
            d["ms_per_round"] = d["wall_ms"] / 8
        else:
            d["simulations"] = 500
            d["ms_per_simulation"] = d["wall_ms"] / 500
            d["branch_queries_per_s"] = d["decode_queries"] / sec
            d["full_copy_over_cow"] = d["full_copy_bytes"] / max(1, d["cow_peak_bytes"])
        d["attend_share_of_wall"] = d["attend_kernel_ms"] / max(1e-9, d["wall_ms"])
        res[key] = d
    return res


def _time_generation_loop(copies, windows, patch, fused=False):
    """A decode loop on the fork workload.  A step appends one token to each of
    the 128 branches (one tkv_append_batch) and runs the decode call; copies
    rotate step by step.  Windows of 16 steps per copy are timed (wall clock,
    synchronised on both sides): in each, the first step opens a block in every
    branch (its plan is rebuilt) and the other 15 fit in it (its plan is
    updated in place, or with patch = 0 rebuilt).  Between windows, untimed,
    the branches are truncated back to their 64 tokens.  With fused, a step
    reserves the token (tkv_append_batch without K/V) and writes it in the
    decode call (tkv_attend_decode_new_token): one launch fewer.  Returns ms
    per step."""
    import torch
    from tree_structured_copy_amd import tkv
    from workloads import device as wdev, gen, recipes
    wl = recipes.llama_fork()
    leaves = len(wl.attend_ops()[0][2])
    items = [_Copy(wl, extra_blocks=leaves) for _ in range(copies)]
    stream = torch.cuda.current_stream().cuda_stream
    k = wdev.kv_tensor(wl, 1 << 20, leaves, gen.KIND_K)
    v = wdev.kv_tensor(wl, 1 << 20, leaves, gen.KIND_V)
    ones = tkv.i32_array([1] * leaves)
    handles = [list(it.calls[0][1]) for it in items]
    base_len = [[tkv.tkv_seq_len(it.lib.c, h) for h in hs] for it, hs in zip(items, handles)]
    for it in items:
        tkv.tkv_set_option(it.lib.c, tkv.TKV_OPT_PLAN_PATCH, patch)
    torch.cuda.synchronize()
    total = 0.0
    counted = 0
    for w in range(windows + 1):   # the first window warms up
        t0 = time.perf_counter()
        for i in range(16 * copies):
            it = items[i % copies]
            if fused:
                layer, seqs, _, q, out = it.calls[0]
                tkv.tkv_append_batch(it.lib.c, seqs, ones)
                tkv.tkv_attend_decode_new_token(it.lib.c, layer, seqs, k, v, q, out, it.ws, it.need, stream)
            else:
                tkv.tkv_append_batch(it.lib.c, it.calls[0][1], ones, k, v, stream)
                it.step(stream)
        torch.cuda.synchronize()
        if w > 0:
            total += time.perf_counter() - t0
            counted += 16 * copies
        for it, hs, lens in zip(items, handles, base_len):
            for h, L in zip(hs, lens):
                tkv.tkv_truncate(it.lib.c, h, L)
    counters = tkv.tkv_get_counters(items[0].lib.c)
    for it in items:
        it.close()
    del items
    torch.cuda.empty_cache()
    return total / counted * 1e3, counters


def measure(name, copies, steps, warmup, rebuild=False):
    """Wall time per step, kernel times and derived rates for one workload."""
    import torch
    from workloads import recipes
    wl = recipes.STANDARD[name]()
    items = _prepare(wl, copies)
    ubytes, info = items[0].unique_bytes()
    queries = items[0].queries()
    ms = _time_wall(items, steps, warmup)
    part_ms, merge_ms = _time_kernels(items, steps)
    ncalls = len(items[0].calls)
    res = {"workload": name, "ms_per_step": ms, "attend_calls_per_step": ncalls,
           "unique_kv_bytes": ubytes, "unique_kv_GBps": ubytes / (ms / 1e3) / 1e9,
           "queries_per_step": queries, "queries_per_s": queries / (ms / 1e3),
           "partial_kernel_ms_per_call": part_ms, "merge_kernel_ms_per_call": merge_ms,
           "partial_kernel_GBps": (ubytes / ncalls) / (part_ms / 1e3) / 1e9 if part_ms > 0 else None,
           "plan": info, "copies_rotated": copies}
    if rebuild:
        res["ms_per_step_plan_rebuild"] = _time_rebuild(items, max(5, steps // 5))
    for it in items:
        it.close()
    del items
    torch.cuda.empty_cache()
    return res


def _counters_run(copies, workload="llama_fork"):
    """What the traffic figures are taken on: 3 launches of a plain streaming
    kernel over a 1 GiB buffer (dst = 2 * src: 1 GiB read + 1 GiB written per
    launch), then 8 steps of the workload (by default the fork workload's decode
    call), rotating over `copies` independent copies."""
    import torch
    from workloads import recipes
    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2, out=dst)
    torch.cuda.synchronize()
    items = _prepare(recipes.STANDARD[workload](), copies)
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(8):
        items[i % len(items)].step(stream)
    torch.cuda.synchronize()
    ubytes, _ = items[0].unique_bytes()
    print(json.dumps({"counters_run": True, "workload": workload, "copy_bytes": n, "copy_launches": 3,
                      "steps": 8, "unique_kv_bytes_per_call": ubytes, "sources_sha256": _kernel_sources_sha()}),
          flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    # the clock ramps up from idle over the first tens of milliseconds of load:
    # 300 warm-up steps (about 30 ms at these shapes) reach its steady state
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--no-verify", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--all", action="store_true", help="also measure the 32-layer workload")
    ap.add_argument("--cpu-requests", type=int, default=32)
    ap.add_argument("--cpu-reps", type=int, default=7)
    ap.add_argument("--counters", action="store_true",
                    help="a short run for rocprofv3 --pmc passes: a plain 1 GiB streaming kernel (the "
                         "counters' calibration), then 8 steps of --counters-workload")
    ap.add_argument("--counters-workload", default="llama_fork",
                    help="workload of the --counters run (llama_fork, spec_verify, mcts_tree, ...)")
    ap.add_argument("--only", default=None,
                    help="measure just this workload (mcts_tree, spec_verify, full_depth, llama_fork, or "
                         "generation_loop: the decode loop with batched appends) and print "
                         "its figures as one JSON line: a short run for a kernel trace of that workload alone")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the fork workload's requests are independent trees, so "
              "more GPUs would shard requests with no communication; --gpus %d is not supported" % args.gpus,
              file=sys.stderr)
        sys.exit(2)

    import torch
    torch.cuda.init()

    if args.counters:
        _counters_run(args.copies, args.counters_workload)
        return
    if args.only == "generation_loop":
        ms, counters = _time_generation_loop(args.copies, 8, 1)
        fused_ms, _ = _time_generation_loop(args.copies, 8, 1, fused=True)
        print(json.dumps({"only": "generation_loop", "ms_per_step": ms, "ms_per_step_fused": fused_ms,
                          "plans_built_patched_one_copy": [counters["plans_built"], counters["plans_patched"]]}),
              flush=True)
        return
    if args.only:
        copies = 1 if args.only == "full_depth" else args.copies
        steps, warmup = (max(3, args.steps // 10), 1) if args.only == "full_depth" else (args.steps, args.warmup)
        res = measure(args.only, copies, steps, warmup)
        print(json.dumps({"only": args.only, "steps": steps, "warmup": warmup, **res}), flush=True)
        return

    main_res = measure("llama_fork", args.copies, args.steps, args.warmup, rebuild=True)
    loop_ms, loop_counters = _time_generation_loop(args.copies, 8, 1)
    loop_rebuild_ms, _ = _time_generation_loop(args.copies, 8, 0)
    loop_fused_ms, _ = _time_generation_loop(args.copies, 8, 1, fused=True)
    generation_loop = {
        "steps_timed": 8 * 16 * args.copies,
        "ms_per_step": loop_ms,
        "ms_per_step_plans_rebuilt": loop_rebuild_ms,
        "ms_per_step_token_written_in_decode_call": loop_fused_ms,
        "branch_tokens_per_s": 128 / (loop_ms / 1e3),
        "plans_built_patched_one_copy": [loop_counters["plans_built"], loop_counters["plans_patched"]],
    }
    ms = main_res["ms_per_step"]
    ubytes = main_res["unique_kv_bytes"]
    value = main_res["unique_kv_GBps"]
    achieved = main_res["partial_kernel_GBps"]

    verify = None
    if not args.no_verify:
        v = measure("spec_verify", args.copies, args.steps, args.warmup)
        v["verify_tokens_per_s"] = v["queries_per_s"]
        verify = v
    # the search tree is part of every run; the 32-layer workload (103 GB of
    # pools to build) only with --all
    others = {"mcts_tree": measure("mcts_tree", args.copies, args.steps, args.warmup)}
    others["mcts_tree"]["branch_queries_per_s"] = others["mcts_tree"]["queries_per_s"]
    if args.all:
        others["full_depth"] = measure("full_depth", 1, max(3, args.steps // 10), 1)
        others["full_depth"]["branch_query_steps_per_s"] = 1024 / (others["full_depth"]["ms_per_step"] / 1e3)

    cpu = None
    if not args.no_cpu:
        cpu = _cpu_baseline(args.cpu_requests, args.cpu_reps)

    line = {
        "metric": "tree-attn decode unique-KV GB/s (% HBM peak) + branch-queries/s; verify tokens/s",
        "value": value,
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "llama_fork", "requests": 32, "prefix_tokens": 4096, "fork_width": 4,
                   "branch_tokens": 64, "q_heads": 32, "kv_heads": 8, "head_dim": 128, "block_size": 16,
                   "decode_queries": main_res["queries_per_step"], "copies_rotated": args.copies},
        "hbm_peak_frac": value / HBM_PEAK_GBS,
        "branch_queries_per_s": main_res["queries_per_s"],
        "ms_per_step_plan_rebuild": main_res["ms_per_step_plan_rebuild"],
        "generation_loop": generation_loop,
        "native_loops": _native_loops(),
        "unique_kv_bytes": ubytes,
        "plan": main_res["plan"],
        "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": (achieved / HBM_PEAK_GBS) if achieved else None, "traffic": _recorded_traffic(),
                     "kernel": "attn_partial_kernel<BF16,128,1,2,false>",
                     "kernel_ms": main_res["partial_kernel_ms_per_call"],
                     "merge_kernel_ms": main_res["merge_kernel_ms_per_call"]},
        "verify": verify,
        "other_workloads": others or None,
        "fork_latency_ns": _fork_sweep_ns(),
        "fork_latency_ns_ctypes": _fork_latency_ns(),
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
