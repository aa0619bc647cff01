#!/usr/bin/env python3
"""Benchmark: tree-attention decode over a forked, copy-on-write KV cache on one MI355X.

The headline step is one decode step of the 32-layer workload: 64 requests,
each an 8192-token prefix forked into 16 branches of 256 tokens, one decode
query per branch in every layer (32 layer calls of 1024 queries x 32 heads,
GQA 32/8, head_dim 128, bf16; 103 GB of K/V resident in HBM).  The tree is
built first (fork + append, untimed); K/V are resident before the timed
region, and the 103 GB dwarf every cache, so no step finds the previous one's
KV cached.

Printed: one JSON line.  ``value`` is unique-KV GB/s: distinct (layer, block,
KV head) tiles the step must read, counted by valid token slots, K and V,
divided by the wall time per step.  ``roofline`` gives the dominant kernel's
rate from HIP events against 8 TB/s, and ``cpu_baseline`` the float64 oracle
on a sample of the same workload.  The other single-layer workloads (the
fork workload, the speculative-verify batch and the search tree) are reported
under ``workloads``, each with its own roofline and CPU baseline, beside the
decode, speculative and search loops and the fork latency.
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

# HBM bytes per launch of each workload's dominant attention kernel, from two
# rocprofv3 --pmc passes (FETCH_SIZE, then WRITE_SIZE) over `bench.py --counters
# --counters-workload <name>`, each scaled by the factor that makes the same
# counter read a plain 1 GiB copy right.  Valid only for the kernel sources
# they were taken on (sha256 over the files listed); after any change to them
# the line reports traffic as null.
KERNEL_SOURCES = {
    "attn_partial_kernel": ("attn.hip", "attn_common.h", "layout.h", "tkv_types.h"),
    "attn_rows_kernel": ("attn_rows.hip", "attn_common.h", "layout.h", "tkv_types.h"),
}
TRAFFIC_RECORDS = {
    "full_depth": {"kernel": "attn_rows_kernel<BF16, 128, 1, 4, 1, 2, false, 2, false>",
                   "sources_sha256": "f18ed1514ed7580fdce3c054154e9d295ea62dd48a184a0a25801d821996d62c",
                   "fetch_kib_per_launch": 1581696.0625, "fetch_factor": 1.99992, "write_kib_per_launch": 16384.0,
                   "write_factor": 1.0, "hbm_bytes_per_launch": 3255961179},
    "llama_fork": {"kernel": "attn_partial_kernel<BF16, 128, 1, 2, false>",
                   "sources_sha256": "18ada46400e7718bc79ffb2a2e66d895f5cc0184f81e2f84198b43b34822585e",
                   "fetch_kib_per_launch": 281803.8125, "fetch_factor": 1.99992, "write_kib_per_launch": 2048.0,
                   "write_factor": 1.0, "hbm_bytes_per_launch": 579208275},
    "spec_verify": {"kernel": "attn_rows_kernel<BF16, 128, 1, 6, 2, 2, false, 3, true>",
                    "sources_sha256": "f18ed1514ed7580fdce3c054154e9d295ea62dd48a184a0a25801d821996d62c",
                    "fetch_kib_per_launch": 275007.46875, "fetch_factor": 1.99992, "write_kib_per_launch": 24576.0,
                    "write_factor": 1.0, "hbm_bytes_per_launch": 588358591},
    # the attention kernel alone; its merge kernel adds 20.2 MB fetched and 4.2 MB written
    "mcts_tree": {"kernel": "attn_rows_kernel<BF16, 128, 1, 8, 1, 2, false, 4, false>",
                  "sources_sha256": "f18ed1514ed7580fdce3c054154e9d295ea62dd48a184a0a25801d821996d62c",
                  "fetch_kib_per_launch": 86828.59375, "fetch_factor": 1.99992, "write_kib_per_launch": 18703.75,
                  "write_factor": 1.0, "hbm_bytes_per_launch": 196970487},
}


def _kernel_sources_sha(kernel):
    """sha256 of a kernel's sources with // comments and blank lines removed, so
    that an edit of the comments alone keeps the recorded traffic."""
    import hashlib
    import re
    base = kernel.split("<")[0]
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "tree_structured_copy_amd", "csrc")
    for f in KERNEL_SOURCES.get(base, ()):
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            for line in fh:
                code = re.sub(r"//.*", "", line).rstrip()
                if code:
                    h.update(code.encode() + b"\n")
    return h.hexdigest()


def _recorded_traffic(workload, kernel):
    rec = TRAFFIC_RECORDS.get(workload)
    if not rec or rec.get("kernel") != kernel or rec.get("sources_sha256") != _kernel_sources_sha(kernel):
        return None
    return rec["hbm_bytes_per_launch"]


def _host_info():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"nproc": os.cpu_count(), "affinity_cpus": len(os.sched_getaffinity(0)), "cpu_model": model}


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


def _cpu_threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))


def _cpu_oracle(wl):
    """The float64 oracle on workload ``wl`` (a benchmarked workload or a sample of
    one): every append call's K/V generated up front (not timed), then, timed, the oracle's replay -- each branch's history
    materialised (a fork copies it) and textbook attention for every query row
    and head of every decode/verify call -- on T host threads with one BLAS
    thread each (cores = T)."""
    from threadpoolctl import threadpool_limits
    from oracle.replay import OracleReplay, PreloadedArrays
    threads = _cpu_threads()
    arrays = PreloadedArrays(wl, threads)
    rows = 0
    with threadpool_limits(1):
        t0 = time.perf_counter()
        orc = OracleReplay(wl, with_alloc=False, threads=threads, arrays=arrays)
        for op in wl.ops:
            if op[0] in ("decode", "verify"):
                orc.attend(op)
                rows += sum(op[3]) if op[0] == "verify" else len(op[2])
            orc.apply(op)
        t = time.perf_counter() - t0
    del arrays
    return t, rows


def _unique_kv_bytes_host(wl):
    """Unique K/V bytes every attend call of wl reads, from a host-only replay of
    its recipe through the library's planner (valid token slots of the distinct
    blocks of each call, K and V, all KV heads)."""
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    lib = LibReplay(wl, None)
    total = 0
    try:
        for op in wl.ops:
            if op[0] in ("decode", "verify"):
                nq = op[3] if op[0] == "verify" else None
                info = tkv.tkv_plan_info_get(lib.c, lib.handles(op), nq)
                total += info["unique_tokens"] * wl.kv_heads * wl.head_dim * wl.elem_bytes * 2
            lib.apply(op)
    finally:
        lib.close()
    return total


def _cpu_baseline(name):
    """The oracle timed on a bounded sample of workload ``name`` (all of it where
    that takes seconds): rates in the GPU line's units."""
    from workloads import recipes
    full = recipes.STANDARD[name]()
    if name == "full_depth":
        wl = recipes.fork_workload("full_depth_sample", dtype="bf16", layers=32, q_heads=32, kv_heads=8,
                                   head_dim=128, requests=4, prefix=8192, width=16, branch_tokens=256,
                                   seed=full.seed)
        scale = 16
        sample = ("4 of the 64 requests (64 branches x 32 layers: 2048 decode queries x 32 heads); the step's "
                  "time extrapolated as 16 x the sample's")
    else:
        wl, scale = full, 1
        sample = "the whole workload"
    t, rows = _cpu_oracle(wl)
    ubytes = _unique_kv_bytes_host(wl)
    res = {"value": ubytes / t / 1e9, "unit": "GB/s", "cores": _cpu_threads(), "kind": "oracle",
           "sample": sample + ", %.2f s" % t, "seconds": t, "queries_per_s": rows / t,
           "extrapolated_ms_per_step": t * scale * 1e3 if scale > 1 else None}
    return res


def _native_loops():
    """The speculative loop and the tree-search loop at full size, timed by the
    native replayer (tree_structured_copy_amd/replay_bench) from their recipes:
    * spec_loop: the verify workload's 64 requests (2048-token prefixes, 3 draft
      paths of 8 tokens) through 8 rounds of fork, draft, verify, accept or
      roll back and a bonus token;
    * spec_loop_one_launch: the same, each round's drafts reserved and written
      by the verify call (tkv_attend_verify_new_tokens);
    * search_loop: 500 tree-search simulations, branching 4, depth 12, a
      2048-token root and 16 tokens per node (GQA 32/8, d = 128, bf16);
    * search_loop_one_launch: the same, each expansion's new nodes reserved and
      written by its decode call (tkv_attend_decode_new_tokens)."""
    import subprocess
    import tempfile
    from workloads import recipes
    exe = os.path.join(ROOT, "tree_structured_copy_amd", "replay_bench")
    res = {}
    for key, wl in (("spec_loop", recipes.spec_loop_workload("spec_loop", rounds=8)),
                    ("spec_loop_one_launch", recipes.spec_loop_workload("spec_loop", rounds=8, one_launch=True)),
                    ("search_loop", recipes.mcts_loop_workload("search_loop")),
                    ("search_loop_one_launch", recipes.mcts_loop_workload("search_loop", one_launch=True))):
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
        if key.startswith("spec_loop"):
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


def _split_kernels(names):
    """(attention kernels, merge kernel or None) from an attention call's launch list."""
    attn = [n for n in names if n.startswith(("attn_partial_kernel", "attn_rows_kernel"))]
    merge = [n for n in names if n.startswith("attn_merge_kernel")]
    return attn, (merge[0] if merge else None)


def measure(name, copies, steps, warmup, rebuild=False):
    """Wall time per step, kernel times and derived rates for one workload."""
    import torch
    from tree_structured_copy_amd import tkv
    from workloads import recipes
    wl = recipes.STANDARD[name]()
    items = _prepare(wl, copies)
    ubytes, info = items[0].unique_bytes()
    queries = items[0].queries()
    ms = _time_wall(items, steps, warmup)
    attn, merge = _split_kernels(tkv.tkv_last_kernels(items[0].lib.c))
    part_ms, merge_ms = _time_kernels(items, steps)
    ncalls = len(items[0].calls)
    achieved = (ubytes / ncalls) / (part_ms / 1e3) / 1e9 if part_ms > 0 else None
    kernel = attn[0] if len(attn) == 1 else (";".join(attn) if attn else None)
    res = {"workload": name, "ms_per_step": ms, "attend_calls_per_step": ncalls,
           "unique_kv_bytes": ubytes, "unique_kv_GBps": ubytes / (ms / 1e3) / 1e9,
           "hbm_peak_frac": ubytes / (ms / 1e3) / 1e9 / HBM_PEAK_GBS,
           "queries_per_step": queries, "queries_per_s": queries / (ms / 1e3),
           "roofline": {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                        "frac": achieved / HBM_PEAK_GBS if achieved else None,
                        "traffic": _recorded_traffic(name, kernel) if kernel else None,
                        "kernel": kernel, "kernel_ms": part_ms, "launches_per_call": len(attn),
                        "merge_kernel": merge, "merge_kernel_ms": merge_ms if merge else None,
                        "timing": "HIP events around the attention launches of each call, on its stream"},
           "plan": info, "copies_rotated": copies, "steps": steps, "warmup": warmup}
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
    launch), then a few steps of the workload (8 single-layer calls, or 2 steps
    of the 32-layer workload), rotating over `copies` independent copies."""
    import torch
    from tree_structured_copy_amd import tkv
    from workloads import recipes
    n = 1 << 30
    src = torch.ones(n // 2, dtype=torch.bfloat16, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        torch.mul(src, 2, out=dst)
    torch.cuda.synchronize()
    del src, dst
    wl = recipes.STANDARD[workload]()
    copies = 1 if wl.layers > 1 else copies
    steps = 2 if wl.layers > 1 else 8
    items = _prepare(wl, copies)
    stream = torch.cuda.current_stream().cuda_stream
    for i in range(steps):
        items[i % len(items)].step(stream)
    torch.cuda.synchronize()
    ubytes, _ = items[0].unique_bytes()
    attn, merge = _split_kernels(tkv.tkv_last_kernels(items[0].lib.c))
    print(json.dumps({"counters_run": True, "workload": workload, "copy_bytes": n, "copy_launches": 3,
                      "steps": steps, "attend_calls": steps * len(items[0].calls),
                      "unique_kv_bytes_per_call": ubytes // len(items[0].calls), "kernels": attn,
                      "merge_kernel": merge,
                      "sources_sha256": {k: _kernel_sources_sha(k) for k in attn}}), flush=True)


SUBS = {
    "llama_fork": ("branch_queries_per_s",
                   {"requests": 32, "prefix_tokens": 4096, "fork_width": 4, "branch_tokens": 64, "layers": 1,
                    "decode_queries": 128}),
    "spec_verify": ("verify_tokens_per_s",
                    {"requests": 64, "prefix_tokens": 2048, "draft_paths": 3, "drafts_per_path": 8, "layers": 1,
                     "verify_queries": 1536}),
    "mcts_tree": ("branch_queries_per_s",
                  {"root_tokens": 2048, "branching": 4, "depth": 12, "node_tokens": 16, "leaves": 256,
                   "layers": 1, "decode_queries": 256}),
}
SHAPE = {"q_heads": 32, "kv_heads": 8, "head_dim": 128, "block_size": 16, "dtype": "bf16"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20, help="timed steps of the 32-layer workload")
    ap.add_argument("--warmup", type=int, default=5, help="untimed steps of the 32-layer workload before them")
    # the clock ramps up from idle over the first tens of milliseconds of load:
    # 300 warm-up calls (about 30 ms at these shapes) reach its steady state
    ap.add_argument("--sub-steps", type=int, default=200, help="timed calls of each single-layer workload")
    ap.add_argument("--sub-warmup", type=int, default=300, help="untimed calls of each single-layer workload")
    ap.add_argument("--copies", type=int, default=4, help="copies of each single-layer workload, rotated")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-loops", action="store_true")
    ap.add_argument("--counters", action="store_true",
                    help="a short run for rocprofv3 --pmc passes: a plain 1 GiB streaming kernel (the "
                         "counters' calibration), then a few steps of --counters-workload")
    ap.add_argument("--counters-workload", default="full_depth",
                    help="workload of the --counters run (full_depth, llama_fork, spec_verify, mcts_tree)")
    ap.add_argument("--only", default=None,
                    help="measure just this workload (full_depth, llama_fork, spec_verify, mcts_tree, or "
                         "generation_loop: the decode loop with batched appends) and print "
                         "its figures as one JSON line: a short run for a kernel trace of that workload alone")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the 32-layer workload's requests are independent trees, so "
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
        if args.only == "full_depth":
            res = measure("full_depth", 1, args.steps, args.warmup)
        else:
            res = measure(args.only, args.copies, args.sub_steps, args.sub_warmup)
        print(json.dumps({"only": args.only, **res}), flush=True)
        return

    # the headline: one decode step (32 layer calls) of the 32-layer workload
    head = measure("full_depth", 1, args.steps, args.warmup)
    print("[bench] full_depth: %.3f ms per step, %.0f GB/s" % (head["ms_per_step"], head["unique_kv_GBps"]),
          file=sys.stderr, flush=True)
    subs = {}
    for name, (rate_key, cfg) in SUBS.items():
        r = measure(name, args.copies, args.sub_steps, args.sub_warmup, rebuild=name == "llama_fork")
        r[rate_key] = r["queries_per_s"]
        r["config"] = dict(cfg, **SHAPE, copies_rotated=args.copies)
        subs[name] = r
        print("[bench] %s: %.1f us per call, %.0f GB/s" % (name, r["ms_per_step"] * 1e3, r["unique_kv_GBps"]),
              file=sys.stderr, flush=True)
    generation_loop = native = None
    if not args.no_loops:
        loop_ms, loop_counters = _time_generation_loop(args.copies, 8, 1)
        loop_rebuild_ms, _ = _time_generation_loop(args.copies, 8, 0)
        loop_fused_ms, fused_counters = _time_generation_loop(args.copies, 8, 1, fused=True)
        generation_loop = {
            "workload": "llama_fork decode loop: one token per branch per step",
            "steps_timed": 8 * 16 * args.copies,
            "ms_per_step": loop_ms,
            "ms_per_step_plans_rebuilt": loop_rebuild_ms,
            "ms_per_step_token_written_in_decode_call": loop_fused_ms,
            "branch_tokens_per_s": 128 / (loop_ms / 1e3),
            "plans_built_patched_one_copy": [loop_counters["plans_built"], loop_counters["plans_patched"]],
            "fused_plans_built_patched_one_copy": [fused_counters["plans_built"], fused_counters["plans_patched"]],
        }
        native = _native_loops()
        print("[bench] loops done", file=sys.stderr, flush=True)

    cpu = None
    if not args.no_cpu:
        for name in SUBS:
            subs[name]["cpu_baseline"] = _cpu_baseline(name)
        cpu = _cpu_baseline("full_depth")
        print("[bench] cpu baselines done", file=sys.stderr, flush=True)

    ms = head["ms_per_step"]
    line = {
        "metric": "tree-attn decode unique-KV GB/s (% HBM peak) + branch-queries/s; verify tokens/s",
        "value": head["unique_kv_GBps"],
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
        "config": dict({"workload": "full_depth", "layers": 32, "requests": 64, "prefix_tokens": 8192,
                        "fork_width": 16, "branch_tokens": 256, "decode_queries_per_layer": 1024,
                        "attend_calls_per_step": head["attend_calls_per_step"], "copies": 1}, **SHAPE),
        "hbm_peak_frac": head["hbm_peak_frac"],
        "branch_queries_per_s": head["queries_per_s"],
        "branch_query_steps_per_s": 1024 / (ms / 1e3),
        "unique_kv_bytes": head["unique_kv_bytes"],
        "plan": head["plan"],
        "roofline": head["roofline"],
        "cpu_baseline": cpu,
        "host": _host_info(),
        "workloads": subs,
        "generation_loop": generation_loop,
        "native_loops": native,
        "fork_latency_ns": _fork_sweep_ns(),
        "fork_latency_ns_ctypes": _fork_latency_ns(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
