"""Shared helpers for the GPU parity tests (library vs oracle on the same seeded inputs)."""

from __future__ import annotations

import sys

import numpy as np
import pytest

TOL = {"f32": 1e-5, "bf16": 2e-3}


def need_gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    # On a GPU machine the HIP library must be there: a missing build is a failure.
    from tree_structured_copy_amd import tkv  # noqa: F401
    return torch


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def oracle_threads():
    """Threads for the oracle's bulk checks: the host's cores, at most 16."""
    import os
    return max(1, min(16, len(os.sched_getaffinity(0))))


def run_both(wl, sample=None, options=None, extra_blocks=0, check_tables=True, threads=1, counters=None):
    """Replay wl on the library (GPU) and the oracle; compare every attend op.

    sample: None = every row and head, or a function (op, nrows) -> [(row, head)]
    (or None for every row and head of that op, or [] for none of it).  threads: the oracle's
    (OracleReplay) for large checks.  counters: a dict to receive the
    library's tkv_get_counters at the end.
    Returns a list of (op, max_abs_err, n_compared).
    """
    torch = need_gpu()
    from oracle.replay import OracleReplay
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay

    say("run_both: %s dtype=%s Hq=%d Hkv=%d D=%d blocks=%d" % (wl.name, wl.dtype, wl.q_heads, wl.kv_heads,
                                                              wl.head_dim, wl.num_blocks))
    lib = LibReplay(wl, "cuda", extra_blocks=extra_blocks)
    orc = OracleReplay(wl, threads=threads)
    for k, v in (options or {}).items():
        tkv.tkv_set_option(lib.c, k, v)
    results = []
    try:
        for op in wl.ops:
            if op[0] in ("decode", "decode_new", "verify", "verify_new"):
                out = lib.attend(op)
                torch.cuda.synchronize()
                rows = lib.nrows(op)
                smp = None if sample is None else sample(op, rows)
                if smp is not None and len(smp) == 0:
                    # nothing of this call is compared (a later one is)
                    lib.apply(op)
                    orc.apply(op)
                    continue
                ref = orc.attend(op, smp)
                got = out.double().cpu().numpy()
                if smp is None:
                    err = float(np.max(np.abs(got - ref)))
                    n = ref.size
                else:
                    idx = np.array(smp)
                    err = float(np.max(np.abs(got[idx[:, 0], idx[:, 1]] - ref[idx[:, 0], idx[:, 1]])))
                    n = len(smp) * wl.head_dim
                assert np.isfinite(got).all(), "non-finite output"
                if check_tables:
                    for hname in op[2]:
                        assert tkv.tkv_block_table(lib.c, lib.h[hname]) == orc.alloc.table(orc.h_alloc[hname])
                results.append((op[0], err, n))
                say("  %s layer %d rows %d: max|err| %.3g over %d values" % (op[0], op[1], rows, err, n))
            lib.apply(op)
            orc.apply(op)
        if check_tables:
            assert tkv.tkv_num_free(lib.c) == orc.alloc.num_free()
        if counters is not None:
            counters.update(tkv.tkv_get_counters(lib.c))
    finally:
        lib.close()
        del lib
        torch.cuda.empty_cache()
    return results


def assert_close(results, dtype):
    for kind, err, n in results:
        say("max abs error %.3e over %d outputs (%s, %s)" % (err, n, kind, dtype))
        assert err <= TOL[dtype], (kind, err)
