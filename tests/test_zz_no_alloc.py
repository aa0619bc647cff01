"""tkv_attend_decode_noalloc against tkv_attend_decode (GPU).

The allocation-free decode call runs the same plan and kernels as the
workspace-taking call, with the plan and the split-K partial records in the
library's fixed per-device workspace.  Its outputs must equal the other
call's bit for bit: on the search tree (split-K chunks and a merge), then a
smaller batch right after (the fixed workspace keeps the previous call's
contents), then a workload with no partial records.  A call whose partial
records exceed the fixed workspace is refused with TKV_E_WORKSPACE.
"""

import numpy as np
import pytest

from workloads import recipes

from _gpu_common import need_gpu, say

pytestmark = pytest.mark.gpu


def _both(lib, layer, handles, q, torch):
    from tree_structured_copy_amd import tkv
    rows = len(handles)
    wl = lib.wl
    out_ref = torch.empty((rows, wl.q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    out_fix = torch.full_like(out_ref, float("nan"))
    need = tkv.tkv_workspace_size(lib.c, handles)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()
    tkv.tkv_attend_decode(lib.c, layer, handles, q, out_ref, ws, need, stream)
    tkv.tkv_attend_decode_noalloc(lib.c, layer, handles, q, out_fix, stream)
    torch.cuda.synchronize()
    return out_ref.cpu().numpy(), out_fix.cpu().numpy(), need


def test_noalloc_decode_equals_decode():
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    from workloads import device as wdev

    wl = recipes.mcts_tree()
    say("noalloc: %s" % wl.name)
    lib = LibReplay(wl, "cuda")
    try:
        i = lib.build()
        op = wl.ops[i]
        handles = lib.handles(op)
        q = wdev.q_tensor(wl, op[-1], len(handles))
        ref, fix, need = _both(lib, op[1], handles, q, torch)
        say("  %d queries, workspace %d bytes: max|diff| %g" % (len(handles), need, np.abs(ref - fix).max()))
        assert need > 0  # the search tree is cut into split-K chunks with partial records
        assert np.isfinite(ref).all()
        np.testing.assert_array_equal(fix, ref)
        assert "attn_merge_kernel" in ";".join(tkv.tkv_last_kernels(lib.c))
        # a smaller batch right after: the first 40 leaves
        small = handles[:40]
        ref2, fix2, need2 = _both(lib, op[1], small, q[:40].contiguous(), torch)
        say("  %d queries, workspace %d bytes: max|diff| %g" % (len(small), need2, np.abs(ref2 - fix2).max()))
        np.testing.assert_array_equal(fix2, ref2)
        # repeated calls change no device allocation
        torch.cuda.synchronize()
        free0 = torch.cuda.mem_get_info()[0]
        out = torch.empty((len(small), wl.q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
        for _ in range(10):
            tkv.tkv_attend_decode_noalloc(lib.c, op[1], small, q[:40].contiguous(), out, torch.cuda.current_stream())
        torch.cuda.synchronize()
        assert torch.cuda.mem_get_info()[0] == free0
        np.testing.assert_array_equal(out.cpu().numpy(), ref2)
    finally:
        lib.close()


def test_noalloc_decode_without_partials_and_refusal():
    torch = need_gpu()
    from tree_structured_copy_amd import tkv
    from tree_structured_copy_amd.replay import LibReplay
    from workloads import device as wdev

    wl = recipes.llama_fork()
    say("noalloc: %s" % wl.name)
    lib = LibReplay(wl, "cuda")
    try:
        i = lib.build()
        op = wl.ops[i]
        handles = lib.handles(op)
        q = wdev.q_tensor(wl, op[-1], len(handles))
        ref, fix, need = _both(lib, op[1], handles, q, torch)
        say("  %d queries, workspace %d bytes: max|diff| %g" % (len(handles), need, np.abs(ref - fix).max()))
        np.testing.assert_array_equal(fix, ref)
        # cut into one-block chunks, the call's partial records (about 550 MB)
        # exceed the fixed workspace: refused before anything is launched
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_TARGET_WGS, 1 << 20)
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_MIN_CHUNK, 1)
        assert tkv.tkv_workspace_size(lib.c, handles) > (64 << 20)
        out = torch.empty_like(torch.from_numpy(ref)).cuda()
        with pytest.raises(tkv.TkvError) as e:
            tkv.tkv_attend_decode_noalloc(lib.c, op[1], handles, q, out, torch.cuda.current_stream())
        assert e.value.code == tkv.TKV_E_WORKSPACE
        # and the cache still serves calls afterwards
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_TARGET_WGS, 256)
        tkv.tkv_set_option(lib.c, tkv.TKV_OPT_MIN_CHUNK, 32)
        ref3, fix3, _ = _both(lib, op[1], handles, q, torch)
        np.testing.assert_array_equal(fix3, ref3)
        np.testing.assert_array_equal(fix3, ref)
    finally:
        lib.close()
