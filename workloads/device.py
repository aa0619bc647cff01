"""Device-side seeded inputs (same definition as ``workloads.gen``), via libtkvgen.so.

Fills torch tensors on the GPU with exactly the values ``gen.values`` returns on
the host, so the HIP path can build large workloads without host copies.
"""

from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

from . import gen

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libtkvgen.so")
_lib = None
_tables = {}


def _load():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libtkvgen.so is not built: %s" % _LIB_PATH)
        _lib = ctypes.CDLL(_LIB_PATH)
        _lib.tkvgen_fill.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint64, ctypes.c_uint64,
                                     ctypes.c_uint64, ctypes.c_uint64, ctypes.c_void_p, ctypes.c_void_p]
        _lib.tkvgen_fill.restype = ctypes.c_int
    return _lib


def torch_dtype(dtype: str):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _table(dtype: str, device) -> torch.Tensor:
    key = (dtype, str(device))
    if key not in _tables:
        bits = gen.normal_table_bits(dtype)
        t = torch.from_numpy(bits.view(np.int16) if dtype == "bf16" else bits.view(np.int32))
        _tables[key] = t.to(device)
    return _tables[key]


def fill(out: torch.Tensor, dtype: str, seed: int, stream: int, offset: int = 0) -> torch.Tensor:
    """out.view(-1)[i] = element (offset + i) of the stream."""
    lib = _load()
    if not out.is_contiguous() or out.dtype != torch_dtype(dtype):
        raise ValueError("fill needs a contiguous tensor of the workload dtype")
    eb = 2 if dtype == "bf16" else 4
    tab = _table(dtype, out.device)
    s = torch.cuda.current_stream(out.device).cuda_stream
    rc = lib.tkvgen_fill(out.data_ptr(), eb, seed, stream, offset, out.numel(), tab.data_ptr(), s)
    if rc != 0:
        raise RuntimeError("tkvgen_fill failed (%d)" % rc)
    return out


def kv_tensor(wl, call: int, ntok: int, kind: int, device="cuda") -> torch.Tensor:
    t = torch.empty((wl.layers, ntok, wl.kv_heads, wl.head_dim), dtype=torch_dtype(wl.dtype), device=device)
    return fill(t, wl.dtype, wl.seed, gen.stream_id(kind, call))


def q_tensor(wl, qcall: int, nrows: int, device="cuda") -> torch.Tensor:
    t = torch.empty((nrows, wl.q_heads, wl.head_dim), dtype=torch_dtype(wl.dtype), device=device)
    t = fill(t, wl.dtype, wl.seed, gen.stream_id(gen.KIND_Q, qcall))
    return t.mul_(wl.q_scale) if wl.q_scale != 1 else t
