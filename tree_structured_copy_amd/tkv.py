"""Python binding of libtkv (ctypes): the C entry points under the same names.

Argument marshalling only -- every step of the attention path runs in the HIP
library.  Device pointers may be given as ints or as objects with a
``data_ptr()`` method (torch tensors); streams as ints, ``None`` (null stream)
or objects with a ``cuda_stream`` attribute (torch streams).  Non-zero status
codes raise ``TkvError``.  Importing this module fails loudly if the library
has not been built.
"""

from __future__ import annotations

import ctypes
import os
from typing import List, Optional, Sequence

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libtkv.so")

TKV_F32 = 0
TKV_BF16 = 1

TKV_OK = 0
TKV_E_INVAL = -1
TKV_E_NOMEM = -2
TKV_E_BADSEQ = -3
TKV_E_SHARED = -4
TKV_E_EMPTY = -5
TKV_E_RANGE = -6
TKV_E_DEVICE = -7
TKV_E_WORKSPACE = -8
TKV_E_NODEVICE = -9

TKV_OPT_TARGET_WGS = 1
TKV_OPT_MIN_CHUNK = 2
TKV_OPT_MAX_ROWS = 3
TKV_OPT_PLAN_CACHE = 4
TKV_OPT_WAVES = 5
TKV_OPT_CASCADE = 6
TKV_OPT_CONCURRENT = 7
TKV_OPT_PLAN_PATCH = 8
TKV_OPT_FUSED_NEW_TOKEN = 9

STATUS_NAMES = {
    TKV_E_INVAL: "inval", TKV_E_NOMEM: "nomem", TKV_E_BADSEQ: "badseq", TKV_E_SHARED: "shared",
    TKV_E_EMPTY: "empty", TKV_E_RANGE: "range", TKV_E_DEVICE: "device",
    TKV_E_WORKSPACE: "workspace", TKV_E_NODEVICE: "nodevice",
}


class TkvError(RuntimeError):
    def __init__(self, code: int, what: str):
        self.code = code
        self.name = STATUS_NAMES.get(code, str(code))
        super().__init__("%s: %s (%d)" % (what, _lib.tkv_strerror(code).decode(), code))


class tkv_config(ctypes.Structure):
    _fields_ = [("num_layers", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("num_blocks", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("k_pool", ctypes.c_void_p), ("v_pool", ctypes.c_void_p)]


class tkv_counters(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in ("blocks_taken", "blocks_freed", "nodes_created",
                                              "nodes_freed", "block_ids_copied", "plans_built",
                                              "plans_uploaded", "plans_patched", "plans_reused")]


class tkv_plan_info(ctypes.Structure):
    _fields_ = [("groups", ctypes.c_int32), ("items", ctypes.c_int32),
                ("block_entries", ctypes.c_int32), ("unique_blocks", ctypes.c_int32),
                ("unique_tokens", ctypes.c_int64), ("partial_slots", ctypes.c_int64),
                ("items_per_kernel", ctypes.c_int32 * 6)]


def _load():
    # One process must hold one HIP runtime.  torch ships its own copy of
    # libamdhip64 and loads it by a file name that does not match the soname
    # this library links against, so if libtkv.so came first a second runtime
    # would be loaded behind torch.  Loading torch first lets libtkv.so bind to
    # torch's runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(_LIB_PATH):
        raise ImportError("libtkv.so is not built (run __graft_entry__.build() or "
                          "python -m tree_structured_copy_amd.build): %s" % _LIB_PATH)
    return ctypes.CDLL(_LIB_PATH)


_lib = _load()

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_U64 = ctypes.c_uint64
_SZ = ctypes.c_size_t
_pU64 = ctypes.POINTER(_U64)
_pI32 = ctypes.POINTER(_I32)

_SIGS = {
    "tkv_create": [ctypes.POINTER(tkv_config), ctypes.POINTER(_P)],
    "tkv_destroy": [_P],
    "tkv_seq_new": [_P, _pU64],
    "tkv_fork": [_P, _U64, _I32, _pU64],
    "tkv_release": [_P, _U64],
    "tkv_append": [_P, _U64, _I32, _P, _P, _P],
    "tkv_append_batch": [_P, _pU64, _pI32, _I32, _P, _P, _P],
    "tkv_truncate": [_P, _U64, _I64],
    "tkv_workspace_size": [_P, _pU64, _pI32, _I32, ctypes.POINTER(_SZ)],
    "tkv_attend_decode": [_P, _I32, _pU64, _I32, _P, _P, _P, _SZ, _P],
    "tkv_attend_verify": [_P, _I32, _pU64, _pI32, _I32, _P, _P, _P, _SZ, _P],
    "tkv_attend_decode_new_token": [_P, _I32, _pU64, _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "tkv_attend_decode_new_tokens": [_P, _I32, _pU64, ctypes.POINTER(_I32), _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "tkv_attend_verify_new_tokens": [_P, _I32, _pU64, ctypes.POINTER(_I32), _I32, _P, _P, _P, _P, _P, _SZ, _P],
    "tkv_attend_decode_noalloc": [_P, _I32, _pU64, _I32, _P, _P, _P],
    "tkv_gather": [_P, _U64, _I32, _P, _P, _P],
    "tkv_seq_len": [_P, _U64, ctypes.POINTER(_I64)],
    "tkv_block_table": [_P, _U64, _pI32, _pI32, _I32, _pI32],
    "tkv_block_refcount": [_P, _I32, _pI32],
    "tkv_block_refcounts": [_P, _pI32],
    "tkv_num_free": [_P, _pI32],
    "tkv_get_counters": [_P, ctypes.POINTER(tkv_counters)],
    "tkv_last_kernels": [_P, ctypes.c_char_p, _I32],
    "tkv_plan_info_get": [_P, _pU64, _pI32, _I32, ctypes.POINTER(tkv_plan_info)],
    "tkv_set_option": [_P, _I32, _I64],
    "tkv_get_option": [_P, _I32, ctypes.POINTER(_I64)],
    "tkv_profile_enable": [_P, _I32],
    "tkv_profile_read": [_P, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double),
                         ctypes.POINTER(_I64)],
}
for _name, _args in _SIGS.items():
    _f = getattr(_lib, _name)
    _f.argtypes = _args
    _f.restype = ctypes.c_int
_lib.tkv_strerror.argtypes = [ctypes.c_int]
_lib.tkv_strerror.restype = ctypes.c_char_p

EXPORTED = sorted(list(_SIGS) + ["tkv_strerror"])


def _check(rc: int, what: str) -> None:
    if rc != 0:
        raise TkvError(rc, what)


def _ptr(x) -> Optional[int]:
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if hasattr(x, "data_ptr"):
        return x.data_ptr()
    raise TypeError("expected a device pointer (int) or a tensor, got %r" % type(x))


def _stream(s) -> Optional[int]:
    if s is None:
        return None
    if isinstance(s, int):
        return s
    if hasattr(s, "cuda_stream"):
        return s.cuda_stream
    raise TypeError("expected a stream")


def seq_array(seqs: Sequence[int]):
    """A ctypes uint64 array of handles (build once, reuse across calls)."""
    if isinstance(seqs, ctypes.Array):
        return seqs
    return (_U64 * len(seqs))(*seqs)


def i32_array(vals: Sequence[int]):
    if isinstance(vals, ctypes.Array):
        return vals
    return (_I32 * len(vals))(*vals)


def tkv_strerror(code: int) -> str:
    return _lib.tkv_strerror(code).decode()


def tkv_create(num_layers: int, num_q_heads: int, num_kv_heads: int, head_dim: int, num_blocks: int,
               dtype: int, k_pool=None, v_pool=None, block_size: int = 16):
    cfg = tkv_config(num_layers, num_q_heads, num_kv_heads, head_dim, block_size, num_blocks, dtype, 0,
                     _ptr(k_pool), _ptr(v_pool))
    out = _P()
    _check(_lib.tkv_create(ctypes.byref(cfg), ctypes.byref(out)), "tkv_create")
    return out


def tkv_destroy(c) -> None:
    _check(_lib.tkv_destroy(c), "tkv_destroy")


def tkv_seq_new(c) -> int:
    s = _U64()
    _check(_lib.tkv_seq_new(c, ctypes.byref(s)), "tkv_seq_new")
    return s.value


def tkv_fork(c, parent: int, n: int) -> List[int]:
    arr = (_U64 * max(1, n))()
    _check(_lib.tkv_fork(c, parent, n, arr), "tkv_fork")
    return list(arr[:n])


def tkv_release(c, s: int) -> None:
    _check(_lib.tkv_release(c, s), "tkv_release")


def tkv_append(c, s: int, ntok: int, k=None, v=None, stream=None) -> None:
    _check(_lib.tkv_append(c, s, ntok, _ptr(k), _ptr(v), _stream(stream)), "tkv_append")


def tkv_append_batch(c, seqs, ntok, k=None, v=None, stream=None) -> None:
    sa = seq_array(seqs)
    na = i32_array(ntok)
    if len(na) != len(sa):
        raise ValueError("one token count per handle")
    _check(_lib.tkv_append_batch(c, sa, na, len(sa), _ptr(k), _ptr(v), _stream(stream)), "tkv_append_batch")


def tkv_truncate(c, s: int, new_len: int) -> None:
    _check(_lib.tkv_truncate(c, s, new_len), "tkv_truncate")


def tkv_workspace_size(c, seqs, nq=None) -> int:
    sa = seq_array(seqs)
    na = i32_array(nq) if nq is not None else None
    out = _SZ()
    _check(_lib.tkv_workspace_size(c, sa, na, len(sa), ctypes.byref(out)), "tkv_workspace_size")
    return out.value


def tkv_attend_decode(c, layer: int, seqs, q, out, ws=None, ws_bytes: int = 0, stream=None) -> None:
    sa = seq_array(seqs)
    _check(_lib.tkv_attend_decode(c, layer, sa, len(sa), _ptr(q), _ptr(out), _ptr(ws), ws_bytes,
                                  _stream(stream)), "tkv_attend_decode")


def tkv_attend_decode_noalloc(c, layer: int, seqs, q, out, stream=None) -> None:
    sa = seq_array(seqs)
    _check(_lib.tkv_attend_decode_noalloc(c, layer, sa, len(sa), _ptr(q), _ptr(out), _stream(stream)),
           "tkv_attend_decode_noalloc")


def tkv_attend_decode_new_token(c, layer: int, seqs, k_new, v_new, q, out, ws=None, ws_bytes: int = 0,
                                stream=None) -> None:
    sa = seq_array(seqs)
    _check(_lib.tkv_attend_decode_new_token(c, layer, sa, len(sa), _ptr(k_new), _ptr(v_new), _ptr(q), _ptr(out),
                                            _ptr(ws), ws_bytes, _stream(stream)), "tkv_attend_decode_new_token")


def tkv_attend_decode_new_tokens(c, layer: int, seqs, ntok, k_new, v_new, q, out, ws=None, ws_bytes: int = 0,
                                 stream=None) -> None:
    sa = seq_array(seqs)
    na = i32_array(ntok)
    _check(_lib.tkv_attend_decode_new_tokens(c, layer, sa, na, len(sa), _ptr(k_new), _ptr(v_new), _ptr(q),
                                             _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
           "tkv_attend_decode_new_tokens")


def tkv_attend_verify(c, layer: int, seqs, nq, q, out, ws=None, ws_bytes: int = 0, stream=None) -> None:
    sa = seq_array(seqs)
    na = i32_array(nq)
    _check(_lib.tkv_attend_verify(c, layer, sa, na, len(sa), _ptr(q), _ptr(out), _ptr(ws), ws_bytes,
                                  _stream(stream)), "tkv_attend_verify")


def tkv_attend_verify_new_tokens(c, layer: int, seqs, nq, k_new, v_new, q, out, ws=None, ws_bytes: int = 0,
                                 stream=None) -> None:
    sa = seq_array(seqs)
    na = i32_array(nq)
    _check(_lib.tkv_attend_verify_new_tokens(c, layer, sa, na, len(sa), _ptr(k_new), _ptr(v_new), _ptr(q),
                                             _ptr(out), _ptr(ws), ws_bytes, _stream(stream)),
           "tkv_attend_verify_new_tokens")


def tkv_gather(c, s: int, layer: int, k_out, v_out, stream=None) -> None:
    _check(_lib.tkv_gather(c, s, layer, _ptr(k_out), _ptr(v_out), _stream(stream)), "tkv_gather")


def tkv_seq_len(c, s: int) -> int:
    n = _I64()
    _check(_lib.tkv_seq_len(c, s, ctypes.byref(n)), "tkv_seq_len")
    return n.value


def tkv_block_table(c, s: int):
    n = _I32()
    rc = _lib.tkv_block_table(c, s, None, None, 0, ctypes.byref(n))
    if rc not in (0, TKV_E_RANGE):
        _check(rc, "tkv_block_table")
    cap = max(1, n.value)
    ids = (_I32 * cap)()
    valid = (_I32 * cap)()
    _check(_lib.tkv_block_table(c, s, ids, valid, cap, ctypes.byref(n)), "tkv_block_table")
    return [(ids[i], valid[i]) for i in range(n.value)]


def tkv_block_refcount(c, block: int) -> int:
    rc = _I32()
    _check(_lib.tkv_block_refcount(c, block, ctypes.byref(rc)), "tkv_block_refcount")
    return rc.value


def tkv_block_refcounts(c, num_blocks: int) -> List[int]:
    arr = (_I32 * num_blocks)()
    _check(_lib.tkv_block_refcounts(c, arr), "tkv_block_refcounts")
    return list(arr)


def tkv_num_free(c) -> int:
    n = _I32()
    _check(_lib.tkv_num_free(c, ctypes.byref(n)), "tkv_num_free")
    return n.value


def tkv_get_counters(c) -> dict:
    x = tkv_counters()
    _check(_lib.tkv_get_counters(c, ctypes.byref(x)), "tkv_get_counters")
    return {f: getattr(x, f) for f, _ in tkv_counters._fields_}


def tkv_last_kernels(c) -> list:
    """Names of the kernels the last attention call on c launched, in order."""
    buf = ctypes.create_string_buffer(1024)
    _check(_lib.tkv_last_kernels(c, buf, len(buf)), "tkv_last_kernels")
    v = buf.value.decode()
    return v.split(";") if v else []


def tkv_plan_info_get(c, seqs, nq=None) -> dict:
    sa = seq_array(seqs)
    na = i32_array(nq) if nq is not None else None
    x = tkv_plan_info()
    _check(_lib.tkv_plan_info_get(c, sa, na, len(sa), ctypes.byref(x)), "tkv_plan_info_get")
    d = {f: getattr(x, f) for f, _ in tkv_plan_info._fields_ if f != "items_per_kernel"}
    d["items_per_kernel"] = list(x.items_per_kernel)
    return d


def tkv_set_option(c, key: int, value: int) -> None:
    _check(_lib.tkv_set_option(c, key, value), "tkv_set_option")


def tkv_get_option(c, key: int) -> int:
    v = _I64()
    _check(_lib.tkv_get_option(c, key, ctypes.byref(v)), "tkv_get_option")
    return v.value


def tkv_profile_enable(c, on: bool) -> None:
    _check(_lib.tkv_profile_enable(c, 1 if on else 0), "tkv_profile_enable")


def tkv_profile_read(c):
    """(partial_ms, merge_ms, calls) since the last read."""
    a, b, n = ctypes.c_double(), ctypes.c_double(), _I64()
    _check(_lib.tkv_profile_read(c, ctypes.byref(a), ctypes.byref(b), ctypes.byref(n)), "tkv_profile_read")
    return a.value, b.value, n.value
