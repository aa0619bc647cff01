"""Replay a workload recipe (``workloads.recipes``) through the tkv C ABI.

Pools, queries and outputs are torch device tensors; K/V/Q values come from
the seeded device generator.  With ``device=None`` the cache is host-only
(block tables and allocator only; appends reserve slots without KV).
"""

from __future__ import annotations

from typing import Dict, Optional

from . import tkv


class LibReplay:
    def __init__(self, wl, device: Optional[str] = "cuda", extra_blocks: int = 0, pools=None):
        self.wl = wl
        self.device = device
        self.num_blocks = wl.num_blocks + extra_blocks
        self.h: Dict[int, int] = {}
        self.k_pool = self.v_pool = None
        dt = tkv.TKV_BF16 if wl.dtype == "bf16" else tkv.TKV_F32
        if device is not None:
            import torch
            from workloads import device as wdev
            if pools is not None:
                self.k_pool, self.v_pool = pools
            else:
                n = wl.layers * self.num_blocks * wl.kv_heads * 16 * wl.head_dim
                self.k_pool = torch.empty(n, dtype=wdev.torch_dtype(wl.dtype), device=device)
                self.v_pool = torch.empty(n, dtype=wdev.torch_dtype(wl.dtype), device=device)
        self.c = tkv.tkv_create(wl.layers, wl.q_heads, wl.kv_heads, wl.head_dim, self.num_blocks, dt,
                                self.k_pool, self.v_pool)
        self._ws = None

    def close(self):
        if self.c is not None:
            tkv.tkv_destroy(self.c)
            self.c = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    # -- structural ops ------------------------------------------------------------
    def apply(self, op) -> None:
        kind = op[0]
        if kind == "new":
            self.h[op[1]] = tkv.tkv_seq_new(self.c)
        elif kind == "append":
            _, h, ntok, call = op
            if self.device is None:
                tkv.tkv_append(self.c, self.h[h], ntok)
            else:
                import torch
                from workloads import device as wdev, gen
                k = wdev.kv_tensor(self.wl, call, ntok, gen.KIND_K, self.device)
                v = wdev.kv_tensor(self.wl, call, ntok, gen.KIND_V, self.device)
                tkv.tkv_append(self.c, self.h[h], ntok, k, v, torch.cuda.current_stream())
        elif kind == "append_batch":
            _, hs, ns, call = op
            seqs = [self.h[h] for h in hs]
            if self.device is None:
                tkv.tkv_append_batch(self.c, seqs, ns)
            else:
                import torch
                from workloads import device as wdev, gen
                total = sum(ns)
                k = wdev.kv_tensor(self.wl, call, total, gen.KIND_K, self.device)
                v = wdev.kv_tensor(self.wl, call, total, gen.KIND_V, self.device)
                tkv.tkv_append_batch(self.c, seqs, ns, k, v, torch.cuda.current_stream())
        elif kind == "reserve_batch":
            hs = op[1]
            ns = list(op[3]) if len(op) > 3 else [1] * len(hs)
            tkv.tkv_append_batch(self.c, [self.h[h] for h in hs], ns)
        elif kind == "fork":
            _, h, n, kids = op
            for name, s in zip(kids, tkv.tkv_fork(self.c, self.h[h], n)):
                self.h[name] = s
        elif kind == "release":
            tkv.tkv_release(self.c, self.h.pop(op[1]))
        elif kind == "truncate":
            _, h, L = op
            tkv.tkv_truncate(self.c, self.h[h], L)
        elif kind in ("decode", "decode_new", "verify", "verify_new", "time_begin"):
            pass
        else:
            raise ValueError(kind)

    def build(self, stop_at_attend: bool = True):
        """Apply ops up to (not including) the first decode/verify; returns its index."""
        for i, op in enumerate(self.wl.ops):
            if stop_at_attend and op[0] in ("decode", "decode_new", "verify", "verify_new"):
                return i
            self.apply(op)
        return len(self.wl.ops)

    # -- attention -------------------------------------------------------------------
    def handles(self, op):
        return [self.h[x] for x in op[2]]

    def nrows(self, op) -> int:
        return sum(op[3]) if op[0] in ("verify", "verify_new") else len(op[2])

    def workspace(self, op):
        import torch
        seqs = self.handles(op)
        nq = op[3] if op[0] in ("verify", "verify_new") else None
        need = tkv.tkv_workspace_size(self.c, seqs, nq)
        if need and (self._ws is None or self._ws.numel() < need):
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.device)
        return (self._ws if need else None), need

    def attend(self, op, q=None, out=None):
        """Run a decode/verify op; returns the fp32 output tensor [rows][Hq][D]."""
        import torch
        from workloads import device as wdev
        wl = self.wl
        rows = self.nrows(op)
        if q is None:
            q = wdev.q_tensor(wl, op[-1], rows, self.device)
        if out is None:
            out = torch.empty((rows, wl.q_heads, wl.head_dim), dtype=torch.float32, device=self.device)
        ws, need = self.workspace(op)
        stream = torch.cuda.current_stream()
        if op[0] == "decode":
            tkv.tkv_attend_decode(self.c, op[1], self.handles(op), q, out, ws, need, stream)
        elif op[0] == "decode_new":
            # the reserved tokens' K/V of this layer: rows of batched append call op[3]
            from workloads import gen
            ns = list(op[4]) if len(op) > 5 else [1] * rows
            total = sum(ns)
            k = wdev.kv_tensor(wl, op[3], total, gen.KIND_K, self.device)[op[1]].contiguous()
            v = wdev.kv_tensor(wl, op[3], total, gen.KIND_V, self.device)[op[1]].contiguous()
            if len(op) > 5:
                tkv.tkv_attend_decode_new_tokens(self.c, op[1], self.handles(op), ns, k, v, q, out, ws, need, stream)
            else:
                tkv.tkv_attend_decode_new_token(self.c, op[1], self.handles(op), k, v, q, out, ws, need, stream)
        elif op[0] == "verify_new":
            # the verified tokens are the reserved ones: their K/V of this layer
            # are rows of batched append call op[4], in batch order
            from workloads import gen
            total = sum(op[3])
            k = wdev.kv_tensor(wl, op[4], total, gen.KIND_K, self.device)[op[1]].contiguous()
            v = wdev.kv_tensor(wl, op[4], total, gen.KIND_V, self.device)[op[1]].contiguous()
            tkv.tkv_attend_verify_new_tokens(self.c, op[1], self.handles(op), op[3], k, v, q, out, ws, need, stream)
        else:
            tkv.tkv_attend_verify(self.c, op[1], self.handles(op), op[3], q, out, ws, need, stream)
        return out
