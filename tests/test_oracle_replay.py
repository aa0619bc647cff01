"""Pins for the oracle's replay layer (CPU only).

``OracleReplay`` turns a recipe into reference outputs: it keeps each handle's
materialised history through forks, appends, batched appends, reserved tokens
and truncations, decides where every query row sits (a decode query at the
last position L - 1; the verify queries of a handle at L - nq .. L - 1, the
parallel verification of a draft block in the DSpark blog, second layer), and
attends over positions 0..p.  Here a short recipe that uses every operation is
replayed, and its outputs are compared with histories written out by hand from
the recipe (whole-call input arrays sliced and concatenated by hand) and
attention computed by torch's scaled_dot_product_attention in float64 with an
explicit boolean mask.  ``MaterializedCache.truncate`` and the index formula
of ``workloads.kv_slice`` are pinned on their own.  Planted mistakes at the
end (an off-by-one query position, a wrong batch offset, a truncation that
keeps one token too many, a transposed generator index, a dropped last key)
must each fail a pin.
"""

import dataclasses

import numpy as np
import pytest
import torch

import workloads
from oracle import attention, cache as oc, replay as orp
from oracle.cache import ArraySource, MaterializedCache
from oracle.replay import OracleReplay
from workloads import gen, recipes

HQ, HKV, D, LAYERS = 4, 2, 8, 2


def _wl():
    ops = [
        ("new", 0),
        ("append", 0, 6, 0),
        ("fork", 0, 2, [1, 2]),
        ("release", 0),
        ("append_batch", [1, 2], [3, 2], 1),
        ("decode", 1, [1, 2], 100),
        ("verify", 0, [1, 2], [3, 2], 101),
        ("truncate", 1, 7),
        ("append", 1, 2, 2),
        ("decode", 0, [2, 1], 102),
        ("verify", 1, [1], [3], 103),
        ("reserve_batch", [2, 1], 3),
        ("decode_new", 0, [2, 1], 3, 104),
        ("fork", 2, 1, [3]),
        ("append", 3, 1, 4),
        ("decode", 1, [3, 2, 1], 105),
        ("truncate", 1, 6),
        ("append_batch", [1, 3], [2, 1], 5),
        ("verify", 0, [1, 3], [2, 2], 106),
        ("reserve_batch", [3, 1], 6, [2, 3]),
        ("decode_new", 1, [3, 1], 6, [2, 3], 107),
        ("reserve_batch", [1, 3], 7, [2, 1]),
        ("verify_new", 0, [1, 3], [2, 1], 7, 108),
    ]
    return recipes.Workload(name="replay_pin", dtype="f32", layers=LAYERS, q_heads=HQ, kv_heads=HKV, head_dim=D,
                            num_blocks=64, ops=ops, seed=11, block_size=4)


def _call(wl, call, ntok):
    """Whole input arrays of one append call: K, V [layers][ntok][Hkv][d]."""
    return (workloads.kv_values(wl, call, ntok, gen.KIND_K).astype(np.float64),
            workloads.kv_values(wl, call, ntok, gen.KIND_V).astype(np.float64))


def _cat(*parts):
    return tuple(np.concatenate([p[i] for p in parts], axis=1) for i in (0, 1))


def _rows(kv, a, b):
    return kv[0][:, a:b], kv[1][:, a:b]


def _expected_cases(wl):
    """Every attend op of the recipe with its query rows (handle, position) and the
    histories of those handles, written out by hand from the recipe."""
    P = _call(wl, 0, 6)
    B1 = _call(wl, 1, 5)      # h1 takes rows 0..2, h2 rows 3..4
    C2 = _call(wl, 2, 2)
    R3 = _call(wl, 3, 2)      # reserved in batch order [2, 1]: h2 row 0, h1 row 1
    C4 = _call(wl, 4, 1)
    B5 = _call(wl, 5, 3)      # h1 rows 0..1, h3 row 2
    h1 = _cat(P, _rows(B1, 0, 3))
    h2 = _cat(P, _rows(B1, 3, 5))
    cases = {
        100: ([(1, 8), (2, 7)], {1: h1, 2: h2}),
        101: ([(1, 6), (1, 7), (1, 8), (2, 6), (2, 7)], {1: h1, 2: h2}),
    }
    h1 = _cat(P, _rows(B1, 0, 1), C2)                  # truncated to 7, then 2 more
    cases[102] = ([(2, 7), (1, 8)], {1: h1, 2: h2})
    cases[103] = ([(1, 6), (1, 7), (1, 8)], {1: h1})
    h2 = _cat(h2, _rows(R3, 0, 1))
    h1 = _cat(h1, _rows(R3, 1, 2))
    cases[104] = ([(2, 8), (1, 9)], {1: h1, 2: h2})
    h3 = _cat(h2, C4)
    cases[105] = ([(3, 9), (2, 8), (1, 9)], {1: h1, 2: h2, 3: h3})
    h1 = _cat(P, _rows(B5, 0, 2))                      # truncated to the prefix, then 2 more
    h3 = _cat(h3, _rows(B5, 2, 3))
    cases[106] = ([(1, 6), (1, 7), (3, 9), (3, 10)], {1: h1, 3: h3})
    R6 = _call(wl, 6, 5)      # reserved with counts [2, 3] in batch order [3, 1]: h3 rows 0..1, h1 rows 2..4
    h3 = _cat(h3, _rows(R6, 0, 2))
    h1 = _cat(h1, _rows(R6, 2, 5))
    cases[107] = ([(3, 12), (1, 10)], {1: h1, 3: h3})
    R7 = _call(wl, 7, 3)      # reserved with counts [2, 1] in batch order [1, 3], then verified
    h1 = _cat(h1, _rows(R7, 0, 2))
    h3 = _cat(h3, _rows(R7, 2, 3))
    cases[108] = ([(1, 11), (1, 12), (3, 13)], {1: h1, 3: h3})
    return cases


def _sdpa_rows(hist, rows, Q, layer):
    """torch SDPA in float64, one row at a time with an explicit mask (key j visible iff j <= p)."""
    out = np.empty((len(rows), HQ, D))
    for r, (h, p) in enumerate(rows):
        K, V = hist[h][0][layer], hist[h][1][layer]          # [L][Hkv][d]
        L = K.shape[0]
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(HQ // HKV, dim=0)
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(HQ // HKV, dim=0)
        q = torch.from_numpy(Q[r].astype(np.float64))[:, None, :]
        mask = torch.from_numpy(np.arange(L) <= p)[None, None, :].expand(HQ, 1, L)
        out[r] = torch.nn.functional.scaled_dot_product_attention(q, Kt, Vt, attn_mask=mask)[:, 0, :].numpy()
    return out


def pin_replay_outputs():
    """Every attend op of the recipe equals SDPA over the hand-written histories, at
    the hand-written query positions; every query row's (handle, position) is the
    hand-written one."""
    wl = _wl()
    cases = _expected_cases(wl)
    orc = OracleReplay(wl)
    seen = 0
    for op in wl.ops:
        if op[0] in ("decode", "decode_new", "verify", "verify_new"):
            qcall = op[-1]
            rows, hist = cases[qcall]
            assert orc.query_rows(op) == rows, (qcall, orc.query_rows(op))
            Q = workloads.q_values(wl, qcall, len(rows))
            ref = _sdpa_rows(hist, rows, Q, op[1])
            got = orc.attend(op)
            np.testing.assert_allclose(got, ref, atol=1e-12, rtol=0)
            # a sample computes the same values and leaves the rest NaN
            smp = [(0, 0), (len(rows) - 1, HQ - 1)]
            part = orc.attend(op, smp)
            for r, hq in smp:
                np.testing.assert_array_equal(part[r, hq], got[r, hq])
            assert np.isnan(part).sum() == (len(rows) * HQ - len(smp)) * D
            seen += 1
        orc.apply(op)
    assert seen == len(cases)


def test_replay_outputs_match_hand_written_histories():
    pin_replay_outputs()


def test_replay_tables_follow_the_recipe():
    """The allocator half of the replay: after the recipe, each live handle's table
    covers exactly its length, and the free count is what the blocks in use leave."""
    wl = _wl()
    orc = OracleReplay(wl)
    for op in wl.ops:
        orc.apply(op)
    lens = {1: 13, 2: 9, 3: 14}
    used = set()
    for h, L in lens.items():
        tab = orc.alloc.table(orc.h_alloc[h])
        assert sum(v for _, v in tab) == L == orc.mat.length(orc.h_mat[h])
        used.update(b for b, _ in tab)
    assert orc.alloc.num_free() == wl.num_blocks - len(used)


def pin_truncate():
    """MaterializedCache.truncate(h, L) keeps exactly the first L tokens: a cut inside a
    segment, at a segment boundary, L = 0 and L = length."""
    r = np.random.default_rng(12)
    segs = [r.standard_normal((1, n, 1, 4)) for n in (5, 3, 7)]
    full = np.concatenate(segs, axis=1)[0, :, 0, :]
    for L in (0, 1, 4, 5, 6, 8, 11, 15):
        mc = MaterializedCache()
        h = mc.seq_new()
        for s in segs:
            mc.append(h, ArraySource(s, -s))
        mc.truncate(h, L)
        assert mc.length(h) == L
        K, V = mc.kv(h, 0, 0)
        if L == 0:
            assert K.size == 0 and V.size == 0
        else:
            np.testing.assert_array_equal(K, full[:L])
            np.testing.assert_array_equal(V, -full[:L])
        # later appends land after the cut
        extra = r.standard_normal((1, 2, 1, 4))
        mc.append(h, ArraySource(extra, extra))
        K, _ = mc.kv(h, 0, 0)
        np.testing.assert_array_equal(K, np.concatenate([full[:L], extra[0, :, 0, :]]))


def test_truncate_keeps_the_first_tokens():
    pin_truncate()


def pin_kv_slice():
    """workloads.kv_slice (one layer, one KV head, tokens [t0, t1), computed from the
    flat index) equals the matching slice of workloads.kv_values (the call's whole
    [layers][ntok][Hkv][d] array generated in order)."""
    r = np.random.default_rng(13)
    for dtype in ("f32", "bf16"):
        wl = recipes.Workload(name="slice", dtype=dtype, layers=3, q_heads=6, kv_heads=3, head_dim=16,
                              num_blocks=1, ops=[], seed=5)
        for call, ntok in ((0, 9), (7, 33)):
            for kind in (gen.KIND_K, gen.KIND_V):
                whole = workloads.kv_values(wl, call, ntok, kind)
                for _ in range(6):
                    layer, kvh = int(r.integers(wl.layers)), int(r.integers(wl.kv_heads))
                    t0 = int(r.integers(ntok))
                    t1 = int(r.integers(t0 + 1, ntok + 1))
                    np.testing.assert_array_equal(workloads.kv_slice(wl, call, ntok, kind, layer, kvh, t0, t1),
                                                  whole[layer, t0:t1, kvh, :])


def test_query_scale_multiplies_every_query_value():
    wl = recipes.verify_workload("qs", dtype="bf16", q_heads=4, kv_heads=2, head_dim=64, requests=1, prefix=5,
                                 paths=2, drafts=3, seed=9)
    base = workloads.q_values(wl, 3, 6)
    for scale in (2, 4):
        scaled = workloads.q_values(dataclasses.replace(wl, q_scale=scale), 3, 6)
        assert np.array_equal(scaled, base * scale)
    with pytest.raises(ValueError):
        recipes.ops_text(dataclasses.replace(wl, q_scale=2))


def test_kv_slice_is_a_slice_of_kv_values():
    pin_kv_slice()


REPLAY_PINS = [pin_replay_outputs, pin_truncate, pin_kv_slice]


def _caught():
    n = 0
    for pin in REPLAY_PINS:
        try:
            pin()
        except (AssertionError, ValueError, IndexError):
            n += 1
    return n


def test_pins_pass_unplanted():
    assert _caught() == 0


def test_pins_catch_verify_position_off_by_one(monkeypatch):
    def rows(self, op):
        out = []
        if op[0] in ("decode", "decode_new"):
            for h in op[2]:
                out.append((h, self.mat.length(self.h_mat[h]) - 1))
        else:
            for h, nq in zip(op[2], op[3]):
                L = self.mat.length(self.h_mat[h])
                out += [(h, L - nq + i - 1) for i in range(nq)]
        return out
    monkeypatch.setattr(OracleReplay, "query_rows", rows)
    assert _caught() > 0


def test_pins_catch_decode_position_off_by_one(monkeypatch):
    orig = OracleReplay.query_rows

    def rows(self, op):
        r = orig(self, op)
        return [(h, p - 1) for h, p in r] if op[0] in ("decode", "decode_new") else r
    monkeypatch.setattr(OracleReplay, "query_rows", rows)
    assert _caught() > 0


def test_pins_catch_wrong_batch_offset(monkeypatch):
    orig = orp._batch_source_for
    monkeypatch.setattr(orp, "_batch_source_for",
                        lambda wl, call, total, first, ntok, arrays=None: orig(wl, call, total, 0, ntok, arrays))
    assert _caught() > 0


def test_pins_catch_truncate_keeping_one_more(monkeypatch):
    orig = oc.MaterializedCache.truncate

    def trunc(self, h, new_len):
        orig(self, h, min(new_len + 1, self.length(h)))
    monkeypatch.setattr(oc.MaterializedCache, "truncate", trunc)
    assert _caught() > 0


def test_pins_catch_transposed_generator_index(monkeypatch):
    def bad_slice(wl, call, ntok, kind, layer, kvh, t0, t1):
        t = np.arange(t0, t1, dtype=np.uint64)[:, None]
        d = np.arange(wl.head_dim, dtype=np.uint64)[None, :]
        # token-major instead of layer-major
        idx = ((t * np.uint64(wl.layers) + np.uint64(layer)) * np.uint64(wl.kv_heads) + np.uint64(kvh)) \
            * np.uint64(wl.head_dim) + d
        return gen.values(wl.seed, gen.stream_id(kind, call), idx.reshape(-1), wl.dtype).reshape(t1 - t0, wl.head_dim)
    monkeypatch.setattr(workloads, "kv_slice", bad_slice)
    assert _caught() > 0


def test_pins_catch_reservation_counts_ignored(monkeypatch):
    orig = OracleReplay.apply

    def apply(self, op):
        if op[0] == "reserve_batch":
            op = op[:3]  # one token per handle whatever the counts
        orig(self, op)
    monkeypatch.setattr(OracleReplay, "apply", apply)
    assert _caught() > 0


def test_pins_catch_dropped_last_key(monkeypatch):
    orig = attention.attend_one

    def drop_last(K, V, q):
        return orig(K[:-1], V[:-1], q) if len(K) > 1 else orig(K, V, q)
    monkeypatch.setattr(attention, "attend_one", drop_last)
    assert _caught() > 0


def test_bulk_generated_replay_is_the_same_replay():
    """OracleReplay with threads (append values generated a whole layer of a call
    at a time, handles attended in parallel) gives bit-identical outputs."""
    wl = _wl()
    a, b = OracleReplay(wl), OracleReplay(wl, threads=4)
    for op in wl.ops:
        if op[0] in ("decode", "decode_new", "verify"):
            np.testing.assert_array_equal(a.attend(op), b.attend(op))
        a.apply(op)
        b.apply(op)


def test_preloaded_replay_is_the_same_replay():
    """OracleReplay over values generated up front (PreloadedArrays) gives
    bit-identical outputs."""
    from oracle.replay import PreloadedArrays
    wl = _wl()
    a, b = OracleReplay(wl), OracleReplay(wl, threads=2, arrays=PreloadedArrays(wl, 2))
    for op in wl.ops:
        if op[0] in ("decode", "decode_new", "verify"):
            np.testing.assert_array_equal(a.attend(op), b.attend(op))
        a.apply(op)
        b.apply(op)
