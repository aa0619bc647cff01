"""Pins for the oracle's attention half (CPU only).

Each check ties the oracle to something other than itself: hand-derived
fixtures, closed forms, invariants of softmax attention, and a library routine
(torch's scaled_dot_product_attention in float64 with an explicit mask).  The
mutation tests at the end plant plausible mistakes in the oracle and confirm
that at least one pin catches each.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import attention
from oracle.cache import ArraySource, MaterializedCache

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------------------
# closed forms and fixtures

def pin_fixtures(attend_one=None):
    attend_one = attend_one or attention.attend_one
    g = json.load(open(os.path.join(GOLD, "attn_small.json")))
    q = np.array(g["q"])
    t = g["two_keys"]
    np.testing.assert_allclose(attend_one(np.array(t["k"]), np.array(t["v"]), q), t["out"], atol=1e-12)
    t = g["three_keys"]
    K, V = np.array(t["k"]), np.array(t["v"])
    np.testing.assert_allclose(attend_one(K, V, q), t["out_all"], atol=1e-12)
    np.testing.assert_allclose(attend_one(K[:2], V[:2], q), t["out_upto_1"], atol=1e-12)


def pin_scale(attend_one=None):
    """d=16: q=4 e0, k0=e0, k1=0 -> scores 1 and 0, so the weight of v0 is the
    logistic function at 1, 1/(1+e^-1).  A 1/d or missing scale moves it."""
    attend_one = attend_one or attention.attend_one
    d = 16
    q = np.zeros(d); q[0] = 4.0
    K = np.zeros((2, d)); K[0, 0] = 1.0
    V = np.zeros((2, d)); V[0, :] = 1.0
    out = attend_one(K, V, q)
    np.testing.assert_allclose(out, np.full(d, 0.7310585786300049), atol=1e-14)


def pin_single_key(attend_one=None):
    attend_one = attend_one or attention.attend_one
    r = _rng(1)
    for d in (4, 64, 128):
        K = r.standard_normal((1, d)); V = r.standard_normal((1, d)); q = r.standard_normal(d) * 10
        np.testing.assert_array_equal(attend_one(K, V, q), V[0])


def pin_uniform_scores(attend_one=None):
    attend_one = attend_one or attention.attend_one
    r = _rng(2)
    K = r.standard_normal((37, 8)); V = r.standard_normal((37, 8))
    np.testing.assert_allclose(attend_one(K, V, np.zeros(8)), V.mean(axis=0), atol=1e-12)
    Ke = np.tile(r.standard_normal((1, 8)), (37, 1))
    np.testing.assert_allclose(attend_one(Ke, V, r.standard_normal(8)), V.mean(axis=0), atol=1e-12)


def pin_constant_v(attend_one=None):
    attend_one = attend_one or attention.attend_one
    r = _rng(3)
    K = r.standard_normal((50, 16)); V = np.full((50, 16), -1.25)
    np.testing.assert_allclose(attend_one(K, V, r.standard_normal(16) * 3), np.full(16, -1.25), atol=1e-12)


def pin_shift_and_permutation(attend_one=None):
    attend_one = attend_one or attention.attend_one
    r = _rng(4)
    K = r.standard_normal((40, 16)); V = r.standard_normal((40, 16)); q = r.standard_normal(16)
    base = attend_one(K, V, q)
    np.testing.assert_allclose(attend_one(K + r.standard_normal(16), V, q), base, atol=1e-12)
    p = r.permutation(40)
    np.testing.assert_allclose(attend_one(K[p], V[p], q), base, atol=1e-12)


def pin_large_scores(attend_one=None):
    """Huge scores: the output is the value of the arg-max key, with no overflow."""
    attend_one = attend_one or attention.attend_one
    r = _rng(5)
    K = r.standard_normal((30, 8)); V = r.standard_normal((30, 8)); q = r.standard_normal(8) * 1e4
    out = attend_one(K, V, q)
    np.testing.assert_allclose(out, V[np.argmax(K @ q)], atol=1e-12)


ATTEND_PINS = [pin_fixtures, pin_scale, pin_single_key, pin_uniform_scores, pin_constant_v,
               pin_shift_and_permutation, pin_large_scores]


@pytest.mark.parametrize("pin", ATTEND_PINS, ids=lambda f: f.__name__)
def test_attend_pins(pin):
    pin()


def pin_gqa_mapping(decode=None):
    """8 query heads over 2 KV heads: heads 0-3 read KV head 0, 4-7 read KV head 1."""
    decode = decode or attention.decode
    r = _rng(6)
    n, d = 20, 8
    K = r.standard_normal((n, 2, d))
    V = np.empty((n, 2, d)); V[:, 0, :] = 1.0; V[:, 1, :] = 2.0
    out = decode(K, V, r.standard_normal((8, d)), kv_heads=2)
    np.testing.assert_allclose(out[:, 0], [1, 1, 1, 1, 2, 2, 2, 2], atol=1e-12)


def test_gqa_mapping():
    pin_gqa_mapping()


# ---------------------------------------------------------------------------
# against a library routine on tiny random trees

def _sdpa(K, V, Q, mask):
    """torch SDPA in float64.  K, V: [n][Hkv][d]; Q: [m][Hq][d]; mask: [m][n] bool."""
    Hq, Hkv = Q.shape[1], K.shape[1]
    Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)  # [Hq][n][d]
    Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(Hq // Hkv, dim=0)
    Qt = torch.from_numpy(Q).permute(1, 0, 2)  # [Hq][m][d]
    mt = torch.from_numpy(mask)[None].expand(Hq, -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, attn_mask=mt)
    return o.permute(1, 0, 2).numpy()


def _random_tree_histories(seed, hkv, d):
    """Build a small random fork tree in the materialised cache; returns (cache, handles)."""
    r = _rng(seed)
    mc = MaterializedCache()
    root = mc.seq_new()
    n0 = int(r.integers(1, 20))
    mc.append(root, ArraySource(r.standard_normal((1, n0, hkv, d)), r.standard_normal((1, n0, hkv, d))))
    live = [root]
    for _ in range(12):
        h = live[r.integers(len(live))]
        if r.random() < 0.35:
            live.extend(mc.fork(h, int(r.integers(1, 4))))
        else:
            n = int(r.integers(1, 9))
            mc.append(h, ArraySource(r.standard_normal((1, n, hkv, d)), r.standard_normal((1, n, hkv, d))))
    return mc, live


@pytest.mark.parametrize("seed", range(6))
def test_decode_and_verify_match_torch_sdpa(seed):
    hq, hkv, d = 8, 2, 16
    mc, live = _random_tree_histories(seed, hkv, d)
    r = _rng(100 + seed)
    for h in live:
        L = mc.length(h)
        K = np.stack([mc.kv(h, 0, g)[0] for g in range(hkv)], axis=1)
        V = np.stack([mc.kv(h, 0, g)[1] for g in range(hkv)], axis=1)
        q = r.standard_normal((hq, d))
        dec = attention.decode(K, V, q, kv_heads=hkv)
        ref = _sdpa(K, V, q[None], np.ones((1, L), dtype=bool))[0]
        np.testing.assert_allclose(dec, ref, atol=1e-12)
        m = int(r.integers(1, L + 1))
        qs = r.standard_normal((m, hq, d))
        pos = np.arange(L - m, L)
        ver = attention.verify(K, V, qs, pos, kv_heads=hkv)
        mask = np.arange(L)[None, :] <= pos[:, None]
        np.testing.assert_allclose(ver, _sdpa(K, V, qs, mask), atol=1e-12)


def test_verify_reductions():
    """verify with one query == decode; verify row i == decode on the prefix up to p_i."""
    r = _rng(7)
    n, hkv, hq, d = 30, 2, 4, 16
    K = r.standard_normal((n, hkv, d)); V = r.standard_normal((n, hkv, d))
    q = r.standard_normal((1, hq, d))
    np.testing.assert_array_equal(attention.verify(K, V, q, [n - 1], hkv)[0],
                                  attention.decode(K, V, q[0], hkv))
    qs = r.standard_normal((6, hq, d))
    pos = list(range(n - 6, n))
    ver = attention.verify(K, V, qs, pos, hkv)
    for i, p in enumerate(pos):
        np.testing.assert_array_equal(ver[i], attention.decode(K[: p + 1], V[: p + 1], qs[i], hkv))


def test_fork_does_not_change_prefix_output():
    """Forking a branch and extending the children leaves the parent's output unchanged."""
    r = _rng(8)
    mc = MaterializedCache()
    h = mc.seq_new()
    mc.append(h, ArraySource(r.standard_normal((1, 21, 1, 8)), r.standard_normal((1, 21, 1, 8))))
    q = r.standard_normal((1, 8))
    before = attention.decode(*(a[:, None, :] for a in mc.kv(h, 0, 0)), q, 1)
    for c in mc.fork(h, 3):
        mc.append(c, ArraySource(r.standard_normal((1, 5, 1, 8)), r.standard_normal((1, 5, 1, 8))))
    after = attention.decode(*(a[:, None, :] for a in mc.kv(h, 0, 0)), q, 1)
    np.testing.assert_array_equal(before, after)


def test_branch_kv_is_its_path_and_identical_siblings_agree():
    """A branch's materialised K/V is its ancestors' tokens followed by its own, in order
    (written out by hand over a two-level fork); siblings given identical tokens give
    identical outputs, and a sibling given other tokens does not."""
    r = _rng(9)
    mc = MaterializedCache()
    root = mc.seq_new()
    pk, pv = r.standard_normal((1, 19, 2, 8)), r.standard_normal((1, 19, 2, 8))
    mc.append(root, ArraySource(pk, pv))
    a, b, c = mc.fork(root, 3)
    sk, sv = r.standard_normal((1, 6, 2, 8)), r.standard_normal((1, 6, 2, 8))
    for h in (a, b):
        mc.append(h, ArraySource(sk.copy(), sv.copy()))
    mc.append(c, ArraySource(r.standard_normal((1, 6, 2, 8)), r.standard_normal((1, 6, 2, 8))))
    (g,) = mc.fork(a, 1)
    gk, gv = r.standard_normal((1, 3, 2, 8)), r.standard_normal((1, 3, 2, 8))
    mc.append(g, ArraySource(gk, gv))
    for head in range(2):
        K, V = mc.kv(g, 0, head)
        np.testing.assert_array_equal(K, np.concatenate([pk[0, :, head], sk[0, :, head], gk[0, :, head]]))
        np.testing.assert_array_equal(V, np.concatenate([pv[0, :, head], sv[0, :, head], gv[0, :, head]]))
    q = r.standard_normal((4, 8))
    out = {h: attention.decode(*(np.stack([mc.kv(h, 0, k)[i] for k in range(2)], axis=1) for i in (0, 1)), q, 2)
           for h in (a, b, c)}
    np.testing.assert_array_equal(out[a], out[b])
    assert np.abs(out[a] - out[c]).max() > 1e-3


# ---------------------------------------------------------------------------
# planted mistakes: each must be caught by at least one pin

def _mut_scale_1_over_d(K, V, q):
    s = (K @ q) / q.shape[-1]
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def _mut_no_scale(K, V, q):
    s = K @ q
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def _mut_no_max_subtraction(K, V, q):
    s = (K @ q) / math.sqrt(q.shape[-1])
    w = np.exp(s)
    return (w @ V) / w.sum()


def _mut_transposed_value(K, V, q):
    s = (K @ q) / math.sqrt(q.shape[-1])
    w = np.exp(s - s.max())
    return (w @ V[::-1]) / w.sum()


def _mut_drop_last_key(K, V, q):
    if K.shape[0] > 1:
        K, V = K[:-1], V[:-1]
    s = (K @ q) / math.sqrt(q.shape[-1])
    w = np.exp(s - s.max())
    return (w @ V) / w.sum()


def _mut_unnormalised(K, V, q):
    s = (K @ q) / math.sqrt(q.shape[-1])
    w = np.exp(s - s.max())
    return w @ V


@pytest.mark.parametrize("mutant", [_mut_scale_1_over_d, _mut_no_scale, _mut_no_max_subtraction,
                                    _mut_transposed_value, _mut_drop_last_key, _mut_unnormalised],
                         ids=lambda f: f.__name__)
def test_pins_catch_planted_attention_mistakes(mutant):
    caught = 0
    for pin in ATTEND_PINS:
        try:
            with np.errstate(all="ignore"):
                pin(mutant)
        except AssertionError:
            caught += 1
    assert caught > 0, "no pin caught the planted mistake"


def test_pins_catch_gqa_modulo_mapping(monkeypatch):
    monkeypatch.setattr(attention, "kv_head_of", lambda hq, q_heads, kv_heads: hq % kv_heads)
    with pytest.raises(AssertionError):
        pin_gqa_mapping()


def test_pins_catch_causal_off_by_one(monkeypatch):
    real = attention.attend_one

    def sees_one_less(K, V, q):  # what a j < p mask would compute for the verify rows
        return real(K[:-1], V[:-1], q) if K.shape[0] > 1 else real(K, V, q)

    monkeypatch.setattr(attention, "attend_one", sees_one_less)
    with pytest.raises(AssertionError):
        test_decode_and_verify_match_torch_sdpa(0)
