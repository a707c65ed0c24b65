"""Pins of the fp64 oracle's attention definition against things other than
itself: brute force with pure-Python loops, hand-derived closed forms,
invariants, finite differences, and planted mistakes that must be caught."""
import json
import math
import os

import numpy as np
import pytest

from oracle import attention as A

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def _ev(expr):
    return float(eval(expr, {"__builtins__": {}}, {"log": math.log}))


def brute_force(q, k, v, qpos, kpos, scale, causal, qdoc=None, kdoc=None):
    """Nested loops and math.fsum, straight from the definition."""
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    o = np.zeros((lq, hq, d))
    lse = np.full((hq, lq), -math.inf)
    for h in range(hq):
        g = h // (hq // hkv)
        for i in range(lq):
            keys = [j for j in range(lk)
                    if (not causal or kpos[j] <= qpos[i])
                    and (qdoc is None or qdoc[i] == kdoc[j])]
            if not keys:
                continue
            s = [scale * math.fsum(float(q[i, h, e]) * float(k[j, g, e]) for e in range(d))
                 for j in keys]
            m = max(s)
            ell = math.fsum(math.exp(x - m) for x in s)
            lse[h, i] = m + math.log(ell)
            for e in range(d):
                o[i, h, e] = math.fsum(math.exp(s[t] - lse[h, i]) * float(v[j, g, e])
                                       for t, j in enumerate(keys))
    return o, lse


def _case(rng, lq, lk, hq, hkv, d, docs):
    q = rng.standard_normal((lq, hq, d))
    k = rng.standard_normal((lk, hkv, d))
    v = rng.standard_normal((lk, hkv, d))
    # monotone but gappy global positions, queries offset into the keys
    kpos = np.cumsum(rng.integers(1, 3, size=lk)) - 1
    qpos = np.sort(rng.choice(np.arange(max(kpos[-1] + 3, lq)), size=lq, replace=False))
    qdoc = kdoc = None
    if docs:
        bounds = np.sort(rng.choice(np.arange(1, kpos[-1] + 3), size=2, replace=False))
        qdoc = np.searchsorted(bounds, qpos, side="right").astype(np.int32)
        kdoc = np.searchsorted(bounds, kpos, side="right").astype(np.int32)
    return q, k, v, qpos, kpos, qdoc, kdoc


@pytest.mark.parametrize("seed", range(6))
def test_forward_matches_brute_force(seed):
    rng = np.random.default_rng(seed)
    hkv = int(rng.integers(1, 3))
    hq = hkv * int(rng.integers(1, 4))
    d = int(rng.integers(1, 9))
    lq, lk = int(rng.integers(1, 20)), int(rng.integers(1, 24))
    causal = bool(seed % 2 == 0)
    docs = seed >= 3
    q, k, v, qpos, kpos, qdoc, kdoc = _case(rng, lq, lk, hq, hkv, d, docs)
    scale = 1.0 / math.sqrt(d)
    o, lse = A.forward(q, k, v, qpos, kpos, scale=scale, causal=causal,
                       qdoc=qdoc, kdoc=kdoc, block=5)
    ob, lb = brute_force(q, k, v, qpos, kpos, scale, causal, qdoc, kdoc)
    assert np.array_equal(np.isneginf(lse), np.isneginf(lb))
    fin = np.isfinite(lb)
    assert np.max(np.abs(lse[fin] - lb[fin]), initial=0) <= 1e-12
    assert np.max(np.abs(o - ob)) <= 1e-12


def test_rows_sum_to_one_and_weights_positive():
    rng = np.random.default_rng(7)
    q, k, v, qpos, kpos, qdoc, kdoc = _case(rng, 17, 23, 4, 2, 8, True)
    scale = 0.3
    _, lse = A.forward(q, k, v, qpos, kpos, scale=scale, causal=True, qdoc=qdoc, kdoc=kdoc)
    allow = A.allowed_mask(qpos, kpos, True, qdoc, kdoc)
    for h in range(4):
        g = h // 2
        for i in range(len(qpos)):
            js = np.nonzero(allow[i])[0]
            if len(js) == 0:
                assert np.isneginf(lse[h, i])
                continue
            w = [math.exp(scale * float(q[i, h] @ k[j, g]) - lse[h, i]) for j in js]
            assert abs(math.fsum(w) - 1.0) <= 1e-13


def test_constant_v_and_gradients_vanish():
    rng = np.random.default_rng(3)
    q, k, _, qpos, kpos, qdoc, kdoc = _case(rng, 12, 15, 2, 1, 6, False)
    c = rng.standard_normal(6)
    v = np.broadcast_to(c, (15, 1, 6)).copy()
    o, lse = A.forward(q, k, v, qpos, kpos, scale=0.5, causal=True)
    live = np.isfinite(lse[0])
    assert np.max(np.abs(o[live] - c)) <= 1e-13
    dout = rng.standard_normal(o.shape)
    dq, dk, dv = A.backward(q, k, v, dout, lse, A.delta(o, dout), qpos, kpos,
                            scale=0.5, causal=True)
    assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12


def test_golden_closed_forms():
    g = json.load(open(GOLDEN))
    t = g["two_keys"]
    q = np.array([[[_ev(t["q"][0])]]])
    k = np.array([[[_ev(x[0])]] for x in t["k"]])
    v = np.array([[[_ev(x[0])]] for x in t["v"]])
    qpos, kpos = np.array(t["qpos"]), np.array(t["kpos"])
    o, lse = A.forward(q, k, v, qpos, kpos, scale=_ev(t["scale"]), causal=True)
    assert abs(lse[0, 0] - _ev(t["lse"])) <= 1e-15
    assert abs(o[0, 0, 0] - _ev(t["o"][0])) <= 1e-14
    dout = np.array([[[_ev(t["dout"][0])]]])
    dq, dk, dv = A.backward(q, k, v, dout, lse, A.delta(o, dout), qpos, kpos,
                            scale=1.0, causal=True)
    assert abs(dq[0, 0, 0] - _ev(t["dq"][0])) <= 1e-14
    for j in range(2):
        assert abs(dk[j, 0, 0] - _ev(t["dk"][j][0])) <= 1e-14
        assert abs(dv[j, 0, 0] - _ev(t["dv"][j][0])) <= 1e-14

    m = g["merge_two_keys"]
    oa = np.array([[[_ev(m["oa"])]]])
    ob = np.array([[[_ev(m["ob"])]]])
    la, lb = np.array([[_ev(m["la"])]]), np.array([[_ev(m["lb"])]])
    om, lm = A.merge(oa, la, ob, lb)
    assert abs(lm[0, 0] - _ev(m["lse"])) <= 1e-15 and abs(om[0, 0, 0] - _ev(m["o"])) <= 1e-14
    oe, le = A.merge(oa, la, np.zeros_like(ob), np.array([[-np.inf]]))
    assert oe[0, 0, 0] == oa[0, 0, 0] and le[0, 0] == la[0, 0]

    z = g["zero_query"]
    pos = np.arange(4)
    vz = np.array([[[j, 1.0]] for j in range(4)])
    o, lse = A.forward(np.zeros((4, 1, 2)), rng_keys(4), vz, pos, pos, scale=0.7, causal=True)
    for i in range(4):
        assert abs(lse[0, i] - _ev(z["lse"][i])) <= 1e-15
        for e in range(2):
            assert abs(o[i, 0, e] - _ev(z["o"][i][e])) <= 1e-15


def rng_keys(n):
    return np.random.default_rng(99).standard_normal((n, 1, 2))


def test_single_allowed_key_closed_form():
    # first token of every document sees only itself: O = v, LSE = scale*q.k
    rng = np.random.default_rng(11)
    L, d = 10, 5
    q, k, v = (rng.standard_normal((L, 1, d)) for _ in range(3))
    pos = np.arange(L)
    doc = np.array([0, 0, 0, 1, 1, 2, 2, 2, 2, 3], dtype=np.int32)
    o, lse = A.forward(q, k, v, pos, pos, scale=0.4, causal=True, qdoc=doc, kdoc=doc)
    for i in (0, 3, 5, 9):
        assert np.max(np.abs(o[i, 0] - v[i, 0])) <= 1e-15
        assert abs(lse[0, i] - 0.4 * float(q[i, 0] @ k[i, 0])) <= 1e-14


def test_key_shift_invariance():
    rng = np.random.default_rng(5)
    q, k, v, qpos, kpos, _, _ = _case(rng, 9, 14, 2, 2, 4, False)
    c = rng.standard_normal(4)
    o1, l1 = A.forward(q, k, v, qpos, kpos, scale=0.6, causal=True)
    o2, l2 = A.forward(q, k + c, v, qpos, kpos, scale=0.6, causal=True)
    fin = np.isfinite(l1)
    shift = 0.6 * np.einsum("lhe,e->hl", q, c)
    assert np.max(np.abs((l2 - l1)[fin] - shift[fin])) <= 1e-12
    assert np.max(np.abs(o2 - o1)) <= 1e-12


@pytest.mark.parametrize("seed", range(4))
def test_merge_over_random_key_partitions(seed):
    rng = np.random.default_rng(100 + seed)
    q, k, v, qpos, kpos, qdoc, kdoc = _case(rng, 13, 29, 4, 2, 6, seed % 2 == 1)
    kw = dict(scale=0.35, causal=True)
    o, lse = A.forward(q, k, v, qpos, kpos, qdoc=qdoc, kdoc=kdoc, **kw)
    nparts = int(rng.integers(2, 6))
    label = rng.integers(0, nparts + 1, size=len(kpos))   # part nparts stays empty
    order = rng.permutation(nparts + 1)
    acc_o, acc_l = None, None
    for p in order:
        sel = label == p
        po, pl = A.forward(q, k[sel], v[sel], qpos, kpos[sel], qdoc=qdoc,
                           kdoc=None if kdoc is None else kdoc[sel], **kw)
        if acc_o is None:
            acc_o, acc_l = po, pl
        else:
            acc_o, acc_l = A.merge(acc_o, acc_l, po, pl)
    assert np.array_equal(np.isneginf(acc_l), np.isneginf(lse))
    fin = np.isfinite(lse)
    assert np.max(np.abs(acc_l[fin] - lse[fin])) <= 1e-12
    assert np.max(np.abs(acc_o - o)) <= 1e-12


def test_masks_entry_by_entry():
    rng = np.random.default_rng(21)
    _, _, _, qpos, kpos, qdoc, kdoc = _case(rng, 19, 27, 1, 1, 1, True)
    for causal in (False, True):
        for docs in (False, True):
            m = A.allowed_mask(qpos, kpos, causal, qdoc if docs else None, kdoc if docs else None)
            for i in range(len(qpos)):
                for j in range(len(kpos)):
                    want = (not causal or kpos[j] <= qpos[i]) and (not docs or qdoc[i] == kdoc[j])
                    assert m[i, j] == want


def test_packed_docs_equal_separate_documents():
    rng = np.random.default_rng(8)
    lens = [5, 1, 9, 3, 7]
    L = sum(lens)
    doc = np.repeat(np.arange(len(lens)), lens).astype(np.int32)
    q = rng.standard_normal((L, 4, 8))
    k = rng.standard_normal((L, 2, 8))
    v = rng.standard_normal((L, 2, 8))
    pos = np.arange(L)
    o, lse = A.forward(q, k, v, pos, pos, scale=0.35, causal=True, qdoc=doc, kdoc=doc)
    start = 0
    for n in lens:
        sl = slice(start, start + n)
        lp = np.arange(n)
        od, ld = A.forward(q[sl], k[sl], v[sl], lp, lp, scale=0.35, causal=True)
        assert np.max(np.abs(od - o[sl])) <= 1e-13
        assert np.max(np.abs(ld - lse[:, sl])) <= 1e-13
        start += n


def test_head_slice_equals_slice_of_full():
    rng = np.random.default_rng(12)
    q = rng.standard_normal((11, 8, 4))
    k = rng.standard_normal((11, 2, 4))
    v = rng.standard_normal((11, 2, 4))
    pos = np.arange(11)
    o, lse = A.forward(q, k, v, pos, pos, scale=0.5, causal=True)
    o2, l2 = A.forward(q[:, 4:8], k[:, 1:2], v[:, 1:2], pos, pos, scale=0.5, causal=True)
    assert np.max(np.abs(o2 - o[:, 4:8])) == 0 and np.max(np.abs(l2 - lse[4:8])) == 0


def _loss(q, k, v, dout, qpos, kpos, scale, qdoc, kdoc):
    o, _ = A.forward(q, k, v, qpos, kpos, scale=scale, causal=True, qdoc=qdoc, kdoc=kdoc)
    return float(np.sum(o * dout))


@pytest.mark.parametrize("seed", range(3))
def test_backward_matches_finite_differences(seed):
    rng = np.random.default_rng(40 + seed)
    q, k, v, qpos, kpos, qdoc, kdoc = _case(rng, 7, 9, 4, 2, 3, seed == 2)
    scale = 0.45
    o, lse = A.forward(q, k, v, qpos, kpos, scale=scale, causal=True, qdoc=qdoc, kdoc=kdoc)
    dout = rng.standard_normal(o.shape)
    dq, dk, dv = A.backward(q, k, v, dout, lse, A.delta(o, dout), qpos, kpos,
                            scale=scale, causal=True, qdoc=qdoc, kdoc=kdoc, block=3)
    eps = 1e-5
    for x, g in ((q, dq), (k, dk), (v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            old = x[idx]
            x[idx] = old + eps
            fp = _loss(q, k, v, dout, qpos, kpos, scale, qdoc, kdoc)
            x[idx] = old - eps
            fm = _loss(q, k, v, dout, qpos, kpos, scale, qdoc, kdoc)
            x[idx] = old
            num[idx] = (fp - fm) / (2 * eps)
        assert np.max(np.abs(num - g)) <= 1e-8


def test_gradient_sum_identities():
    rng = np.random.default_rng(77)
    q, k, v, qpos, kpos, _, _ = _case(rng, 16, 16, 4, 2, 5, False)
    kpos = np.arange(16)
    qpos = np.arange(16)
    o, lse = A.forward(q, k, v, qpos, kpos, scale=0.3, causal=True)
    dout = rng.standard_normal(o.shape)
    dq, dk, dv = A.backward(q, k, v, dout, lse, A.delta(o, dout), qpos, kpos,
                            scale=0.3, causal=True)
    # each row of dS sums to zero, so the key gradients cancel per KV head
    assert np.max(np.abs(dk.sum(axis=0))) <= 1e-12
    # each row of P sums to one, so dV summed over keys is dO summed over the group
    want = np.stack([dout[:, 2 * g:2 * g + 2].sum(axis=(0, 1)) for g in range(2)])
    assert np.max(np.abs(dv.sum(axis=0) - want)) <= 1e-12


def test_sampled_rows_and_keys_match_full():
    rng = np.random.default_rng(31)
    q, k, v, qpos, kpos, qdoc, kdoc = _case(rng, 20, 20, 4, 2, 6, True)
    kw = dict(scale=0.4, causal=True, qdoc=qdoc, kdoc=kdoc)
    o, lse = A.forward(q, k, v, qpos, kpos, **kw)
    dout = rng.standard_normal(o.shape)
    dlt = A.delta(o, dout)
    dq, dk, dv = A.backward(q, k, v, dout, lse, dlt, qpos, kpos, **kw)
    rows = rng.integers(0, 20, size=12)
    heads = rng.integers(0, 4, size=12)
    so, sl = A.forward_rows(q, k, v, qpos, kpos, rows, heads, **kw)
    assert np.max(np.abs(so - o[rows, heads])) <= 1e-13
    fin = np.isfinite(sl)
    assert np.array_equal(fin, np.isfinite(lse[heads, rows]))
    assert np.max(np.abs(sl[fin] - lse[heads, rows][fin]), initial=0) <= 1e-13
    sdq = A.dq_rows(q, k, v, dout, lse[heads, rows], dlt[heads, rows], qpos, kpos,
                    rows, heads, **kw)
    assert np.max(np.abs(sdq - dq[rows, heads])) <= 1e-13
    keys = rng.integers(0, 20, size=10)
    kvh = rng.integers(0, 2, size=10)
    sdk, sdv = A.dkv_keys(q, k, v, dout, lse, dlt, qpos, kpos, keys, kvh, **kw)
    assert np.max(np.abs(sdk - dk[keys, kvh])) <= 1e-13
    assert np.max(np.abs(sdv - dv[keys, kvh])) <= 1e-13


def test_tile_classes_definition():
    rng = np.random.default_rng(4)
    _, _, _, qpos, kpos, qdoc, kdoc = _case(rng, 37, 41, 1, 1, 1, True)
    cls = A.tile_classes(qpos, kpos, True, 8, 16, qdoc, kdoc)
    allow = A.allowed_mask(qpos, kpos, True, qdoc, kdoc)
    assert cls.shape == (5, 3)
    for a in range(5):
        for b in range(3):
            blk = allow[a * 8:(a + 1) * 8, b * 16:(b + 1) * 16]
            assert (cls[a, b] == 0) == (not blk.any())
            assert (cls[a, b] == 1) == bool(blk.all())


def test_planted_mistakes_are_caught(monkeypatch):
    """A dropped term, a wrong sign or a transposed operand in the oracle must
    fail the pins above; plant each one and check that brute force disagrees."""
    rng = np.random.default_rng(1)
    q, k, v, qpos, kpos, _, _ = _case(rng, 8, 8, 2, 1, 3, False)
    ob, lb = brute_force(q, k, v, qpos, kpos, 0.5, True)

    def bad_mask(qp, kp, causal, qd=None, kd=None):   # strict causal (diagonal dropped)
        m = np.asarray(kp)[None, :] < np.asarray(qp)[:, None]
        return m
    monkeypatch.setattr(A, "allowed_mask", bad_mask)
    o, lse = A.forward(q, k, v, qpos, kpos, scale=0.5, causal=True)
    monkeypatch.undo()
    assert np.max(np.abs(np.nan_to_num(o - ob))) > 1e-6 or not np.array_equal(np.isinf(lse), np.isinf(lb))

    # wrong merge weight (uses La for both partials)
    def bad_merge(oa, la, ob_, lb_):
        m = np.maximum(la, lb_)
        L = m + np.log(np.exp(la - m) + np.exp(lb_ - m))
        w = np.exp(la - L).T[:, :, None]
        return w * oa + w * ob_, L
    o1, l1 = A.forward(q, k[:4], v[:4], qpos, kpos[:4], scale=0.5, causal=True)
    o2, l2 = A.forward(q, k[4:], v[4:], qpos, kpos[4:], scale=0.5, causal=True)
    fin = np.isfinite(l1) & np.isfinite(l2)
    bo, _ = bad_merge(o1, l1, o2, l2)
    assert np.max(np.abs((bo - ob)[fin.T])) > 1e-6

    # interleaved GQA head map (h mod Hkv) instead of contiguous groups
    q2, k2, v2, qp2, kp2, _, _ = _case(rng, 6, 6, 4, 2, 3, False)
    ob2, _ = brute_force(q2, k2, v2, qp2, kp2, 0.5, True)
    monkeypatch.setattr(A, "kv_head", lambda h, hq, hkv: h % hkv)
    o2b, _ = A.forward(q2, k2, v2, qp2, kp2, scale=0.5, causal=True)
    monkeypatch.undo()
    assert np.max(np.abs(o2b - ob2)) > 1e-6

    # wrong sign of Delta (dS = P (dP + Delta)): the gradient leaves the
    # finite-difference value
    o3, l3 = A.forward(q, k, v, qpos, kpos, scale=0.5, causal=True)
    dout = rng.standard_normal(o3.shape)
    good = A.delta(o3, dout)
    dq_bad, _, _ = A.backward(q, k, v, dout, l3, -good, qpos, kpos, scale=0.5, causal=True)
    eps, idx = 1e-5, (3, 1, 2)
    old = q[idx]
    q[idx] = old + eps
    fp = _loss(q, k, v, dout, qpos, kpos, 0.5, None, None)
    q[idx] = old - eps
    fm = _loss(q, k, v, dout, qpos, kpos, 0.5, None, None)
    q[idx] = old
    dq_good, _, _ = A.backward(q, k, v, dout, l3, good, qpos, kpos, scale=0.5, causal=True)
    num = (fp - fm) / (2 * eps)
    assert abs(dq_good[idx] - num) <= 1e-8
    assert abs(dq_bad[idx] - num) > 1e-6
