"""Pins of the oracle's zigzag sharding, ring schedule and ring / Ulysses / USP
emulations: hand-derived literals, brute-force counts, and equality with the
unsharded definition."""
import json
import os

import numpy as np
import pytest

from oracle import attention as A
from oracle import schedule as Z

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")


def test_zigzag_golden_S16_P2():
    g = json.load(open(GOLDEN))["zigzag_S16_P2"]
    for r in (0, 1):
        (p0, p1), (l0, l1) = Z.zigzag_layout(16, 2, r)
        assert [[p0, p1], [l0, l1]] == g["layout"][str(r)]
        for s in (0, 1):
            src, kinds = Z.ring_schedule(16, 2, r, s)
            assert [src, kinds] == g["schedule"][f"{r},{s}"]
            pairs = Z.causal_pairs(Z.rank_positions(16, 2, r),
                                   Z.rank_positions(16, 2, src))
            assert pairs == g["pairs"][f"{r},{s}"]


@pytest.mark.parametrize("S,P", [(8, 1), (16, 2), (48, 3), (64, 4), (128, 8), (96, 6)])
def test_zigzag_partition_and_balance(S, P):
    c = S // (2 * P)
    allpos = np.concatenate([Z.rank_positions(S, P, r) for r in range(P)])
    assert np.array_equal(np.sort(allpos), np.arange(S))
    assert np.array_equal(Z.sharded_order(S, P), allpos)
    total = 0
    for r in range(P):
        qp = Z.rank_positions(S, P, r)
        seen = set()
        for s in range(P):
            src, kinds = Z.ring_schedule(S, P, r, s)
            seen.add(src)
            kp = Z.rank_positions(S, P, src)
            n = Z.causal_pairs(qp, kp)          # brute-force count
            assert n == 2 * c * c + (c if s == 0 else 0)
            total += n
            # kinds agree with the explicit mask at chunk granularity
            allow = A.allowed_mask(qp, kp, True)
            for a in range(2):
                for b in range(2):
                    blk = allow[a * c:(a + 1) * c, b * c:(b + 1) * c]
                    want = Z.SKIP if not blk.any() else (Z.FULL if blk.all() else Z.DIAG)
                    assert kinds[a * 2 + b] == want
        assert seen == set(range(P))
    assert total == S * (S + 1) // 2


def test_zigzag_rejects_bad_sizes():
    for args in ((10, 3, 0), (16, 2, 2), (16, 0, 0), (16, 2, -1)):
        with pytest.raises(ValueError):
            Z.zigzag_layout(*args)


def _global_to_sharded(x, S, P):
    return x[Z.sharded_order(S, P)]


@pytest.mark.parametrize("S,P,docs", [(32, 2, False), (48, 3, True), (64, 4, False), (64, 4, True)])
def test_ring_forward_equals_full_attention(S, P, docs):
    rng = np.random.default_rng(S + P)
    q = rng.standard_normal((S, 4, 8))
    k = rng.standard_normal((S, 2, 8))
    v = rng.standard_normal((S, 2, 8))
    doc = np.repeat(np.arange(4), [5, S // 2 - 5, 3, S // 2 - 3]).astype(np.int32) if docs else None
    pos = np.arange(S)
    o, lse = A.forward(q, k, v, pos, pos, scale=0.35, causal=True, qdoc=doc, kdoc=doc)
    order = Z.sharded_order(S, P)
    qs, ks, vs = q[order], k[order], v[order]
    ds = None if doc is None else doc[order]
    c2 = S // P
    for r in range(P):
        ro, rl, steps = Z.ring_forward(qs, ks, vs, S, P, r, scale=0.35, doc=ds)
        rows = order[r * c2:(r + 1) * c2]
        assert np.max(np.abs(ro - o[rows])) <= 1e-12
        assert np.max(np.abs(rl - lse[:, rows])) <= 1e-12
        assert len(steps) == P
        # each step's partial is the attention over exactly that step's keys
        for s, (po, pl) in enumerate(steps):
            j = Z.ring_source(P, r, s)
            kp = Z.rank_positions(S, P, j)
            eo, el = A.forward(q[rows], k[kp], v[kp], rows, kp, scale=0.35, causal=True,
                               qdoc=None if doc is None else doc[rows],
                               kdoc=None if doc is None else doc[kp])
            assert np.max(np.abs(po - eo)) <= 1e-13
            assert np.array_equal(np.isneginf(pl), np.isneginf(el))


def test_ring_backward_sums_to_full_gradient():
    S, P = 48, 3
    rng = np.random.default_rng(9)
    q = rng.standard_normal((S, 4, 6))
    k = rng.standard_normal((S, 2, 6))
    v = rng.standard_normal((S, 2, 6))
    dout = rng.standard_normal((S, 4, 6))
    pos = np.arange(S)
    o, lse = A.forward(q, k, v, pos, pos, scale=0.4, causal=True)
    dq, dk, dv = A.backward(q, k, v, dout, lse, A.delta(o, dout), pos, pos, scale=0.4, causal=True)
    order = Z.sharded_order(S, P)
    qs, ks, vs, dos = q[order], k[order], v[order], dout[order]
    c2 = S // P
    dk_sum = np.zeros_like(dk)
    dv_sum = np.zeros_like(dv)
    for r in range(P):
        ro, rl, _ = Z.ring_forward(qs, ks, vs, S, P, r, scale=0.4)
        gq, gk, gv = Z.ring_backward(qs, ks, vs, dos[r * c2:(r + 1) * c2], ro, rl, S, P, r, scale=0.4)
        assert np.max(np.abs(gq - dq[order[r * c2:(r + 1) * c2]])) <= 1e-12
        dk_sum += gk
        dv_sum += gv
    assert np.max(np.abs(dk_sum - dk[order])) <= 1e-12
    assert np.max(np.abs(dv_sum - dv[order])) <= 1e-12


def test_ulysses_and_usp_shares_equal_slices_of_full():
    S = 32
    rng = np.random.default_rng(13)
    q = rng.standard_normal((S, 8, 4))
    k = rng.standard_normal((S, 4, 4))
    v = rng.standard_normal((S, 4, 4))
    pos = np.arange(S)
    o, lse = A.forward(q, k, v, pos, pos, scale=0.5, causal=True)
    for sp in (1, 2, 4):
        for r in range(sp):
            so, sl = Z.ulysses_share(q, k, v, sp, r, scale=0.5)
            (h0, h1), _ = Z.head_slice(8, 4, sp, r)
            assert np.max(np.abs(so - o[:, h0:h1])) <= 1e-13
            assert np.max(np.abs(sl - lse[h0:h1])) <= 1e-13
    with pytest.raises(ValueError):
        Z.head_slice(8, 4, 8, 0)       # KV heads bound the Ulysses degree
    # USP: Ulysses 2 x ring 2 -> a head slice run through the ring
    (h0, h1), (g0, g1) = Z.head_slice(8, 4, 2, 1)
    order = Z.sharded_order(S, 2)
    for r in range(2):
        ro, rl, _ = Z.ring_forward(q[order][:, h0:h1], k[order][:, g0:g1], v[order][:, g0:g1],
                                   S, 2, r, scale=0.5)
        rows = order[r * 16:(r + 1) * 16]
        assert np.max(np.abs(ro - o[rows][:, h0:h1])) <= 1e-12


def test_dropped_or_misordered_ring_step_is_caught():
    """Planted mistakes in the emulation: dropping a step or merging a step's
    partial with another step's LSE must break equality with full attention."""
    S, P = 32, 2
    rng = np.random.default_rng(2)
    q = rng.standard_normal((S, 2, 4))
    k = rng.standard_normal((S, 1, 4))
    v = rng.standard_normal((S, 1, 4))
    pos = np.arange(S)
    o, lse = A.forward(q, k, v, pos, pos, scale=0.5, causal=True)
    order = Z.sharded_order(S, P)
    r = 1
    _, _, steps = Z.ring_forward(q[order], k[order], v[order], S, P, r, scale=0.5)
    rows = order[r * 16:(r + 1) * 16]
    (o0, l0), (o1, l1) = steps
    assert np.max(np.abs(o0 - o[rows])) > 1e-3                       # step dropped
    bo, _ = A.merge(o0, l1, o1, l0)                                   # LSEs swapped
    assert np.max(np.abs(bo - o[rows])) > 1e-3
    go, _ = A.merge(o0, l0, o1, l1)
    assert np.max(np.abs(go - o[rows])) <= 1e-12


def test_a2a_golden_and_round_trip():
    """The all-to-all on labelled integers: element (token, head) carries
    100*token + head, so every message is checkable by eye; the reverse
    exchange of the forward result is the identity."""
    S, h, sp, d = 8, 4, 2, 1
    full = np.array([[[100 * t + hd] for hd in range(h)] for t in range(S)])
    shards = [full[j * S // sp:(j + 1) * S // sp] for j in range(sp)]
    y1 = Z.a2a_tokens_to_heads(shards, 1)
    assert y1.shape == (S, 2, 1)
    assert y1[:, :, 0].tolist() == [[100 * t + 2, 100 * t + 3] for t in range(S)]
    outs = [Z.a2a_tokens_to_heads(shards, r) for r in range(sp)]
    for j in range(sp):
        assert np.array_equal(Z.a2a_heads_to_tokens(outs, j), shards[j])


def test_a2a_kv_replication_when_ranks_exceed_heads():
    S, h, sp = 16, 2, 8
    rng = np.random.default_rng(4)
    full = rng.standard_normal((S, h, 3))
    shards = np.split(full, sp)
    ys = [Z.a2a_tokens_to_heads(shards, r) for r in range(sp)]
    for r in range(sp):
        assert ys[r].shape == (S, 1, 3)
        # the KV head that rank r's query heads read (contiguous GQA groups)
        hq = 32
        q_heads = range(r * hq // sp, (r + 1) * hq // sp)
        kv = {A.kv_head(qh, hq, h) for qh in q_heads}
        assert kv == {r * h // sp}
        assert np.array_equal(ys[r][:, 0], full[:, r * h // sp])
    with pytest.raises(ValueError):
        Z.a2a_heads_of_rank(3, 2, 0)


def test_a2a_result_is_the_ulysses_head_slice():
    S, hq, hkv, d, sp = 12, 8, 4, 2, 4
    rng = np.random.default_rng(5)
    q = rng.standard_normal((S, hq, d))
    qs = np.split(q, sp)
    for r in range(sp):
        (a, b), _ = Z.head_slice(hq, hkv, sp, r)
        assert np.array_equal(Z.a2a_tokens_to_heads(qs, r), q[:, a:b])


def test_allgather_shares_sum_to_full_attention():
    """Every rank's all-gather share equals the full attention on its rows, and
    the ranks' dK/dV contributions sum to the full gradient."""
    S, P, hq, hkv, d = 48, 3, 4, 2, 3
    rng = np.random.default_rng(21)
    q = rng.standard_normal((S, hq, d))
    k = rng.standard_normal((S, hkv, d))
    v = rng.standard_normal((S, hkv, d))
    do = rng.standard_normal((S, hq, d))
    doc = np.repeat(np.arange(4), 12).astype(np.int32)
    pos = np.arange(S)
    o, lse = A.forward(q, k, v, pos, pos, scale=0.5, causal=True, qdoc=doc, kdoc=doc)
    dq, dk, dv = A.backward(q, k, v, do, lse, A.delta(o, do), pos, pos, scale=0.5, causal=True, qdoc=doc, kdoc=doc)
    dk_sum = np.zeros_like(dk)
    dv_sum = np.zeros_like(dv)
    for r in range(P):
        rows = Z.rank_positions(S, P, r)
        ro, rl, rdq, rdk, rdv = Z.allgather_share(q[rows], k, v, S, P, r, scale=0.5, doc=doc, dout=do[rows])
        assert np.max(np.abs(ro - o[rows])) <= 1e-12
        assert np.max(np.abs(rl - lse[:, rows])) <= 1e-12
        assert np.max(np.abs(rdq - dq[rows])) <= 1e-12
        dk_sum += rdk
        dv_sum += rdv
    assert np.max(np.abs(dk_sum - dk)) <= 1e-12 and np.max(np.abs(dv_sum - dv)) <= 1e-12
