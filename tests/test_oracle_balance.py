"""Pins of the oracle's work-balancing and tile-classification functions
(oracle.schedule.chunk_work, oracle.schedule.best_pairing,
oracle.attention.tile_classes) against facts the mathematics fixes, not
against the library: closed-form pair counts, hand-solved pairings with their
lower bounds (tests/golden/closed_forms.json), brute force on tiny inputs,
and planted mistakes that each pin must catch.

Source of the balancing rule: siliconandsystems.com, "Llama 3 parallelism",
section "긴 문맥은 어텐션 비용 이상을 바꾸는 방식" (ranks are balanced by the
attention work they do, not by their token count)."""
import itertools
import json
import os

import numpy as np
import pytest

import cpinputs
from oracle import attention as A
from oracle import schedule as Z

GOLDEN = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "closed_forms.json")))


def _doc_layouts():
    rng = np.random.default_rng(77)
    out = []
    for S, P in ((64, 2), (96, 3), (256, 4), (480, 5)):
        for k in range(3):
            lens = cpinputs.lognormal_doc_lengths(S, seed=int(rng.integers(1 << 30)), median=max(2, S // 7),
                                                  sigma=1.0, lo=1, hi=S)
            out.append((S, P, cpinputs.doc_ids_from_lengths(lens), lens))
    return out


# ---- chunk_work -------------------------------------------------------------

@pytest.mark.parametrize("S,P", [(8, 2), (64, 1), (96, 3), (1024, 8)])
def test_chunk_work_causal_closed_form(S, P):
    """No documents: chunk i has i*c^2 + c(c+1)/2 pairs; all chunks S(S+1)/2."""
    c = S // (2 * P)
    w = Z.chunk_work(S, P)
    want = np.array([i * c * c + c * (c + 1) // 2 for i in range(2 * P)])
    assert np.array_equal(w, want)
    assert int(w.sum()) == S * (S + 1) // 2


@pytest.mark.parametrize("S,P,doc,lens", _doc_layouts())
def test_chunk_work_documents_closed_form(S, P, doc, lens):
    """With documents: the total is sum_k L_k(L_k+1)/2, and each chunk's share
    is the sum over its queries of (position - start of its document + 1)."""
    w = Z.chunk_work(S, P, doc)
    assert int(w.sum()) == int(sum(int(L) * (int(L) + 1) // 2 for L in lens))
    starts = np.concatenate([[0], np.cumsum(lens)[:-1]])          # first position of each document
    pos = np.arange(S)
    keys_of = pos - starts[doc] + 1                                # keys each query may see
    c = S // (2 * P)
    assert np.array_equal(w, keys_of.reshape(2 * P, c).sum(axis=1))


def test_chunk_work_golden():
    g = GOLDEN["chunk_work"]
    assert Z.chunk_work(g["S"], g["P"], np.array(g["doc"], dtype=np.int32)).tolist() == g["work"]
    assert Z.chunk_work(g["S"], g["P"]).tolist() == g["no_docs_S8_P2"]


def test_chunk_work_planted_mistakes_are_caught(monkeypatch):
    """A strict causal mask (diagonal dropped) and an off-by-one chunk
    boundary each break the closed forms above."""
    S, P = 96, 3

    def strict(qp, kp, causal, qd=None, kd=None):
        m = np.asarray(kp)[None, :] < np.asarray(qp)[:, None]
        if qd is not None:
            m &= np.asarray(kd)[None, :] == np.asarray(qd)[:, None]
        return m
    monkeypatch.setattr(A, "allowed_mask", strict)
    bad = Z.chunk_work(S, P)
    monkeypatch.undo()
    assert int(bad.sum()) != S * (S + 1) // 2

    def shifted_chunk_work(S, P):           # chunk i taken as queries [i*c + 1, (i+1)*c + 1)
        c = S // (2 * P)
        pos = np.arange(S + 1)
        return np.array([int(A.allowed_mask(pos[i * c + 1:(i + 1) * c + 1], pos, True).sum())
                         for i in range(2 * P)])
    c = S // (2 * P)
    want = np.array([i * c * c + c * (c + 1) // 2 for i in range(2 * P)])
    assert not np.array_equal(shifted_chunk_work(S, P), want)


# ---- best_pairing -----------------------------------------------------------

def _brute_min_max(work):
    """Every perfect matching of the chunks into pairs, by enumeration of
    permutations (tiny inputs only)."""
    n = len(work)
    best = None
    for perm in itertools.permutations(range(n)):
        worst = max(work[perm[2 * i]] + work[perm[2 * i + 1]] for i in range(n // 2))
        best = worst if best is None else min(best, worst)
    return best


def test_best_pairing_golden():
    for case in GOLDEN["best_pairing"]["cases"]:
        w = case["work"]
        assert Z.best_pairing(w) == case["min_max"], case
        # the optimum respects both lower bounds of the derivation
        assert case["min_max"] >= -(-sum(w) // (len(w) // 2))
        assert case["min_max"] >= max(w) + min(w)


@pytest.mark.parametrize("seed", range(6))
def test_best_pairing_matches_enumeration(seed):
    rng = np.random.default_rng(seed)
    n = 2 * int(rng.integers(1, 5))           # 2..8 chunks
    w = [int(x) for x in rng.integers(0, 50, size=n)]
    assert Z.best_pairing(w) == _brute_min_max(w)


def test_best_pairing_planted_mistake_is_caught():
    """Pairing neighbours in sorted order is a plausible wrong rule; it fails
    the hand-solved golden."""
    def neighbours(work):
        s = sorted(work)
        return max(s[i] + s[i + 1] for i in range(0, len(s), 2))
    cases = GOLDEN["best_pairing"]["cases"]
    assert any(neighbours(c["work"]) != c["min_max"] for c in cases)


def test_zigzag_pairing_is_optimal_without_documents():
    """Without documents the chunk works grow linearly, so pairing chunk r with
    2P-1-r gives every rank the same sum, which meets the total/P bound."""
    for S, P in ((64, 2), (96, 3), (128, 4)):
        w = Z.chunk_work(S, P)
        zz = [int(w[r] + w[2 * P - 1 - r]) for r in range(P)]
        assert min(zz) == max(zz) == Z.best_pairing(w) == S * (S + 1) // 2 // P


# ---- pair_layout / rank_positions with an explicit assignment ---------------

def test_pair_layout_positions_and_errors():
    S, P = 24, 3
    chunks = [(0, 1), (2, 5), (3, 4)]
    assert Z.rank_positions(S, P, 1, chunks).tolist() == list(range(8, 12)) + list(range(20, 24))
    order = Z.sharded_order(S, P, chunks)
    assert sorted(order.tolist()) == list(range(S))
    zz = [(r, 2 * P - 1 - r) for r in range(P)]
    assert np.array_equal(Z.sharded_order(S, P, zz), Z.sharded_order(S, P))
    for bad in ([(0, 1), (2, 3)], [(0, 1), (1, 2), (3, 4)], [(1, 0), (2, 5), (3, 4)]):
        with pytest.raises(ValueError):
            Z.rank_positions(S, P, 0, bad)


# ---- tile_classes ------------------------------------------------------------

def test_tile_classes_golden():
    g = GOLDEN["tile_classes"]
    pos = np.arange(g["S"])
    assert A.tile_classes(pos, pos, True, g["bq"], g["bk"]).tolist() == g["causal"]
    doc = np.repeat(np.arange(2), g["S"] // 2).astype(np.int32)
    assert A.tile_classes(pos, pos, True, g["bq"], g["bk"], doc, doc).tolist() == g["causal_two_docs"]


def test_tile_classes_unit_tiles_are_the_mask():
    """With 1 x 1 tiles every tile is one entry: 1 where allowed, 0 where not."""
    rng = np.random.default_rng(9)
    qpos = np.sort(rng.choice(40, size=13, replace=False))
    kpos = np.sort(rng.choice(40, size=11, replace=False))
    qd, kd = (np.searchsorted([10, 25], p, side="right").astype(np.int32) for p in (qpos, kpos))
    cls = A.tile_classes(qpos, kpos, True, 1, 1, qd, kd)
    manual = np.array([[int(kp <= qp and a == b) for kp, b in zip(kpos, kd)] for qp, a in zip(qpos, qd)])
    assert np.array_equal(cls, manual)


def test_tile_classes_count_closed_form():
    """Aligned causal square of n x n tiles of B: n(n-1)/2 skipped, n(n-1)/2
    full, n partial (the diagonal)."""
    for n, B in ((5, 4), (8, 2), (3, 7)):
        pos = np.arange(n * B)
        cls = A.tile_classes(pos, pos, True, B, B)
        assert (cls == 0).sum() == n * (n - 1) // 2
        assert (cls == 1).sum() == n * (n - 1) // 2
        assert (cls == 2).sum() == n
