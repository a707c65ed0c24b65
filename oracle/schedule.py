"""Oracle for the context-parallel schedules: zigzag sharding, the ring's
per-step block kinds, and emulations of the ring (P2P), Ulysses (A2A) and USP
shares built only from ``oracle.attention``.

TEST INFRASTRUCTURE ONLY: imported by the test suite, the smoke check and the
benchmark's CPU-baseline leg; never by the library.

Sources:

* nougat.kr, "MaxText long-context training: KV parallelism", diagram text
  (sequence split; All-gather; A2A; P2P) and section "헤드를 나누거나, KV를
  돌리거나" (split the heads, or rotate the KV): the sequence is split by
  tokens; a ring rank keeps its own KV chunk and one visiting chunk, computes
  a partial result, merges it and receives the next chunk; later tokens see
  more context, so the causal work must be balanced across ranks; A2A turns
  the token split into a head split; USP combines an A2A group with a ring.
* siliconandsystems.com, "Llama 3 parallelism", section "긴 문맥은 어텐션 비용
  이상을 바꾸는 방식" (long context changes more than the attention cost): work
  is to be balanced by actual attention compute.

The balancing scheme itself is not spelled out on the pages.  The reading used
here ("zigzag"): cut the S tokens into 2P equal chunks; rank r holds chunks r
and 2P-1-r; ring step s brings rank (r - s) mod P's KV.  S must be a multiple
of 2P.  Arrays in "sharded order" concatenate the ranks' local shards:
rank 0's two chunks, then rank 1's, and so on.
"""
from __future__ import annotations

import numpy as np

from . import attention as A

SKIP, DIAG, FULL = 0, 1, 2


def zigzag_layout(S, P, r):
    """Global start and length of rank r's two chunks: ((r*c, (2P-1-r)*c), (c, c))."""
    if P < 1 or S < 1 or S % (2 * P) != 0 or not 0 <= r < P:
        raise ValueError("need P >= 1, S > 0 divisible by 2P and 0 <= r < P")
    c = S // (2 * P)
    return (r * c, (2 * P - 1 - r) * c), (c, c)


def pair_layout(S, P, r, chunks):
    """Rank r's two chunks under an explicit two-chunks-per-rank assignment:
    chunks[r] = (a, b) with a < b, every chunk 0..2P-1 used once.  Same
    return form as zigzag_layout."""
    if P < 1 or S < 1 or S % (2 * P) != 0 or not 0 <= r < P:
        raise ValueError("need P >= 1, S > 0 divisible by 2P and 0 <= r < P")
    flat = sorted(int(x) for pair in chunks for x in pair)
    if len(chunks) != P or flat != list(range(2 * P)):
        raise ValueError("chunks must give each of the P ranks two of the 2P chunks, each chunk once")
    a, b = (int(x) for x in chunks[r])
    if not a < b:
        raise ValueError("a rank's chunks must be in increasing order")
    c = S // (2 * P)
    return (a * c, b * c), (c, c)


def rank_positions(S, P, r, chunks=None):
    """Global positions of rank r's local tokens, in local order (zigzag, or
    the assignment ``chunks`` of pair_layout)."""
    lay = zigzag_layout(S, P, r) if chunks is None else pair_layout(S, P, r, chunks)
    (p0, p1), (l0, l1) = lay
    return np.concatenate([np.arange(p0, p0 + l0), np.arange(p1, p1 + l1)])


def sharded_order(S, P, chunks=None):
    """Global position of each row of a sharded-order array."""
    return np.concatenate([rank_positions(S, P, r, chunks) for r in range(P)])


def ring_source(P, r, s):
    """Rank whose KV chunk rank r holds at ring step s (neighbour passing)."""
    return (r - s) % P


def ring_schedule(S, P, r, s):
    """(source rank, kinds[4]) for rank r at step s.

    kinds[a*2 + b] classifies local Q chunk a of rank r against local KV chunk
    b of the source rank at chunk granularity under the causal mask: SKIP if
    the KV chunk lies after the Q chunk, DIAG if it is the same chunk, FULL if
    it lies before.
    """
    zigzag_layout(S, P, r)
    src = ring_source(P, r, s)
    qchunks = (r, 2 * P - 1 - r)
    kchunks = (src, 2 * P - 1 - src)
    kinds = []
    for a in range(2):
        for b in range(2):
            if kchunks[b] > qchunks[a]:
                kinds.append(SKIP)
            elif kchunks[b] == qchunks[a]:
                kinds.append(DIAG)
            else:
                kinds.append(FULL)
    return src, kinds


def causal_pairs(qpos, kpos):
    """Number of (query, key) pairs with key position <= query position."""
    return int(A.allowed_mask(qpos, kpos, True).sum())


def _shard(x, S, P, r):
    c2 = S // P
    return x[r * c2:(r + 1) * c2]


def ring_forward(q, k, v, S, P, r, *, scale, causal=True, doc=None, chunks=None):
    """Rank r's forward under the ring, all inputs in sharded order (of the
    zigzag layout, or of the assignment ``chunks``, see pair_layout).

    At each step the rank's Q shard attends to the visiting KV shard (every
    mask entry evaluated on global positions), and the partial (O, LSE) is
    merged into the running result.  Returns (o, lse, steps) where steps is the
    list of per-step partials (o_s, lse_s).
    """
    qpos = rank_positions(S, P, r, chunks)
    qd = None if doc is None else _shard(doc, S, P, r)
    qs = _shard(q, S, P, r)
    o = lse = None
    steps = []
    for s in range(P):
        j = ring_source(P, r, s)
        kpos = rank_positions(S, P, j, chunks)
        kd = None if doc is None else _shard(doc, S, P, j)
        po, pl = A.forward(qs, _shard(k, S, P, j), _shard(v, S, P, j), qpos, kpos,
                           scale=scale, causal=causal, qdoc=qd, kdoc=kd)
        steps.append((po, pl))
        if o is None:
            o, lse = po, pl
        else:
            o, lse = A.merge(o, lse, po, pl)
    return o, lse, steps


def ring_backward(q, k, v, dout, o, lse, S, P, r, *, scale, causal=True, doc=None, chunks=None):
    """Rank r's backward under the ring (sharded order; ``chunks`` as in
    ring_forward).

    Delta comes from the rank's final O; each step's chunk backward uses the
    final LSE.  Returns (dq of the rank's rows, dk, dv over all S rows) where
    dk/dv hold only this rank's query rows' contributions, each in the
    visiting rank's slot: what a ring carries back to each KV owner.
    """
    qpos = rank_positions(S, P, r, chunks)
    qd = None if doc is None else _shard(doc, S, P, r)
    qs = _shard(q, S, P, r)
    dlt = A.delta(o, dout)
    dq = np.zeros(qs.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    c2 = S // P
    for s in range(P):
        j = ring_source(P, r, s)
        kd = None if doc is None else _shard(doc, S, P, j)
        gq, gk, gv = A.backward(qs, _shard(k, S, P, j), _shard(v, S, P, j), dout,
                                lse, dlt, qpos, rank_positions(S, P, j, chunks),
                                scale=scale, causal=causal, qdoc=qd, kdoc=kd)
        dq += gq
        dk[j * c2:(j + 1) * c2] += gk
        dv[j * c2:(j + 1) * c2] += gv
    return dq, dk, dv


def head_slice(hq, hkv, sp, rank):
    """Query and KV head ranges of Ulysses rank ``rank`` out of ``sp``: the
    all-to-all hands each rank a contiguous slice of heads for the whole
    sequence (nougat.kr MaxText page, A2A diagram text)."""
    if hq % sp or hkv % sp:
        raise ValueError("sp must divide both the query and the KV head counts")
    a, b = hq // sp, hkv // sp
    return (rank * a, (rank + 1) * a), (rank * b, (rank + 1) * b)


def ulysses_share(q, k, v, sp, rank, *, scale, causal=True, doc=None):
    """Ulysses rank's share: full-sequence attention for its head slice.
    q [S, Hq, d], k/v [S, Hkv, d] in global order (the layer's full heads)."""
    (h0, h1), (g0, g1) = head_slice(q.shape[1], k.shape[1], sp, rank)
    pos = np.arange(q.shape[0])
    return A.forward(q[:, h0:h1], k[:, g0:g1], v[:, g0:g1], pos, pos,
                     scale=scale, causal=causal, qdoc=doc, kdoc=doc)


# ---- the Ulysses all-to-all exchange ---------------------------------------
# [Ulysses] section 현황 and [MaxText] diagram text (A2A): before attention
# each rank holds a token shard of every head; the all-to-all gives each rank
# every token of its own heads; after attention the reverse exchange returns
# each rank its tokens of every head.  Written as the messages the ranks send
# each other.

def a2a_heads_of_rank(h, sp, rank):
    """Heads rank `rank` holds after the forward exchange: its slice of h/sp
    heads, or -- with more ranks than heads (KV heads under GQA) -- the one
    head its query heads read, shared with the other sp/h ranks."""
    if h % sp == 0:
        return list(range(rank * (h // sp), (rank + 1) * (h // sp)))
    if sp % h == 0:
        return [rank * h // sp]
    raise ValueError(f"h={h} and sp={sp}: one must divide the other")


def a2a_tokens_to_heads(shards, rank):
    """Forward exchange seen by `rank`: rank j sends it the heads of its slice
    from j's token shard; `rank` stacks the messages in sender order.
    shards: list of sp arrays [S/sp, h, d]; returns [S, len(heads), d]."""
    sp = len(shards)
    heads = a2a_heads_of_rank(shards[0].shape[1], sp, rank)
    messages = [np.asarray(shards[j])[:, heads, :] for j in range(sp)]
    return np.concatenate(messages, axis=0)


def a2a_heads_to_tokens(outputs, j):
    """Reverse exchange seen by rank j: rank r sends it j's tokens of r's
    head-split output; j places them at r's heads.  outputs: list of sp
    arrays [S, h/sp, d]; returns j's shard [S/sp, h, d]."""
    sp = len(outputs)
    n = outputs[0].shape[0] // sp
    return np.concatenate([np.asarray(outputs[r])[j * n:(j + 1) * n] for r in range(sp)], axis=1)


# ---- balancing ranks by attention work -------------------------------------
# [Llama3] section 긴 문맥은 어텐션 비용 이상을 바꾸는 방식: with packed documents
# the ranks must be balanced by the attention each performs, not by tokens.

def chunk_work(S, P, doc=None):
    """Allowed (query, key) pairs per chunk of S/(2P) queries, counted from
    the causal (and document) mask itself."""
    if P < 1 or S <= 0 or S % (2 * P):
        raise ValueError("need P >= 1 and S > 0 divisible by 2P")
    c = S // (2 * P)
    pos = np.arange(S)
    d = None if doc is None else np.asarray(doc)
    work = []
    for i in range(2 * P):
        rows = pos[i * c:(i + 1) * c]
        m = A.allowed_mask(rows, pos, True, None if d is None else d[rows], d)
        work.append(int(m.sum()))
    return np.array(work, dtype=np.int64)


def best_pairing(work):
    """The two-chunks-per-rank assignment that minimises the largest rank's
    work, by exhaustive search over all pairings (small P only).  Returns that
    minimum."""
    items = list(range(len(work)))
    best = [None]

    def rec(rest, worst):
        if best[0] is not None and worst >= best[0]:
            return
        if not rest:
            best[0] = worst
            return
        a = rest[0]
        for k in range(1, len(rest)):
            b = rest[k]
            rec(rest[1:k] + rest[k + 1:], max(worst, int(work[a]) + int(work[b])))

    rec(items, 0)
    return best[0]


# ---- all-gather share --------------------------------------------------------
# [MaxText] diagram text, All-gather: a rank keeps its query shard and gathers
# every key and value, so its share is its queries against the whole sequence.

def allgather_share(q_rank, k, v, S, P, r, *, scale, doc=None, dout=None):
    """Rank r's share: q_rank holds its rows (zigzag chunks r and 2P-1-r, in
    local order); k, v the whole sequence in global order.  Returns (o, lse)
    and, with dout, (dq, dk, dv) where dk, dv are rank r's rows' contributions
    to every key."""
    qpos = rank_positions(S, P, r)
    kpos = np.arange(S)
    qdoc = None if doc is None else np.asarray(doc)[qpos]
    o, lse = A.forward(q_rank, k, v, qpos, kpos, scale=scale, causal=True, qdoc=qdoc, kdoc=doc)
    if dout is None:
        return o, lse
    dq, dk, dv = A.backward(q_rank, k, v, dout, lse, A.delta(o, dout), qpos, kpos, scale=scale, causal=True,
                            qdoc=qdoc, kdoc=doc)
    return o, lse, dq, dk, dv
