"""Plain fp64 CPU oracle: masked softmax attention, its log-sum-exp, the exact
merge of partial results, and the closed-form backward.

TEST INFRASTRUCTURE ONLY.  This module is the independent checker of the HIP
path: only the test suite, the smoke check and the CPU-baseline leg of the
benchmark may import it.  It shares no code, table or helper with the library
under ``sequence_context_parallelism_amd``; it never imports it and is never
imported by it.

Every function is written for clarity, in float64, with numpy (BLAS ``matmul``
is the only library step).  Inputs of any float dtype are upcast to float64
first, so bf16 inputs are consumed as their exact values.

Sources (the pages this method is described on):

* nougat.kr, "MaxText long-context training: KV parallelism", section
  "입력을 나눠도 KV가 다시 모이는 이유" (why the KV meets again after the input
  is split): a causal query needs the KV of the tokens before it, and the
  attention work grows with the square of the sequence length.
* same page, section "헤드를 나누거나, KV를 돌리거나" (split the heads, or rotate
  the KV): heads are computed independently; a ring step computes a partial
  attention against the KV chunk it holds and merges it into the running
  result; with grouped-query attention the KV heads bound the head split.
* siliconandsystems.com, "Llama 3 parallelism", section "네 병렬화는 서로 다른
  자원을 확보하는 방식" (the four parallelisms secure different resources):
  packed multi-document input must keep its document mask under context
  parallelism.

The pages state no formula.  The readings taken where they are silent (all
documented in the design notes): the causal mask includes the diagonal
(key position <= query position); a document mask allows only equal document
ids; the softmax scale is passed in (1/sqrt(d) in every workload); the
log-sum-exp is in natural-log units; a row with no allowed key has O = 0 and
LSE = -inf, and -inf is the identity of the merge; query head h reads KV head
floor(h * Hkv / Hq) (contiguous groups).
"""
from __future__ import annotations

import numpy as np

NEG_INF = -np.inf


def _f64(x):
    return None if x is None else np.asarray(x, dtype=np.float64)


def allowed_mask(qpos, kpos, causal, qdoc=None, kdoc=None):
    """Boolean [Lq, Lk]: may query i attend to key j.

    Causal access to earlier tokens (nougat.kr MaxText page, section on why the
    KV meets again) including the token itself; document mask for packed input
    (siliconandsystems.com Llama 3 page, section on the four parallelisms).
    Positions are global token positions; doc ids are per token.
    """
    qpos = np.asarray(qpos, dtype=np.int64)
    kpos = np.asarray(kpos, dtype=np.int64)
    m = np.ones((qpos.shape[0], kpos.shape[0]), dtype=bool)
    if causal:
        m &= kpos[None, :] <= qpos[:, None]
    if qdoc is not None or kdoc is not None:
        if qdoc is None or kdoc is None:
            raise ValueError("doc ids must be given for both queries and keys")
        m &= np.asarray(kdoc)[None, :] == np.asarray(qdoc)[:, None]
    return m


def kv_head(h, hq, hkv):
    """KV head read by query head h under grouped-query attention: the Hq/Hkv
    query heads of a group are contiguous (reading of the nougat.kr MaxText
    page's remark that KV heads bound the head split)."""
    if hq % hkv != 0:
        raise ValueError("hq must be a multiple of hkv")
    return (h * hkv) // hq


def forward(q, k, v, qpos, kpos, *, scale, causal, qdoc=None, kdoc=None,
            block=512):
    """Softmax attention of every query row against the allowed keys.

    q [Lq, Hq, d], k and v [Lk, Hkv, d].  Returns (o [Lq, Hq, d], lse [Hq, Lq])
    in float64.  For query head h and row i with allowed set J_i:
        s_ij = scale * <q_i, k_j>,  lse_i = log(sum_{j in J_i} exp(s_ij)),
        o_i  = sum_{j in J_i} exp(s_ij - lse_i) * v_j,
    and o_i = 0, lse_i = -inf when J_i is empty.  Rows are processed in blocks
    of ``block`` only to bound memory; every row is computed over all keys.
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    o = np.zeros((lq, hq, d))
    lse = np.full((hq, lq), NEG_INF)
    for i0 in range(0, lq, block):
        i1 = min(lq, i0 + block)
        allow = allowed_mask(qpos[i0:i1], kpos, causal,
                             None if qdoc is None else qdoc[i0:i1], kdoc)
        live = allow.any(axis=1)
        for h in range(hq):
            g = kv_head(h, hq, hkv)
            s = scale * (q[i0:i1, h, :] @ k[:, g, :].T)
            s = np.where(allow, s, NEG_INF)
            m = np.where(live, s.max(axis=1, initial=NEG_INF), 0.0)
            ell = np.exp(s - m[:, None]).sum(axis=1)
            with np.errstate(divide="ignore"):
                row_lse = np.where(live, m + np.log(ell), NEG_INF)
            p = np.where(allow, np.exp(s - np.where(live, row_lse, 0.0)[:, None]), 0.0)
            o[i0:i1, h, :] = p @ v[:, g, :]
            lse[h, i0:i1] = row_lse
    return o, lse


def forward_rows(q, k, v, qpos, kpos, rows, heads, *, scale, causal,
                 qdoc=None, kdoc=None):
    """The same definition as ``forward`` for a sample of (row, head) pairs.

    rows and heads are equal-length integer arrays.  Each sampled output is
    exact over all of its keys.  Returns (o [n, d], lse [n]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    hq, hkv = q.shape[1], k.shape[1]
    n = len(rows)
    o = np.zeros((n, q.shape[2]))
    lse = np.full(n, NEG_INF)
    for t, (i, h) in enumerate(zip(rows, heads)):
        g = kv_head(int(h), hq, hkv)
        allow = allowed_mask(np.asarray(qpos)[[i]], kpos, causal,
                             None if qdoc is None else np.asarray(qdoc)[[i]], kdoc)[0]
        if not allow.any():
            continue
        s = scale * (k[allow, g, :] @ q[i, h, :])
        m = s.max()
        lse[t] = m + np.log(np.exp(s - m).sum())
        o[t] = np.exp(s - lse[t]) @ v[allow, g, :]
    return o, lse


def merge(oa, lsea, ob, lseb):
    """Exact combination of two partial results over disjoint key sets.

    The ring step's "merge" (nougat.kr MaxText page, section on splitting heads
    or rotating the KV) written through the per-row log-sum-exp:
        L = log(exp(La) + exp(Lb)),
        O = exp(La - L) * Oa + exp(Lb - L) * Ob,
    with -inf as the identity (an empty partial leaves the other unchanged and
    two empty partials stay empty).  o* are [rows, H, d], lse* are [H, rows].
    """
    oa, ob = _f64(oa), _f64(ob)
    la, lb = _f64(lsea), _f64(lseb)
    m = np.maximum(la, lb)
    both_empty = np.isneginf(m)
    m_safe = np.where(both_empty, 0.0, m)
    wa = np.exp(la - m_safe)
    wb = np.exp(lb - m_safe)
    with np.errstate(divide="ignore"):
        lse = np.where(both_empty, NEG_INF, m_safe + np.log(wa + wb))
    lse_safe = np.where(both_empty, 0.0, lse)
    ca = np.where(both_empty, 0.0, np.exp(la - lse_safe))   # [H, rows]
    cb = np.where(both_empty, 0.0, np.exp(lb - lse_safe))
    o = ca.T[:, :, None] * oa + cb.T[:, :, None] * ob
    return o, lse


def delta(o, dout):
    """Delta_i = sum_e dO_ie * O_ie per row and head, returned as [H, L]."""
    return np.einsum("lhe,lhe->hl", _f64(o), _f64(dout))


def backward(q, k, v, dout, lse, dlt, qpos, kpos, *, scale, causal,
             qdoc=None, kdoc=None, block=512):
    """Gradient of the attention above, in closed form, given the row LSE and
    Delta of the *final* (merged) output.

    P_ij = exp(s_ij - lse_i) on allowed entries, else 0;
    dV_j = sum_i P_ij dO_i;   dP_ij = <dO_i, v_j>;   dS_ij = P_ij (dP_ij - Delta_i);
    dQ_i = scale sum_j dS_ij k_j;   dK_j = scale sum_i dS_ij q_i;
    dK and dV are summed over the query heads of each KV group.  Restricting the
    keys (or rows) to a chunk gives that chunk's contribution, which is how a
    ring step's backward is formed.  The pages say nothing of the backward; this
    is the derivative of the definition in ``forward``.
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    lse, dlt = _f64(lse), _f64(dlt)
    lq, hq, d = q.shape
    lk, hkv, _ = k.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for i0 in range(0, lq, block):
        i1 = min(lq, i0 + block)
        allow = allowed_mask(qpos[i0:i1], kpos, causal,
                             None if qdoc is None else qdoc[i0:i1], kdoc)
        for h in range(hq):
            g = kv_head(h, hq, hkv)
            row_lse = lse[h, i0:i1]
            live = ~np.isneginf(row_lse)
            s = scale * (q[i0:i1, h, :] @ k[:, g, :].T)
            p = np.where(allow & live[:, None],
                         np.exp(s - np.where(live, row_lse, 0.0)[:, None]), 0.0)
            dv[:, g, :] += p.T @ dout[i0:i1, h, :]
            dp = dout[i0:i1, h, :] @ v[:, g, :].T
            ds = p * (dp - dlt[h, i0:i1][:, None])
            dq[i0:i1, h, :] += scale * (ds @ k[:, g, :])
            dk[:, g, :] += scale * (ds.T @ q[i0:i1, h, :])
    return dq, dk, dv


def dq_rows(q, k, v, dout, lse, dlt, qpos, kpos, rows, heads, *, scale, causal,
            qdoc=None, kdoc=None):
    """dQ of sampled (row, head) pairs by the closed form of ``backward``.
    ``lse`` and ``dlt`` hold the final LSE and Delta of each sample ([n])."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    hq, hkv = q.shape[1], k.shape[1]
    out = np.zeros((len(rows), q.shape[2]))
    for t, (i, h) in enumerate(zip(rows, heads)):
        g = kv_head(int(h), hq, hkv)
        allow = allowed_mask(np.asarray(qpos)[[i]], kpos, causal,
                             None if qdoc is None else np.asarray(qdoc)[[i]], kdoc)[0]
        if not allow.any():
            continue
        s = scale * (k[allow, g, :] @ q[i, h, :])
        p = np.exp(s - lse[t])
        dp = v[allow, g, :] @ dout[i, h, :]
        ds = p * (dp - dlt[t])
        out[t] = scale * (ds @ k[allow, g, :])
    return out


def dkv_keys(q, k, v, dout, lse, dlt, qpos, kpos, keys, kvheads, *, scale, causal,
             qdoc=None, kdoc=None, rows=None):
    """dK and dV of sampled (key, KV head) pairs by the closed form of
    ``backward``.  ``lse`` and ``dlt`` are full [Hq, Lq] arrays, but only the
    rows that attend to a sampled key are read, so a caller may fill only
    those.  ``rows`` optionally restricts the query rows that contribute
    (a single ring rank's rows)."""
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    lq, hq, d = q.shape
    hkv = k.shape[1]
    grp = hq // hkv
    qpos = np.asarray(qpos)
    row_sel = np.ones(lq, bool) if rows is None else np.isin(np.arange(lq), rows)
    dk = np.zeros((len(keys), d))
    dv = np.zeros((len(keys), d))
    for t, (j, g) in enumerate(zip(keys, kvheads)):
        allow = allowed_mask(qpos, np.asarray(kpos)[[j]], causal, qdoc,
                             None if kdoc is None else np.asarray(kdoc)[[j]])[:, 0]
        allow &= row_sel
        idx = np.nonzero(allow)[0]
        for h in range(g * grp, (g + 1) * grp):
            s = scale * (q[idx, h, :] @ k[j, g, :])
            p = np.exp(s - lse[h, idx])
            dv[t] += p @ dout[idx, h, :]
            dp = dout[idx, h, :] @ v[j, g, :]
            ds = p * (dp - dlt[h, idx])
            dk[t] += scale * (ds @ q[idx, h, :])
    return dk, dv


def tile_classes(qpos, kpos, causal, bq, bk, qdoc=None, kdoc=None):
    """Per (bq x bk) tile: 0 if no entry is allowed, 1 if every entry is
    allowed, 2 otherwise.  Only entries inside [0, Lq) x [0, Lk) count (the
    last row and column of tiles may be ragged).  Defined by reducing the
    explicit mask, so skipping class-0 tiles provably drops nothing."""
    allow = allowed_mask(qpos, kpos, causal, qdoc, kdoc)
    lq, lk = allow.shape
    nq, nk = -(-lq // bq), -(-lk // bk)
    out = np.zeros((nq, nk), dtype=np.int8)
    for a in range(nq):
        for b in range(nk):
            t = allow[a * bq:(a + 1) * bq, b * bk:(b + 1) * bk]
            out[a, b] = 1 if t.all() else (2 if t.any() else 0)
    return out
