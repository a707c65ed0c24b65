"""GPU parity at the benchmark's full sizes, in the launch configuration that
bench.py times (its Workload class: same shapes, seeds, entry points and
workspace), on outputs the fp64 oracle computes exactly:

* O, LSE and dQ of sampled (row, head) pairs -- each row exact over all of
  its keys (512 rows for the 64K Ulysses share, 256 for the 1M USP share, 64
  for the 128K ring and packed-document workloads);
* the same for rank P-1 of the 128K ring, whose rows sit in the middle of
  the sequence (test_full_size_ring_last_rank);
* dK and dV of sampled keys spread over the sequence -- key 0, keys of the
  first 128-key block, of middle blocks and of the last one.  The oracle
  first runs its forward over every query row that attends those keys (one
  KV group: its query heads) to get each row's final LSE and Delta, then the
  closed-form dK/dV of each sampled key over all of those rows.  For the
  packed documents the keys sit at the start of the longest documents; for a
  ring rank they sit at the start of each visiting rank's shard, and the
  contributions are those of rank 0's rows (what its dK/dV hold).

The forward over all rows of a KV group is split into query-row blocks that
the plain oracle runs on a thread pool (numpy releases the interpreter lock
in its array work); each block's keys are cut at the block's last position,
which drops only keys the causal mask gives zero weight.

Partial results merged exactly through the LSE (nougat.kr, "MaxText
long-context training: KV parallelism", section "헤드를 나누거나, KV를
돌리거나") are what these checks cover at scale."""
import concurrent.futures as cf
import math
import os
import sys

import numpy as np
import pytest
import torch

import cpinputs
import sequence_context_parallelism_amd as cp
from gpu_util import TOL, grad_tol, lse_err, max_abs
from oracle import attention as A
from oracle import schedule as Z

pytestmark = pytest.mark.gpu

NAMES = ["ulysses_64k", "ring_128k", "docs_128k", "usp_1m"]
ROWS = {"ulysses_64k": 512, "ring_128k": 64, "docs_128k": 64, "usp_1m": 256}
WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def _say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _positions(wl):
    """Global positions of the workload's query rows and key rows, and doc ids."""
    if wl.name in ("ring_128k", "usp_1m"):
        S, P = wl.S, wl.P
        qpos = Z.rank_positions(S, P, 0)
        kpos = np.concatenate([Z.rank_positions(S, P, r) for r in range(P)])
        return qpos, kpos, None, None
    pos = np.arange(wl.S)
    if wl.doc is None:
        return pos, pos, None, None
    doc = wl.doc.cpu().numpy()
    return pos, pos, doc, doc


def _rows(t, idx):
    """Rows `idx` of a device tensor, on the host in float64."""
    return t[torch.as_tensor(idx, device=t.device)].double().cpu().numpy()


def _blas_single_thread():
    try:
        import threadpoolctl
        return threadpoolctl.threadpool_limits(1)
    except Exception:                      # pragma: no cover - threadpoolctl is installed here
        import contextlib
        return contextlib.nullcontext()


def _key_range(kpos, kdoc, qpos_blk, qdoc_blk):
    """Key rows that some query of the block may attend: position at most the
    block's last query position and, with documents, id at least the block's
    smallest (ids do not decrease along positions).  The other keys are
    masked for every row of the block and carry zero weight."""
    order = np.argsort(kpos, kind="stable")
    ks = np.asarray(kpos)[order]
    hi = np.searchsorted(ks, int(np.max(qpos_blk)), side="right")
    lo = 0
    if kdoc is not None:
        lo = np.searchsorted(np.asarray(kdoc)[order], int(np.min(qdoc_blk)), side="left")
    return order[lo:hi]


def _parallel_forward(q, k, v, qpos, kpos, qdoc, kdoc, scale, block_rows):
    """The oracle forward of every row of q, in row blocks on a thread pool,
    each block against the keys _key_range keeps."""
    n = q.shape[0]

    def one(i0):
        i1 = min(n, i0 + block_rows)
        qd = None if qdoc is None else qdoc[i0:i1]
        sel = _key_range(kpos, kdoc, qpos[i0:i1], qd)
        return i0, A.forward(q[i0:i1], k[sel], v[sel], qpos[i0:i1], np.asarray(kpos)[sel], scale=scale,
                             causal=True, qdoc=qd, kdoc=None if kdoc is None else kdoc[sel], block=256)

    o = np.zeros(q.shape)
    lse = np.zeros((q.shape[1], n))
    with _blas_single_thread(), cf.ThreadPoolExecutor(WORKERS) as ex:
        for i0, (bo, bl) in ex.map(one, range(0, n, block_rows)):
            o[i0:i0 + bo.shape[0]] = bo
            lse[:, i0:i0 + bo.shape[0]] = bl
    return o, lse


@pytest.fixture(scope="module")
def workloads():
    """The bench's workloads, one at a time (each is dropped before the next
    is built, so device memory holds one)."""
    cache = {}

    def get(name):
        if name not in cache:
            cache.clear()
            torch.cuda.empty_cache()
            import bench
            _say(f"[fullsize] {name}: building inputs and running one step")
            wl = bench.Workload(name, torch, cp, cpinputs)
            wl.step(cp)
            torch.cuda.synchronize()
            cache[name] = wl
        return cache[name]
    yield get
    cache.clear()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", NAMES)
def test_full_size_sampled_rows(gpu_lib, workloads, name):
    wl = workloads(name)
    qpos, kpos, qdoc, kdoc = _positions(wl)
    scale = 1.0 / math.sqrt(wl.d)
    tol = TOL[torch.bfloat16]
    rng = np.random.default_rng(12345)
    k = wl.k.float().cpu().numpy()
    v = wl.v.float().cpu().numpy()
    lq = wl.rows
    n_rows = ROWS[name]
    rows = np.unique(np.concatenate([[0, lq - 1], rng.choice(lq, size=n_rows - 2, replace=False)]))
    q_s, do_s = _rows(wl.q, rows), _rows(wl.dout, rows)
    qd_s = None if qdoc is None else qdoc[rows]
    _say(f"[fullsize] {name}: oracle on {len(rows)} rows x {wl.hq} heads")

    def one(idx):
        sub = rows[idx]
        qd = None if qd_s is None else qd_s[idx]
        sel = _key_range(kpos, kdoc, qpos[sub], qd)
        kp, ks_, vs_ = np.asarray(kpos)[sel], k[sel], v[sel]
        kd = None if kdoc is None else kdoc[sel]
        o_r, l_r = A.forward(q_s[idx], ks_, vs_, qpos[sub], kp, scale=scale, causal=True, qdoc=qd, kdoc=kd)
        dq_r, _, _ = A.backward(q_s[idx], ks_, vs_, do_s[idx], l_r, A.delta(o_r, do_s[idx]), qpos[sub], kp,
                                scale=scale, causal=True, qdoc=qd, kdoc=kd)
        return idx, o_r, l_r, dq_r

    parts = np.array_split(np.arange(len(rows)), min(len(rows), 4 * WORKERS))
    o_ref = np.zeros((len(rows), wl.hq, wl.d))
    lse_ref = np.zeros((wl.hq, len(rows)))
    dq_ref = np.zeros_like(o_ref)
    # the oracle backward holds dK/dV of every key it is given: at 1M keys a
    # few GB per call, so fewer calls run at once there
    workers = 4 if wl.S > (1 << 18) else WORKERS
    with _blas_single_thread(), cf.ThreadPoolExecutor(workers) as ex:
        for idx, o_r, l_r, dq_r in ex.map(one, parts):
            o_ref[idx], lse_ref[:, idx], dq_ref[idx] = o_r, l_r, dq_r
    o_gpu = _rows(wl.o, rows)
    lse_gpu = wl.lse[:, torch.as_tensor(rows, device=wl.lse.device)].double().cpu().numpy()
    dq_gpu = _rows(wl.dq, rows)
    e_o, e_l, e_dq = max_abs(o_gpu, o_ref), lse_err(lse_gpu, lse_ref), max_abs(dq_gpu, dq_ref)
    _say(f"[fullsize] {name}: {len(rows)} rows x {wl.hq} heads: O {e_o:.2e} LSE {e_l:.2e} dQ {e_dq:.2e}")
    assert e_o <= tol["o"]
    assert e_l <= tol["lse"]
    assert e_dq <= grad_tol(dq_ref, tol["grad"])


def _key_samples(wl, kpos, kdoc, rng):
    """Indices (into the key rows) of the sampled keys: spread over the
    sequence and over the key blocks the dK/dV kernel owns."""
    S = int(np.max(kpos)) + 1
    if kdoc is not None:
        # the start and later tokens of the two longest documents
        ids, starts, counts = np.unique(kdoc, return_index=True, return_counts=True)
        longest = np.argsort(counts, kind="stable")[::-1][:2]
        want = []
        for t in longest:
            s0, L = int(starts[t]), int(counts[t])
            want += [s0, s0 + 1, s0 + min(L - 1, 200), s0 + L // 2]
        want = np.array(want)
    elif wl.name == "usp_1m":
        # keys among the last 2,048 global positions (the tail of rank 0's own
        # second chunk): the rows that attend them are few
        c = wl.S // (2 * wl.P)
        tail = np.arange(2 * c - 2048, 2 * c)
        return np.unique(np.concatenate([[tail[0], tail[-1]], rng.choice(tail, size=6, replace=False)]))
    elif wl.name == "ring_128k":
        # the first rows of every visiting shard, and one later row of each
        n = wl.S // wl.P
        want = []
        for j in range(wl.P):
            want += [j * n, j * n + 1, j * n + int(rng.integers(2, 128)), j * n + n // 2 + 7]
        return np.array(want)                       # already key-row indices (sharded order)
    else:
        blk = 128
        want = [0, 1, 63, 127, 128 + 5, S // 2 - 1, S // 2 + 64, S - blk, S - 1]
        want += list(rng.choice(S, size=3, replace=False))
        want = np.array(want)
    pos_to_row = np.empty(S, dtype=np.int64)
    pos_to_row[np.asarray(kpos)] = np.arange(len(kpos))
    return pos_to_row[np.unique(want)]


@pytest.mark.parametrize("name", NAMES)
def test_full_size_dkdv_long_paths(gpu_lib, workloads, name):
    wl = workloads(name)
    qpos, kpos, qdoc, kdoc = _positions(wl)
    scale = 1.0 / math.sqrt(wl.d)
    tol = TOL[torch.bfloat16]
    rng = np.random.default_rng(777)
    keys = _key_samples(wl, kpos, kdoc, rng)
    g = 0                                           # one KV group: KV head 0 and its query heads
    grp = wl.hq // wl.hkv
    heads = slice(g * grp, (g + 1) * grp)
    kmin = int(np.min(np.asarray(kpos)[keys]))
    att = np.nonzero(qpos >= kmin)[0]               # every query row that can attend a sampled key
    if qdoc is not None:
        att = att[np.isin(qdoc[att], kdoc[keys])]   # ... in the sampled keys' documents
    _say(f"[fullsize] {name}: dK/dV of {len(keys)} keys, oracle forward over {len(att)} rows x {grp} heads")
    q_a = wl.q[torch.as_tensor(att, device=wl.q.device)][:, heads].double().cpu().numpy()
    do_a = wl.dout[torch.as_tensor(att, device=wl.dout.device)][:, heads].double().cpu().numpy()
    k1 = wl.k[:, g:g + 1].double().cpu().numpy()
    v1 = wl.v[:, g:g + 1].double().cpu().numpy()
    qd_a = None if qdoc is None else qdoc[att]
    o_a, lse_a = _parallel_forward(q_a, k1, v1, qpos[att], kpos, qd_a, kdoc, scale, 1024)
    dlt_a = A.delta(o_a, do_a)
    _say(f"[fullsize] {name}: oracle forward done")
    dk_ref, dv_ref = A.dkv_keys(q_a, k1, v1, do_a, lse_a, dlt_a, qpos[att], kpos, keys, np.zeros(len(keys), int),
                                scale=scale, causal=True, qdoc=qd_a, kdoc=kdoc)
    dk_gpu = _rows(wl.dk, keys)[:, g]
    dv_gpu = _rows(wl.dv, keys)[:, g]
    e_dk, e_dv = max_abs(dk_gpu, dk_ref), max_abs(dv_gpu, dv_ref)
    _say(f"[fullsize] {name}: keys at positions {np.asarray(kpos)[keys].tolist()}: dK {e_dk:.2e} dV {e_dv:.2e}")
    assert e_dk <= grad_tol(dk_ref, tol["grad"])
    assert e_dv <= grad_tol(dv_ref, tol["grad"])


def test_full_size_ring_last_rank(gpu_lib):
    """Rank P-1 of the 128K zigzag ring (its chunks P-1 and P, the middle of the
    sequence, so its steps mix diagonal, full and skipped blocks differently
    from rank 0): sampled rows' O, LSE, dQ and sampled keys' dK/dV (this
    rank's rows' contributions) against the oracle, through cp_ring_emulate
    at the bench's shapes."""
    torch.cuda.empty_cache()
    S, hq, hkv, d, P = 131072, 32, 8, 128, 8
    r = P - 1
    n = S // P
    seed = cpinputs.SEEDS["ring_128k"] + 17
    q, k, v = cpinputs.normal_torch(seed, [(S, hq, d), (S, hkv, d), (S, hkv, d)], "cuda", torch.bfloat16)
    (dout,) = cpinputs.normal_torch(seed + 1, [(n, hq, d)], "cuda", torch.bfloat16)
    sh = cp.make_shape(hq, hkv, d, hq * d, hkv * d, 1.0 / math.sqrt(d), True, cp.CP_BF16)
    o = torch.empty(n, hq, d, device="cuda", dtype=torch.bfloat16)
    lse = torch.empty(hq, n, device="cuda")
    dq = torch.empty(n, hq, d, device="cuda")
    dk = torch.empty(S, hkv, d, device="cuda")
    dv = torch.empty_like(dk)
    ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, r, cp.CP_BF16, True))
    _say(f"[fullsize] ring_128k rank {r}: running the ring")
    cp.cp_ring_emulate(sh, S, P, r, q, k, v, None, o, lse, dout, dq, dk, dv, workspace=ws)
    torch.cuda.synchronize()

    qpos = Z.rank_positions(S, P, r)
    kpos = np.concatenate([Z.rank_positions(S, P, j) for j in range(P)])
    scale = 1.0 / math.sqrt(d)
    tol = TOL[torch.bfloat16]
    qr = q[r * n:(r + 1) * n]                      # this rank's rows (sharded order)
    kh = k.float().cpu().numpy()
    vh = v.float().cpu().numpy()

    # sampled rows: O, LSE, dQ
    rng = np.random.default_rng(4242)
    rows = np.unique(np.concatenate([[0, n // 2 - 1, n // 2, n - 1], rng.choice(n, size=60, replace=False)]))
    q_s, do_s = _rows(qr, rows), _rows(dout, rows)
    _say(f"[fullsize] ring_128k rank {r}: oracle on {len(rows)} rows x {hq} heads")

    def one(idx):
        sub = rows[idx]
        sel = _key_range(kpos, None, qpos[sub], None)
        kp = np.asarray(kpos)[sel]
        o_r, l_r = A.forward(q_s[idx], kh[sel], vh[sel], qpos[sub], kp, scale=scale, causal=True)
        dq_r, _, _ = A.backward(q_s[idx], kh[sel], vh[sel], do_s[idx], l_r, A.delta(o_r, do_s[idx]), qpos[sub],
                                kp, scale=scale, causal=True)
        return idx, o_r, l_r, dq_r

    parts = np.array_split(np.arange(len(rows)), min(len(rows), 4 * WORKERS))
    o_ref = np.zeros((len(rows), hq, d))
    lse_ref = np.zeros((hq, len(rows)))
    dq_ref = np.zeros_like(o_ref)
    with _blas_single_thread(), cf.ThreadPoolExecutor(WORKERS) as ex:
        for idx, o_r, l_r, dq_r in ex.map(one, parts):
            o_ref[idx], lse_ref[:, idx], dq_ref[idx] = o_r, l_r, dq_r
    e_o = max_abs(_rows(o, rows), o_ref)
    e_l = lse_err(lse[:, torch.as_tensor(rows, device=lse.device)].double().cpu().numpy(), lse_ref)
    e_dq = max_abs(_rows(dq, rows), dq_ref)
    _say(f"[fullsize] ring_128k rank {r}: O {e_o:.2e} LSE {e_l:.2e} dQ {e_dq:.2e}")
    assert e_o <= tol["o"]
    assert e_l <= tol["lse"]
    assert e_dq <= grad_tol(dq_ref, tol["grad"])

    # sampled keys: dK/dV of this rank's rows, KV head 0 and its query heads
    keys = []
    for j in range(P):
        keys += [j * n, j * n + 1, j * n + int(rng.integers(2, 128)), j * n + n // 2 + 7]
    keys = np.array(keys)
    g, grp = 0, hq // hkv
    kmin = int(np.min(np.asarray(kpos)[keys]))
    att = np.nonzero(qpos >= kmin)[0]
    q_a = qr[torch.as_tensor(att, device=q.device)][:, g * grp:(g + 1) * grp].double().cpu().numpy()
    do_a = dout[torch.as_tensor(att, device=q.device)][:, g * grp:(g + 1) * grp].double().cpu().numpy()
    k1 = k[:, g:g + 1].double().cpu().numpy()
    v1 = v[:, g:g + 1].double().cpu().numpy()
    _say(f"[fullsize] ring_128k rank {r}: dK/dV of {len(keys)} keys, oracle forward over {len(att)} rows x {grp} heads")
    o_a, lse_a = _parallel_forward(q_a, k1, v1, qpos[att], kpos, None, None, scale, 1024)
    dlt_a = A.delta(o_a, do_a)
    dk_ref, dv_ref = A.dkv_keys(q_a, k1, v1, do_a, lse_a, dlt_a, qpos[att], kpos, keys, np.zeros(len(keys), int),
                                scale=scale, causal=True)
    e_dk = max_abs(_rows(dk, keys)[:, g], dk_ref)
    e_dv = max_abs(_rows(dv, keys)[:, g], dv_ref)
    _say(f"[fullsize] ring_128k rank {r}: dK {e_dk:.2e} dV {e_dv:.2e}")
    assert e_dk <= grad_tol(dk_ref, tol["grad"])
    assert e_dv <= grad_tol(dv_ref, tol["grad"])
    del q, k, v, dout, o, lse, dq, dk, dv, ws
    torch.cuda.empty_cache()
