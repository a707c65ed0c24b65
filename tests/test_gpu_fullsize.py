"""GPU parity at the benchmark's full sizes, in the launch configuration that
bench.py times (its Workload class: same shapes, seeds, entry points and
workspace), on sampled outputs the fp64 oracle computes exactly (512 rows on
every head for the 64K Ulysses share, fewer where the oracle's dense rows
over 131K-1M keys would take minutes):

* O, LSE and dQ of sampled (row, head) pairs -- each row exact over all of
  its keys (the oracle's forward/backward on that subset of query rows);
* dK and dV of sampled keys among the last global positions -- the rows that
  attend to them are few, so the oracle runs the backward over exactly those
  rows (for a single ring rank, only that rank's rows, which is what its dK/dV
  hold).

Workloads: the Ulysses share (S=65,536, 8/2 heads), rank 0 of the zigzag ring
(S=131,072, P=8, 32/8 heads), packed documents (S=131,072, 32/8 heads) and
rank 0 of the USP share (S=1,048,576, ring of 4, 8/2 heads)."""
import math
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

SAMPLES = {"ulysses_64k": (512, 96, 6), "ring_128k": (48, 96, 6), "docs_128k": (48, 96, 6),
           "usp_1m": (16, 16, 4)}   # (sampled rows, last positions, sampled keys)


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


@pytest.mark.parametrize("name", ["ulysses_64k", "ring_128k", "docs_128k", "usp_1m"])
def test_full_size_sampled_parity(gpu_lib, name):
    import bench
    _say(f"[fullsize] {name}: building inputs")
    wl = bench.Workload(name, torch, cp, cpinputs)
    wl.step(cp)
    torch.cuda.synchronize()
    _say(f"[fullsize] {name}: step done, checking samples")
    n_rows, last, n_keys = SAMPLES[name]
    qpos, kpos, qdoc, kdoc = _positions(wl)
    scale = 1.0 / math.sqrt(wl.d)
    tol = TOL[torch.bfloat16]
    rng = np.random.default_rng(12345)
    k = wl.k.float().cpu().numpy()
    v = wl.v.float().cpu().numpy()

    # ---- sampled query rows: O, LSE, dQ --------------------------------
    lq = wl.rows
    rows = np.unique(np.concatenate([[0, lq - 1], rng.choice(lq, size=n_rows - 2, replace=False)]))
    q_s, do_s = _rows(wl.q, rows), _rows(wl.dout, rows)
    qd_s = None if qdoc is None else qdoc[rows]
    o_ref, lse_ref = A.forward(q_s, k, v, qpos[rows], kpos, scale=scale, causal=True, qdoc=qd_s, kdoc=kdoc)
    dlt_ref = A.delta(o_ref, do_s)
    dq_ref, _, _ = A.backward(q_s, k, v, do_s, lse_ref, dlt_ref, qpos[rows], kpos, scale=scale,
                              causal=True, qdoc=qd_s, kdoc=kdoc)
    o_gpu = _rows(wl.o, rows)
    lse_gpu = wl.lse[:, torch.as_tensor(rows, device=wl.lse.device)].double().cpu().numpy()
    dq_gpu = _rows(wl.dq, rows)
    e_o, e_l, e_dq = max_abs(o_gpu, o_ref), lse_err(lse_gpu, lse_ref), max_abs(dq_gpu, dq_ref)
    _say(f"[fullsize] {name}: {len(rows)} rows x {wl.hq} heads: O {e_o:.2e} LSE {e_l:.2e} dQ {e_dq:.2e}")
    assert e_o <= tol["o"]
    assert e_l <= tol["lse"]
    assert e_dq <= grad_tol(dq_ref, tol["grad"])

    # ---- sampled keys among the last positions: dK, dV -------------------
    kp_min = np.sort(kpos)[-last]
    key_idx = np.nonzero(kpos >= kp_min)[0]
    keys = np.sort(rng.choice(key_idx, size=n_keys, replace=False))
    att = np.nonzero(qpos >= kp_min)[0]            # every row that can attend a sampled key
    q_a, do_a = _rows(wl.q, att), _rows(wl.dout, att)
    qd_a = None if qdoc is None else qdoc[att]
    o_a, lse_a = A.forward(q_a, k, v, qpos[att], kpos, scale=scale, causal=True, qdoc=qd_a, kdoc=kdoc)
    _, dk_ref, dv_ref = A.backward(q_a, k, v, do_a, lse_a, A.delta(o_a, do_a), qpos[att], kpos,
                                   scale=scale, causal=True, qdoc=qd_a, kdoc=kdoc)
    dk_gpu, dv_gpu = _rows(wl.dk, keys), _rows(wl.dv, keys)
    e_dk, e_dv = max_abs(dk_gpu, dk_ref[keys]), max_abs(dv_gpu, dv_ref[keys])
    _say(f"[fullsize] {name}: {len(keys)} keys ({len(att)} attending rows): dK {e_dk:.2e} dV {e_dv:.2e}")
    assert e_dk <= grad_tol(dk_ref[keys], tol["grad"])
    assert e_dv <= grad_tol(dv_ref[keys], tol["grad"])
