"""Benchmark of one GPU's share of context-parallel attention on MI355X.

Default workload: the Ulysses share of a Llama-3.1-8B-shaped layer at SP=4:
the full S=65536 causal sequence for this GPU's 8 query heads / 2 KV heads,
d=128, bf16, forward + backward (dO ~ N(0,1)).  One step = one
cp_ulysses_share call with the backward (forward chunk attention, Delta,
backward chunk attention writing the gradients), all in libcpattn's kernels.

Prints ONE JSON line.  ``value`` is the causal-FLOP throughput of the step:
algorithmic FLOPs (4*d per allowed (query, key) pair per query head forward,
10*d backward) divided by the step time.  ``roofline`` describes the dominant
kernel (timed alone with HIP events on its stream), ``cpu_baseline`` the
fp64 oracle timed on the host cores on a bounded sample.

Other workloads (``--workload``): ring_128k (rank 0 of a zigzag ring of
P=8 over S=131072, 32/8 heads), docs_128k (S=131072 packed lognormal
documents, 32/8 heads), usp_1m (rank 0 of a 4-rank ring over S=1,048,576 for
an 8/2 head slice).  The default run also carries a ``workloads`` object with
a short run of each of them (1 warm-up, 2 timed steps, medians), and for the
packed documents the per-rank time of a P=8 ring under the zigzag layout and
under the document-balanced pairing.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA, published
METRIC = "causal attn fwd+bwd TFLOPS & tokens/s, 64K GQA32/8 d128 bf16; % MFMA peak"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="ulysses_64k",
                    choices=["ulysses_64k", "ring_128k", "docs_128k", "usp_1m"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-kernel-timing", action="store_true")
    ap.add_argument("--no-workloads", action="store_true",
                    help="with the default workload, skip the short runs of the other workloads")
    ap.add_argument("--gemm-ceiling", action="store_true",
                    help="only measure the vendor library's bf16 GEMM throughput (16384^3) and print it")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain 512 MiB device copy (3 times), the reference for "
                         "scaling HBM traffic counters")
    return ap.parse_args()


def causal_pairs_zigzag_rank(S, P):
    c = S // (2 * P)
    return P * 2 * c * c + c


class Workload:
    """Seeded synthetic inputs of one configuration, resident in HBM."""

    def __init__(self, name, torch, cp, cpinputs):
        self.name = name
        dev = "cuda"
        bf = torch.bfloat16
        self.dev = dev
        if name == "ulysses_64k":
            S, hq, hkv, d, sp = 65536, 32, 8, 128, 4
            self.S, self.hq, self.hkv, self.d = S, hq // sp, hkv // sp, d
            seed = cpinputs.SEEDS["ulysses_64k"]
            # the share after the all-to-all: 8 query heads, 2 KV heads, full sequence
            self.q, self.k, self.v, self.dout = cpinputs.normal_torch(
                seed, [(S, self.hq, d), (S, self.hkv, d), (S, self.hkv, d), (S, self.hq, d)], dev, bf)
            self.doc = None
            self.rows = S
            self.pairs_per_head = S * (S + 1) // 2
            self.tokens = S
            self.group = sp
            self.config = {"workload": "ulysses_share_sp4", "S": S, "heads_q": self.hq, "heads_kv": self.hkv,
                           "layer_heads": f"{hq}/{hkv}", "d": d, "causal": True, "sp": sp}
        elif name in ("ring_128k", "usp_1m"):
            if name == "ring_128k":
                S, hq, hkv, d, P = 131072, 32, 8, 128, 8
            else:
                S, hq, hkv, d, P = 1048576, 8, 2, 128, 4
            self.S, self.hq, self.hkv, self.d, self.P = S, hq, hkv, d, P
            seed = cpinputs.SEEDS[name]
            n = S // P
            # every rank's shard, in sharded order (random data: order is immaterial)
            self.q, self.k, self.v = cpinputs.normal_torch(seed, [(n, hq, d), (S, hkv, d), (S, hkv, d)], dev, bf)
            (self.dout,) = cpinputs.normal_torch(seed + 1, [(n, hq, d)], dev, bf)
            self.doc = None
            self.rows = n
            self.pairs_per_head = causal_pairs_zigzag_rank(S, P)
            self.tokens = S
            self.group = P if name == "ring_128k" else 16
            self.config = {"workload": "ring_rank0_zigzag" if name == "ring_128k" else "usp_share_a2a4_ring4",
                           "S": S, "P": P, "local_q": n, "heads_q": hq, "heads_kv": hkv, "d": d, "causal": True}
        else:
            S, hq, hkv, d = 131072, 32, 8, 128
            self.S, self.hq, self.hkv, self.d = S, hq, hkv, d
            seed = cpinputs.SEEDS["docs_128k"]
            self.q, self.k, self.v, self.dout = cpinputs.normal_torch(
                seed, [(S, hq, d), (S, hkv, d), (S, hkv, d), (S, hq, d)], dev, bf)
            lens = cpinputs.lognormal_doc_lengths(S)
            self.doc = torch.from_numpy(cpinputs.doc_ids_from_lengths(lens)).to(dev)
            self.rows = S
            self.pairs_per_head = int(sum(int(L) * (int(L) + 1) // 2 for L in lens))
            self.tokens = S
            self.group = 1
            self.config = {"workload": "packed_docs", "S": S, "heads_q": hq, "heads_kv": hkv, "d": d,
                           "causal": True, "docs": int(len(lens)), "doc_len_median": 4096, "doc_sigma": 1.0}
        self.flops_fwd = 4 * self.d * self.pairs_per_head * self.hq
        self.flops_bwd = 10 * self.d * self.pairs_per_head * self.hq
        hq, hkv, d, rows = self.hq, self.hkv, self.d, self.rows
        self.o = torch.empty(rows, hq, d, device=dev, dtype=bf)
        self.lse_shape = (hq, rows)
        self.lse = torch.empty(hq, rows, device=dev)
        self.dq = torch.empty(rows, hq, d, device=dev)
        kv_rows = self.k.shape[0]
        self.dk = torch.empty(kv_rows, hkv, d, device=dev)
        self.dv = torch.empty_like(self.dk)
        self.delta = torch.empty(hq, rows, device=dev)
        self.sh = cp.make_shape(hq, hkv, d, hq * d, hkv * d, 1.0 / math.sqrt(d), True, cp.CP_BF16)
        if name in ("ring_128k", "usp_1m"):
            self.ws = cp.workspace(cp.cp_ring_workspace_bytes(self.sh, self.S, self.P, 0, cp.CP_BF16, True))
        else:
            self.ws = cp.workspace(cp.cp_ulysses_workspace_bytes(self.sh, self.S, 1, True))

    def step(self, cp):
        if self.name in ("ring_128k", "usp_1m"):
            # this GPU is rank 0; the KV for the steps is every rank's shard
            cp.cp_ring_emulate(self.sh, self.S, self.P, 0, self.q_full_rank0(), self.k, self.v, None,
                               self.o, self.lse, self.dout, self.dq, self.dk, self.dv, workspace=self.ws)
        else:
            cp.cp_ulysses_share(self.sh, self.S, 1, 0, self.q, self.k, self.v, self.doc, self.o, self.lse,
                                self.dout, self.dq, self.dk, self.dv, workspace=self.ws)

    def q_full_rank0(self):
        # cp_ring_emulate reads rank r's Q rows at offset r * S/P of a sharded
        # array; rank 0's rows are first, so the rank-0 shard alone suffices.
        return self.q


def kernel_times(wl, cp, torch, iters):
    """Average duration (ms) of each hot kernel launched alone, timed with HIP
    events on the stream it is launched on: the forward chunk kernel, the two
    backward kernels (dK/dV and dQ) and the LSE merge.  Returns a dict with the
    algorithmic work of one launch of each."""
    st = torch.cuda.current_stream()
    if wl.name in ("ring_128k", "usp_1m"):
        S, P = wl.S, wl.P
        c = S // (2 * P)
        n = S // P
        qs = cp.make_span(0, c, (2 * P - 1) * c, c)
        ks = cp.make_span(0, c, (2 * P - 1) * c, c)           # step 0: the rank's own KV
        k, v = wl.k[:n], wl.v[:n]
        pairs = 2 * c * c + c
        dk, dv = wl.dk[:n], wl.dv[:n]
    else:
        qs = cp.make_span(0, wl.rows, 0, 0, wl.doc)
        ks = cp.make_span(0, wl.rows, 0, 0, wl.doc)
        k, v = wl.k, wl.v
        pairs = wl.pairs_per_head
        dk, dv = wl.dk, wl.dv
    o32 = torch.empty(wl.rows, wl.hq, wl.d, device=wl.dev)
    lse2 = torch.empty_like(wl.lse)
    o_part = torch.empty_like(o32)
    # the forward as the step runs it: a single-chunk share writes its final
    # bf16 output; a ring step writes an fp32 partial
    o_fwd = o32 if wl.name in ("ring_128k", "usp_1m") else wl.o
    cp.cp_attn_chunk_fwd(wl.sh, wl.q, qs, k, v, ks, wl.o, wl.lse)
    cp.cp_attn_delta(wl.o, wl.dout, wl.delta)
    cp.cp_attn_chunk_fwd(wl.sh, wl.q, qs, k, v, ks, o_part, lse2)
    torch.cuda.synchronize()
    launches = [
        lambda: cp.cp_attn_chunk_fwd(wl.sh, wl.q, qs, k, v, ks, o_fwd, lse2),
        lambda: cp.cp_attn_chunk_bwd_dkdv(wl.sh, wl.q, qs, k, v, ks, wl.dout, wl.lse, wl.delta, dk, dv),
        lambda: cp.cp_attn_chunk_bwd_dq(wl.sh, wl.q, qs, k, v, ks, wl.dout, wl.lse, wl.delta, wl.dq),
        lambda: cp.cp_lse_merge(o32, lse2, o_part, wl.lse),       # a partial into an accumulator
        lambda: cp.cp_attn_delta(wl.o, wl.dout, wl.delta),        # Delta = rowsum(dO * O), final output
    ]
    ms, med = [], []
    for fn in launches:         # each launch bracketed by events on the stream it runs on
        ev = [torch.cuda.Event(enable_timing=True) for _ in range(iters + 1)]
        ev[0].record(st)
        for i in range(iters):
            fn()
            ev[i + 1].record(st)
        torch.cuda.synchronize()
        per = [ev[i].elapsed_time(ev[i + 1]) for i in range(iters)]
        ms.append(sum(per) / iters)
        med.append(float(np.median(per)))
    rh = wl.rows * wl.hq
    extra = {}
    if wl.name == "ulysses_64k":
        # the all-to-all on either side of the share, emulated: rank 0's query
        # heads out of the full token-split layer tensor, and its output back
        layer_hq = wl.hq * wl.group
        x = torch.empty(wl.S, layer_hq, wl.d, device=wl.dev, dtype=torch.bfloat16)
        x.normal_()
        y = torch.empty(wl.S, wl.hq, wl.d, device=wl.dev, dtype=torch.bfloat16)
        cp.cp_a2a_tokens_to_heads(x, wl.group, 0, y)
        cp.cp_a2a_heads_to_tokens(y, wl.group, 0, x)
        ev2 = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        torch.cuda.synchronize()
        ev2[0].record(st)
        for _ in range(iters):
            cp.cp_a2a_tokens_to_heads(x, wl.group, 0, y)
        ev2[1].record(st)
        for _ in range(iters):
            cp.cp_a2a_heads_to_tokens(y, wl.group, 0, x)
        ev2[2].record(st)
        torch.cuda.synchronize()
        moved = 2 * y.numel() * y.element_size()          # read + write of the rank's heads
        extra["a2a_tokens_to_heads"] = {"ms": ev2[0].elapsed_time(ev2[1]) / iters, "bytes": moved}
        extra["a2a_heads_to_tokens"] = {"ms": ev2[1].elapsed_time(ev2[2]) / iters, "bytes": moved}
        del x, y
    # Algorithmic FLOPs per launch (2*d per live pair per Q head per GEMM):
    # the forward's 2 GEMMs; the backward's 5 GEMMs split as dK/dV kernel =
    # S recompute, dP, dV, dK (4) and dQ kernel = dQ (1).  The dQ kernel also
    # recomputes S and dP (executed, not algorithmic).
    unit = 2 * wl.d * pairs * wl.hq
    return {
        "fwd_bf16_kernel": {"ms": ms[0], "ms_median": med[0], "flops": 2 * unit, "flops_executed": 2 * unit,
                            "o_dtype": "f32" if o_fwd is o32 else "bf16"},
        "dkdv_bf16_kernel": {"ms": ms[1], "ms_median": med[1], "flops": 4 * unit, "flops_executed": 4 * unit},
        "dq_bf16_kernel": {"ms": ms[2], "ms_median": med[2], "flops": 1 * unit, "flops_executed": 3 * unit},
        "merge_kernel": {"ms": ms[3], "ms_median": med[3], "bytes": rh * (3 * wl.d * 4 + 3 * 4)},
        # read O, dO (bf16), write Delta
        "delta_kernel": {"ms": ms[4], "ms_median": med[4], "bytes": rh * (2 * wl.d * 2 + 4)},
        **extra,
    }


# Source files each hot kernel is compiled from: a traffic figure measured
# with rocprofv3 counters is reported only while these are unchanged.
KERNEL_SOURCES = {
    "dkdv_bf16_kernel": ["attn_bwd_bf16.hip", "tile_io.h", "common.h", "kernels.h"],
    "dq_bf16_kernel": ["attn_bwd_bf16.hip", "tile_io.h", "common.h", "kernels.h"],
    "fwd_bf16_kernel": ["attn_fwd_bf16.hip", "tile_io.h", "common.h", "kernels.h"],
}


def kernel_source_hash(kernel):
    import hashlib
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        with open(os.path.join(ROOT, "sequence_context_parallelism_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def measured_traffic(kernel, workload):
    """HBM bytes per launch of `kernel` on `workload` from the committed
    counter summary profiles/traffic_<kernel>_<workload>.txt (FETCH_SIZE and
    WRITE_SIZE per dispatch, scaled by the same counters' reading for a plain
    copy of known size), or None if there is none or the kernel's sources have
    changed since it was taken."""
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel}_{workload}.txt")
    if not os.path.exists(path):
        return None
    kv = {}
    with open(path) as fh:
        for line in fh:
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                kv[key.strip()] = val.strip()
    if kv.get("source_sha256_16") != kernel_source_hash(kernel):
        return None
    return float(kv["hbm_bytes_per_launch"])


def sampled_parity(wl, torch):
    """Max error of O, LSE and dQ on 16 sampled rows of one query head vs the
    fp64 oracle (every sampled row exact over all its keys)."""
    from oracle import attention as A
    if wl.name != "ulysses_64k":
        return None
    rng = np.random.default_rng(0)
    rows = np.sort(rng.choice(wl.S, size=16, replace=False))
    heads = rng.integers(0, wl.hq, size=16)
    q = wl.q.float().cpu().numpy()
    k = wl.k.float().cpu().numpy()
    v = wl.v.float().cpu().numpy()
    do = wl.dout.float().cpu().numpy()
    pos = np.arange(wl.S)
    scale = 1.0 / math.sqrt(wl.d)
    o, lse = A.forward_rows(q, k, v, pos, pos, rows, heads, scale=scale, causal=True)
    dlt = np.einsum("ne,ne->n", o, do[rows, heads].astype(np.float64))
    dq = A.dq_rows(q, k, v, do, lse, dlt, pos, pos, rows, heads, scale=scale, causal=True)
    go = wl.o.float().cpu().numpy()[rows, heads]
    gl = wl.lse.cpu().numpy()[heads, rows]
    gdq = wl.dq.cpu().numpy()[rows, heads]
    return {"rows": 16, "o": float(np.abs(go - o).max()), "lse": float(np.abs(gl - lse).max()),
            "dq": float(np.abs(gdq - dq).max())}


def cpu_baseline(wl):
    """The oracle (untuned) on the host cores: forward + backward of one KV
    group (hq/hkv query heads sharing one KV head) over the first 16384 tokens
    of the causal sequence, in causal-FLOP TFLOPS."""
    import torch
    from oracle import attention as A
    L = 16384
    g = wl.hq // wl.hkv
    q = wl.q[:L, :g].float().cpu().numpy()
    k = wl.k[:L, :1].float().cpu().numpy()
    v = wl.v[:L, :1].float().cpu().numpy()
    do = wl.dout[:L, :g].float().cpu().numpy()
    pos = np.arange(L)
    scale = 1.0 / math.sqrt(wl.d)
    t0 = time.perf_counter()
    o, lse = A.forward(q, k, v, pos, pos, scale=scale, causal=True)
    A.backward(q, k, v, do, lse, A.delta(o, do), pos, pos, scale=scale, causal=True)
    t = time.perf_counter() - t0
    pairs = (L * (L + 1) // 2) * g
    flops = 14 * wl.d * pairs
    cores = len(os.sched_getaffinity(0))
    try:   # the threads the BLAS behind numpy actually ran with
        import threadpoolctl
        blas = [p["num_threads"] for p in threadpoolctl.threadpool_info() if p.get("user_api") == "blas"]
        if blas:
            cores = min(cores, max(blas))
    except Exception:
        pass
    model = cpu_model()
    return {"value": flops / t / 1e12, "unit": "TFLOPS", "cores": cores, "kind": "oracle",
            "sample": f"fp64 numpy oracle, forward+backward of one KV group ({g} query heads) over the "
                      f"first {L} tokens, causal; {t:.1f} s",
            "seconds": t, "pairs_per_s": pairs / t, "gflops_fp64": flops / t / 1e9, "cpu_model": model["name"],
            "cpu_id": model["id"], "cpu_logical_cpus": model["logical"],
            "torch_threads": torch.get_num_threads()}


def cpu_model():
    """The host CPU as /proc/cpuinfo names it, with its family/model/stepping
    numbers (some hosts report only a short marketing name)."""
    info = {}
    n = 0
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ":" not in ln:
                    continue
                key, val = (x.strip() for x in ln.split(":", 1))
                if key == "processor":
                    n += 1
                info.setdefault(key, val)
    except OSError:
        pass
    ident = " ".join(f"{k.replace('cpu ', '')} {info[k]}" for k in ("vendor_id", "cpu family", "model", "stepping")
                     if k in info)
    return {"name": info.get("model name", ""), "id": ident, "logical": n}


XGMI_LINK_GBS = 153.0   # one xGMI link, per direction (the ring's neighbour link)


def ring_overlap(wl, cp, torch, steps, ms_plain):
    """One ring rank's step with the ring's traffic emulated on a second
    stream (cp_ring_emulate_overlap): each ring step's KV shard arrives through
    a strided copy issued one step ahead, and in the backward each step's
    dK/dV shard leaves through a copy.  Reports the step time beside the plain
    one, the bytes one ring step moves, and what those bytes take over one
    xGMI link against the compute of one ring step."""
    ws = cp.workspace(cp.cp_ring_overlap_workspace_bytes(wl.sh, wl.S, wl.P, cp.CP_BF16, True))
    side = torch.cuda.Stream()

    def run():
        cp.cp_ring_emulate_overlap(wl.sh, wl.S, wl.P, 0, wl.q, wl.k, wl.v, None, wl.o, wl.lse, wl.dout,
                                   wl.dq, wl.dk, wl.dv, workspace=ws, copy_stream=side)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    n, kvrow = wl.S // wl.P, wl.hkv * wl.d
    kv_b = 2 * n * kvrow * 2          # K and V shard, bf16
    grad_b = 2 * n * kvrow * 4        # dK and dV shard, fp32
    ring_steps = 2 * (wl.P - 1)       # forward and backward steps that receive a shard
    return {"ms_per_step_plain": round(ms_plain, 4), "ms_per_step_with_traffic": round(ms, 4),
            "overhead_frac": round(ms / ms_plain - 1.0, 4),
            "bytes_per_ring_step_fwd": kv_b, "bytes_per_ring_step_bwd": kv_b + grad_b,
            "copies_per_step": ring_steps, "grad_sends_per_step": wl.P,
            "compute_ms_per_ring_step": round(ms_plain / (2 * wl.P), 4),
            "xgmi_link_ms_per_ring_step_bwd": round((kv_b + grad_b) / (XGMI_LINK_GBS * 1e9) * 1e3, 4)}


def allgather_share(wl, cp, torch, steps, ms_ring):
    """The same rank's share under all-gather context parallelism
    (cp_allgather_share): its two query runs against the whole gathered
    sequence in one forward and one backward call -- the same causal pairs as
    its ring share.  K/V here are random rows, so their order does not matter
    for the timing."""
    ws = cp.workspace(cp.cp_allgather_workspace_bytes(wl.sh, wl.S, wl.P, False, True))

    def run():
        cp.cp_allgather_share(wl.sh, wl.S, wl.P, 0, wl.q, wl.k, wl.v, None, wl.o, wl.lse, wl.dout, wl.dq,
                              wl.dk, wl.dv, workspace=ws)
    run()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        run()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = wl.flops_fwd + wl.flops_bwd
    return {"ms_per_step": round(ms, 4), "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "vs_ring_step": round(ms / ms_ring, 4)}


def gemm_ceiling(torch, n=16384, iters=10):
    """The MFMA throughput the vendor library reaches on this GPU: one large
    square bf16 GEMM (torch.matmul, i.e. hipBLASLt), timed with events.  Not
    part of the attention path; reported beside the roofline as the practical
    ceiling under sustained load, where the shader clock drops well below the
    2.4 GHz that the published 2.5 PFLOP/s assumes."""
    a = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    b = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    per = timed_steps(lambda: a @ b, torch, 3, iters)
    ms = float(np.median(per))
    tf = 2.0 * n ** 3 / (ms * 1e-3) / 1e12
    del a, b
    torch.cuda.empty_cache()
    return {"what": f"bf16 GEMM {n}x{n}x{n} via torch.matmul (hipBLASLt)", "ms_median": round(ms, 4),
            "tflops": round(tf, 1), "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4)}


def timed_steps(fn, torch, warmup, steps):
    """Per-step milliseconds of `steps` calls after `warmup`, each bracketed by
    events on the current stream."""
    st = torch.cuda.current_stream()
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record(st)
    for i in range(steps):
        fn()
        ev[i + 1].record(st)
    torch.cuda.synchronize()
    return [ev[i].elapsed_time(ev[i + 1]) for i in range(steps)]


def layout_rows(S, P, pairs):
    """Global row of every row of a sharded-order array when rank r holds
    chunks pairs[r] = (a, b): rank 0's two chunks first, then rank 1's."""
    c = S // (2 * P)
    return np.concatenate([np.arange(x * c, (x + 1) * c) for a, b in pairs for x in (a, b)])


def ring_balance_timing(wl, cp, torch, P=8, passes=2):
    """Per-rank time of a ring over the packed documents (forward +
    backward of each rank's share, every rank run in turn on this GPU), for
    the zigzag layout and for the document-balanced pairing of
    cp_balanced_pairs.  The ids are put in each layout's sharded order; the
    random Q/K/V rows need no reordering for timing."""
    S, hq, hkv, d = wl.S, wl.hq, wl.hkv, wl.d
    n = S // P
    doc_g = wl.doc.cpu().numpy()
    work = cp.cp_chunk_work(S, P, doc_g)
    zz = [(r, 2 * P - 1 - r) for r in range(P)]
    bal, _ = cp.cp_balanced_pairs(S, P, doc_g)
    bal = [tuple(int(x) for x in p) for p in bal]
    lse = torch.empty(hq, n, device=wl.dev)
    o, dq, dout = wl.o[:n], wl.dq[:n], wl.dout[:n]
    ws = cp.workspace(max(cp.cp_ring_workspace_bytes(wl.sh, S, P, r, cp.CP_BF16, True) for r in range(P)))
    res = {"P": P}
    for name, pairs in (("zigzag", zz), ("doc_balanced", bal)):
        doc = torch.from_numpy(np.ascontiguousarray(doc_g[layout_rows(S, P, pairs)])).to(wl.dev)
        rank_ms = []
        for r in range(P):
            def run(r=r):
                cp.cp_ring_emulate_layout(wl.sh, S, P, r, pairs, wl.q, wl.k, wl.v, doc, o, lse, dout, dq,
                                          wl.dk, wl.dv, workspace=ws)
            rank_ms.append(float(np.median(timed_steps(run, torch, 1, passes))))
        w = np.array([work[a] + work[b] for a, b in pairs], dtype=np.float64)
        t = np.array(rank_ms)
        res[name] = {"chunks": [list(p) for p in pairs], "rank_ms": [round(x, 3) for x in rank_ms],
                     "max_over_mean_ms": round(float(t.max() / t.mean()), 3),
                     "max_over_mean_work": round(float(w.max() / w.mean()), 3),
                     "busiest_rank_ms": round(float(t.max()), 3)}
    res["busiest_rank_speedup"] = round(res["zigzag"]["busiest_rank_ms"] / res["doc_balanced"]["busiest_rank_ms"], 3)
    return res


def other_workloads(head_wl, cp, torch, cpinputs, warmup=1, steps=2):
    """Short runs of the other workloads (ring rank of P=8 over 128K tokens,
    packed documents over 128K, the USP share over 1M tokens): warmup + steps
    calls each, per-step medians.  The packed-document entry also carries the
    per-rank ring timing of the zigzag and document-balanced layouts."""
    out = {}
    for name in ("ring_128k", "docs_128k", "usp_1m"):
        torch.cuda.empty_cache()
        wl = Workload(name, torch, cp, cpinputs)
        torch.cuda.synchronize()
        print(f"[bench] workload {name} ready", file=sys.stderr, flush=True)
        per = timed_steps(lambda: wl.step(cp), torch, warmup, steps)
        ms = float(np.median(per))
        flops = wl.flops_fwd + wl.flops_bwd
        tf = flops / (ms * 1e-3) / 1e12
        e = {"config": wl.config, "steps": steps, "warmup": warmup, "ms_per_step_median": round(ms, 3),
             "ms_per_step": [round(x, 3) for x in per], "tflops": round(tf, 1),
             "frac_of_peak": round(tf / PEAK_BF16_TFLOPS, 4),
             "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1),
             "tokens_per_s_per_gpu": round(wl.tokens / (ms * 1e-3) / wl.group, 1),
             "flops_per_step": flops}
        print(f"[bench] {name}: {ms:.2f} ms/step, {tf:.1f} TFLOPS", file=sys.stderr, flush=True)
        if name == "docs_128k":
            e["ring_balance"] = ring_balance_timing(wl, cp, torch)
            print(f"[bench] docs_128k ring balance: {e['ring_balance']['busiest_rank_speedup']}x on the busiest "
                  "rank", file=sys.stderr, flush=True)
        out[name] = e
        del wl
    torch.cuda.empty_cache()
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share; --gpus {args.gpus} is not supported "
              "(this build runs on a single GPU, with no collectives)", file=sys.stderr)
        sys.exit(2)
    import torch

    import cpinputs
    import sequence_context_parallelism_amd as cp

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    cp.load()
    if args.copy_calibration:
        n = 512 * 2**20 // 4
        src = torch.ones(n, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_each_way": n * 4, "launches": 3}), flush=True)
        return
    if args.gemm_ceiling:
        print(json.dumps({"measured_gemm_ceiling": gemm_ceiling(torch)}), flush=True)
        return
    wl = Workload(args.workload, torch, cp, cpinputs)
    torch.cuda.synchronize()
    print(f"[bench] workload {args.workload} ready", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        wl.step(cp)
    torch.cuda.synchronize()
    st = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    w0 = time.perf_counter()
    evs[0].record(st)
    for i in range(args.steps):
        wl.step(cp)
        evs[i + 1].record(st)
    torch.cuda.synchronize()
    wall = time.perf_counter() - w0
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    ms_med = float(np.median([evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]))
    print(f"[bench] timed {args.steps} steps: {ms:.3f} ms/step", file=sys.stderr, flush=True)
    parity = sampled_parity(wl, torch)

    flops = wl.flops_fwd + wl.flops_bwd
    tflops = flops / (ms * 1e-3) / 1e12
    out = {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOPS",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "ms_per_step_median": round(ms_med, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16", "data": "synthetic",
        "config": wl.config,
        "tokens_per_s": round(wl.tokens / (ms * 1e-3), 1),
        "tokens_per_s_per_gpu": round(wl.tokens / (ms * 1e-3) / wl.group, 1),
        "pct_mfma_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "flops_per_step": flops, "wall_s_timed": round(wall, 3),
        "max_memory_allocated_gib": round(torch.cuda.max_memory_allocated() / 2**30, 2),
    }
    if parity:
        out["parity_sample"] = parity
    if not args.no_kernel_timing:
        kt = kernel_times(wl, cp, torch, max(3, args.steps))
        out["kernels"] = {}
        for name, r in kt.items():
            e = {"ms": round(r["ms"], 4)}
            if "ms_median" in r:
                e["ms_median"] = round(r["ms_median"], 4)
            if "o_dtype" in r:
                e["o_dtype"] = r["o_dtype"]
            if "flops" in r:
                e["tflops"] = round(r["flops"] / (r["ms"] * 1e-3) / 1e12, 1)
                e["tflops_executed"] = round(r["flops_executed"] / (r["ms"] * 1e-3) / 1e12, 1)
            else:
                e["gb_s"] = round(r["bytes"] / (r["ms"] * 1e-3) / 1e9, 1)
                e["frac_hbm_8tbs"] = round(r["bytes"] / (r["ms"] * 1e-3) / 8e12, 3)
            out["kernels"][name] = e
        # forward-only and backward-only causal-FLOP throughput of the launches
        # timed alone (the backward's Delta pass, ~0.2 % of it, is not included)
        if all(n in kt for n in ("fwd_bf16_kernel", "dkdv_bf16_kernel", "dq_bf16_kernel")):
            bwd_ms = kt["dkdv_bf16_kernel"]["ms"] + kt["dq_bf16_kernel"]["ms"]
            bwd_flops = kt["dkdv_bf16_kernel"]["flops"] + kt["dq_bf16_kernel"]["flops"]
            out["forward_tflops"] = round(kt["fwd_bf16_kernel"]["flops"] / (kt["fwd_bf16_kernel"]["ms"] * 1e-3) / 1e12, 1)
            out["backward_tflops"] = round(bwd_flops / (bwd_ms * 1e-3) / 1e12, 1)
        dom = max((n for n in kt if "flops" in kt[n]), key=lambda n: kt[n]["ms"])
        ach = kt[dom]["flops"] / (kt[dom]["ms"] * 1e-3) / 1e12
        traffic = measured_traffic(dom, args.workload)
        ceiling = gemm_ceiling(torch)
        out["roofline"] = {"kernel": dom, "bound": "mfma", "achieved": round(ach, 1),
                           "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                           "frac": round(ach / PEAK_BF16_TFLOPS, 4),
                           "traffic": None if traffic is None else round(traffic),
                           "flops_per_launch": kt[dom]["flops"], "ms_per_launch": round(kt[dom]["ms"], 4),
                           "source_sha256_16": kernel_source_hash(dom),
                           "frac_of_measured_gemm": round(ach / ceiling["tflops"], 4),
                           "measured_gemm_ceiling": ceiling}
    if wl.name == "docs_128k":
        # rank balance of a ring over these documents (host integer work): the
        # zigzag layout vs the document-aware two-chunk pairing
        doc = wl.doc.cpu().numpy()
        bal = {}
        for P in (4, 8):
            w = cp.cp_chunk_work(wl.S, P, doc)
            zz = np.array([w[r] + w[2 * P - 1 - r] for r in range(P)])
            _, rw = cp.cp_balanced_pairs(wl.S, P, doc)
            bal[f"P{P}"] = {"zigzag_max_over_mean": round(float(zz.max() / zz.mean()), 3),
                            "doc_aware_max_over_mean": round(float(rw.max() / rw.mean()), 3)}
        out["ring_balance"] = bal
    if wl.name in ("ring_128k", "usp_1m"):
        out["ring_overlap"] = ring_overlap(wl, cp, torch, max(1, min(args.steps, 3)), ms)
    if wl.name == "ring_128k":
        out["allgather_share"] = allgather_share(wl, cp, torch, max(1, min(args.steps, 3)), ms)
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(wl)
    if args.workload == "ulysses_64k" and not args.no_workloads:
        out["workloads"] = other_workloads(wl, cp, torch, cpinputs)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
