"""GPU parity of the ring (P2P), Ulysses (A2A) and USP drivers against the
oracle's emulations: every ring step's partial, the merged result, and the
backward of one rank and of all ranks."""
import numpy as np
import pytest
import torch

import cpinputs
import sequence_context_parallelism_amd as cp
from gpu_util import TOL, grad_tol, host, inputs, lse_err, max_abs, shape_for, DEV
from oracle import attention as A
from oracle import schedule as Z

pytestmark = pytest.mark.gpu


def _ring_inputs(S, P, hq, hkv, d, dtype, seed, docs=False):
    (qh, kh, vh, doh), (qd, kd, vd, dod) = inputs(seed, [(S, hq, d), (S, hkv, d), (S, hkv, d), (S, hq, d)], dtype)
    doc = None
    if docs:
        lens = cpinputs.lognormal_doc_lengths(S, seed=seed, median=S // 6, sigma=1.0, lo=8, hi=S)
        doc = cpinputs.doc_ids_from_lengths(lens)[Z.sharded_order(S, P)]   # sharded order
    return (qh, kh, vh, doh), (qd, kd, vd, dod), doc


def test_tiny_ring_fp32_every_step(gpu_lib):
    """Tiny ring emulation: S=256, 4 Q / 2 KV heads, d=64, fp32, zigzag over
    P=2 ranks; each step's partial and the merged result vs the oracle."""
    S, P, hq, hkv, d = 256, 2, 4, 2, 64
    seed = cpinputs.SEEDS["tiny_ring"]
    hostg = cpinputs.normal_host(seed, [(S, hq, d), (S, hkv, d), (S, hkv, d)])
    order = Z.sharded_order(S, P)
    qh, kh, vh = (x[order].astype(np.float64) for x in hostg)     # inputs in sharded order
    qd, kd, vd = (torch.from_numpy(x.astype(np.float32)).to(DEV) for x in (qh, kh, vh))
    sh = shape_for(hq, hkv, d, torch.float32)
    n = S // P
    full_o, full_l = A.forward(hostg[0], hostg[1], hostg[2], np.arange(S), np.arange(S),
                               scale=sh.scale, causal=True)
    for r in range(P):
        o = torch.empty(n, hq, d, device=DEV)
        lse = torch.empty(hq, n, device=DEV)
        so = torch.empty(P, n, hq, d, device=DEV)
        sl = torch.empty(P, hq, n, device=DEV)
        ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, r, cp.CP_F32, False))
        cp.cp_ring_emulate(sh, S, P, r, qd, kd, vd, None, o, lse, step_o=so, step_lse=sl, workspace=ws)
        torch.cuda.synchronize()
        ro, rl, steps = Z.ring_forward(qh, kh, vh, S, P, r, scale=sh.scale)
        for s, (po, pl) in enumerate(steps):
            assert max_abs(host(so[s]), po) <= 1e-5, f"rank {r} step {s} O"
            assert lse_err(host(sl[s]), pl) <= 1e-6, f"rank {r} step {s} LSE"
        assert max_abs(host(o), ro) <= 1e-5
        assert lse_err(host(lse), rl) <= 1e-6
        rows = order[r * n:(r + 1) * n]                 # and the unsharded definition
        assert max_abs(host(o), full_o[rows]) <= 1e-5
        assert lse_err(host(lse), full_l[:, rows]) <= 1e-6


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("docs", [False, True], ids=["causal", "docs"])
def test_ring_forward_backward_one_rank(gpu_lib, dtype, docs, d):
    S, P, hq, hkv = 768, 3, 8, 2
    print(f"ring one rank {dtype} docs={docs} d={d}", flush=True)
    (qh, kh, vh, doh), (qd, kd, vd, dod), doc = _ring_inputs(S, P, hq, hkv, d, dtype, 7, docs)
    doc_d = None if doc is None else torch.from_numpy(doc).to(DEV)
    sh = shape_for(hq, hkv, d, dtype)
    n = S // P
    tol = TOL[dtype]
    for r in (0, P - 1):
        o = torch.empty(n, hq, d, device=DEV, dtype=dtype)
        lse = torch.empty(hq, n, device=DEV)
        dq = torch.empty(n, hq, d, device=DEV)
        dk = torch.empty(S, hkv, d, device=DEV)
        dv = torch.empty_like(dk)
        dout = dod[r * n:(r + 1) * n]
        ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, r, sh.dtype, True))
        cp.cp_ring_emulate(sh, S, P, r, qd, kd, vd, doc_d, o, lse, dout, dq, dk, dv, workspace=ws)
        torch.cuda.synchronize()
        ro, rl, _ = Z.ring_forward(qh, kh, vh, S, P, r, scale=sh.scale, doc=doc)
        assert max_abs(host(o), ro) <= tol["o"]
        assert lse_err(host(lse), rl) <= tol["lse"]
        rdq, rdk, rdv = Z.ring_backward(qh, kh, vh, doh[r * n:(r + 1) * n], ro, rl, S, P, r,
                                        scale=sh.scale, doc=doc)
        assert max_abs(host(dq), rdq) <= grad_tol(rdq, tol["grad"])
        assert max_abs(host(dk), rdk) <= grad_tol(rdk, tol["grad"])
        assert max_abs(host(dv), rdv) <= grad_tol(rdv, tol["grad"])


def test_ring_all_ranks_full_gradient(gpu_lib):
    S, P, hq, hkv, d = 1024, 4, 4, 2, 128
    dtype = torch.bfloat16
    (qh, kh, vh, doh), (qd, kd, vd, dod), _ = _ring_inputs(S, P, hq, hkv, d, dtype, 11)
    sh = shape_for(hq, hkv, d, dtype)
    n = S // P
    o = torch.empty(S, hq, d, device=DEV, dtype=dtype)
    lse = torch.empty(P, hq, n, device=DEV)
    dq = torch.empty(S, hq, d, device=DEV)
    dk = torch.empty(S, hkv, d, device=DEV)
    dv = torch.empty_like(dk)
    ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, -1, cp.CP_BF16, True))
    cp.cp_ring_emulate(sh, S, P, -1, qd, kd, vd, None, o, lse, dod, dq, dk, dv, workspace=ws)
    torch.cuda.synchronize()
    order = Z.sharded_order(S, P)
    inv = np.argsort(order)                              # sharded -> global
    pos = np.arange(S)
    qg, kg, vg, dog = qh[inv], kh[inv], vh[inv], doh[inv]
    ro, rl = A.forward(qg, kg, vg, pos, pos, scale=sh.scale, causal=True)
    rdq, rdk, rdv = A.backward(qg, kg, vg, dog, rl, A.delta(ro, dog), pos, pos, scale=sh.scale, causal=True)
    tol = TOL[dtype]
    assert max_abs(host(o), ro[order]) <= tol["o"]
    gl = host(lse).transpose(1, 0, 2).reshape(hq, S)      # [P, hq, n] -> [hq, S] sharded
    assert lse_err(gl, rl[:, order]) <= tol["lse"]
    assert max_abs(host(dq), rdq[order]) <= grad_tol(rdq, tol["grad"])
    assert max_abs(host(dk), rdk[order]) <= grad_tol(rdk, tol["grad"])
    assert max_abs(host(dv), rdv[order]) <= grad_tol(rdv, tol["grad"])


@pytest.mark.parametrize("d", [128, 64])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_ulysses_share_is_head_slice(gpu_lib, dtype, d):
    S, hq, hkv, sp = 640, 16, 4, 2
    (qh, kh, vh, _), (qd, kd, vd, _), _ = _ring_inputs(S, 1, hq, hkv, d, dtype, 21)
    sh = shape_for(hq, hkv, d, dtype)
    tol = TOL[dtype]
    for r in range(sp):
        hs, gs = hq // sp, hkv // sp
        (_, dosh), (_, dosd) = inputs(33 + r, [(1,), (S, hs, d)], dtype)
        nan = float("nan")   # outputs start as NaN: every row must be written
        o = torch.full((S, hs, d), nan, device=DEV, dtype=dtype)
        lse = torch.full((hs, S), nan, device=DEV)
        dq = torch.full((S, hs, d), nan, device=DEV)
        dk = torch.full((S, gs, d), nan, device=DEV)
        dv = torch.full_like(dk, nan)
        ws = cp.workspace(cp.cp_ulysses_workspace_bytes(sh, S, sp, True))
        cp.cp_ulysses_share(sh, S, sp, r, qd, kd, vd, None, o, lse, dosd, dq, dk, dv, workspace=ws)
        torch.cuda.synchronize()
        ro, rl = Z.ulysses_share(qh, kh, vh, sp, r, scale=sh.scale)
        assert max_abs(host(o), ro) <= tol["o"]
        assert lse_err(host(lse), rl) <= tol["lse"]
        (h0, h1), (g0, g1) = Z.head_slice(hq, hkv, sp, r)
        pos = np.arange(S)
        rdq, rdk, rdv = A.backward(qh[:, h0:h1], kh[:, g0:g1], vh[:, g0:g1], dosh, rl, A.delta(ro, dosh),
                                   pos, pos, scale=sh.scale, causal=True)
        assert max_abs(host(dq), rdq) <= grad_tol(rdq, tol["grad"])
        assert max_abs(host(dk), rdk) <= grad_tol(rdk, tol["grad"])
        assert max_abs(host(dv), rdv) <= grad_tol(rdv, tol["grad"])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("docs", [False, True], ids=["causal", "docs"])
def test_allgather_share_one_rank(gpu_lib, dtype, docs):
    """All-gather share of rank 1 of P=3 (S=768, 8/2 heads, d=128): O, LSE, dQ
    of its rows and its dK/dV contributions to every key, vs the oracle."""
    S, P, hq, hkv, d, r = 768, 3, 8, 2, 128, 1
    (qh, kh, vh, doh), (qd, kd, vd, dod) = inputs(3300 + docs, [(S, hq, d), (S, hkv, d), (S, hkv, d), (S, hq, d)], dtype)
    doc = None
    if docs:
        lens = cpinputs.lognormal_doc_lengths(S, seed=77, median=S // 5, sigma=1.0, lo=8, hi=S)
        doc = cpinputs.doc_ids_from_lengths(lens)
    rows = Z.rank_positions(S, P, r)
    sh = shape_for(hq, hkv, d, dtype)
    n = S // P
    q_r = qd[torch.as_tensor(rows, device=DEV)].contiguous()
    do_r = dod[torch.as_tensor(rows, device=DEV)].contiguous()
    nan = float("nan")   # outputs start as NaN: every row must be written
    o = torch.full((n, hq, d), nan, device=DEV, dtype=dtype)
    lse = torch.full((hq, n), nan, device=DEV)
    dq = torch.full((n, hq, d), nan, device=DEV)
    dk = torch.full((S, hkv, d), nan, device=DEV)
    dv = torch.full_like(dk, nan)
    doc_d = None if doc is None else torch.from_numpy(doc).to(DEV)
    ws = cp.workspace(cp.cp_allgather_workspace_bytes(sh, S, P, docs, True))
    cp.cp_allgather_share(sh, S, P, r, q_r, kd, vd, doc_d, o, lse, do_r, dq, dk, dv, workspace=ws)
    torch.cuda.synchronize()
    ro, rl, rdq, rdk, rdv = Z.allgather_share(qh[rows], kh, vh, S, P, r, scale=sh.scale, doc=doc, dout=doh[rows])
    tol = TOL[dtype]
    assert max_abs(host(o), ro) <= tol["o"]
    assert lse_err(host(lse), rl) <= tol["lse"]
    assert max_abs(host(dq), rdq) <= grad_tol(rdq, tol["grad"])
    assert max_abs(host(dk), rdk) <= grad_tol(rdk, tol["grad"])
    assert max_abs(host(dv), rdv) <= grad_tol(rdv, tol["grad"])


@pytest.mark.parametrize("dtype,P,docs", [(torch.bfloat16, 4, False), (torch.bfloat16, 4, True),
                                          (torch.float32, 4, False), (torch.bfloat16, 2, True),
                                          (torch.bfloat16, 1, False)],
                         ids=["bf16-P4", "bf16-P4-docs", "f32-P4", "bf16-P2-docs", "bf16-P1"])
def test_ring_overlap_matches_plain_bitwise(gpu_lib, dtype, P, docs):
    """The traffic emulation only moves where each step's KV shard is read
    from (a receive area filled on a second stream), so its outputs equal the
    plain driver's bit for bit; K/V are head slices of a wider layer, so the
    receive copy is a strided one.  Two calls in a row reuse the workspace.
    P = 1 has no transfers; P = 2 uses one of the two receive buffers."""
    S, hq, hkv, d = 1024, 4, 2, 128
    print(f"ring overlap {dtype} P={P} docs={docs}", flush=True)
    (_, _, _, _), (qd, kw, vw, dod), doc = _ring_inputs(S, P, hq, 2 * hkv, d, dtype, 21, docs)
    kd, vd = kw[:, hkv:], vw[:, hkv:]                    # the second half of the layer's KV heads
    doc_d = None if doc is None else torch.from_numpy(doc).to(DEV)
    sh = cp.make_shape(hq, hkv, d, hq * d, 2 * hkv * d, 1.0 / np.sqrt(d), True,
                       cp.CP_BF16 if dtype == torch.bfloat16 else cp.CP_F32)
    n = S // P
    side = torch.cuda.Stream()

    def outputs():
        return (torch.empty(n, hq, d, device=DEV, dtype=dtype), torch.empty(hq, n, device=DEV),
                torch.empty(n, hq, d, device=DEV), torch.empty(S, hkv, d, device=DEV),
                torch.empty(S, hkv, d, device=DEV))

    for r in (0, P - 1):
        dout = dod[r * n:(r + 1) * n]
        ref = outputs()
        ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, r, sh.dtype, True))
        cp.cp_ring_emulate(sh, S, P, r, qd, kd, vd, doc_d, ref[0], ref[1], dout, *ref[2:], workspace=ws)
        wso = cp.workspace(cp.cp_ring_overlap_workspace_bytes(sh, S, P, sh.dtype, True))
        for call in range(2):
            got = outputs()
            cp.cp_ring_emulate_overlap(sh, S, P, r, qd, kd, vd, doc_d, got[0], got[1], dout, *got[2:],
                                       workspace=wso, copy_stream=side)
            torch.cuda.synchronize()
            for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
                assert torch.equal(a, b), f"rank {r} call {call}: {name} differs"


def test_usp_mini_full(gpu_lib):
    """The USP structure (Ulysses 4 x ring 4) at S=8,192: the Ulysses rank-2
    head slice of a 16/4-head layer (4 query heads, 1 KV head, read in place
    through the strides) driven through the zigzag ring over all 4 ring
    ranks, checked in full against the oracle's attention over that slice --
    O, LSE, dQ and the complete dK, dV."""
    S, P, HQ, HKV, d, sp, u = 8192, 4, 16, 4, 128, 4, 2
    dtype = torch.bfloat16
    (h0, h1), (g0, g1) = Z.head_slice(HQ, HKV, sp, u)
    hq, hkv = h1 - h0, g1 - g0
    print(f"usp mini: heads {h0}:{h1}, kv {g0}:{g1}", flush=True)
    (qh, kh, vh), (qd, kd, vd) = inputs(41, [(S, HQ, d), (S, HKV, d), (S, HKV, d)], dtype)
    (doh,), (dod,) = inputs(42, [(S, hq, d)], dtype)
    order = Z.sharded_order(S, P)                         # global rows in sharded order
    order_d = torch.as_tensor(order, device=DEV)
    qs_d, ks_d, vs_d, dos_d = qd[order_d], kd[order_d], vd[order_d], dod[order_d]
    sh = cp.make_shape(hq, hkv, d, HQ * d, HKV * d, 1.0 / np.sqrt(d), True, cp.CP_BF16)
    n = S // P
    o = torch.empty(S, hq, d, device=DEV, dtype=dtype)
    lse = torch.empty(P, hq, n, device=DEV)
    dq = torch.empty(S, hq, d, device=DEV)
    dk = torch.empty(S, hkv, d, device=DEV)
    dv = torch.empty_like(dk)
    ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, -1, cp.CP_BF16, True))
    cp.cp_ring_emulate(sh, S, P, -1, qs_d[:, h0:h1], ks_d[:, g0:g1], vs_d[:, g0:g1], None, o, lse, dos_d,
                       dq, dk, dv, workspace=ws)
    torch.cuda.synchronize()
    pos = np.arange(S)
    q1, k1, v1 = qh[:, h0:h1], kh[:, g0:g1], vh[:, g0:g1]
    ro, rl = A.forward(q1, k1, v1, pos, pos, scale=sh.scale, causal=True)
    rdq, rdk, rdv = A.backward(q1, k1, v1, doh, rl, A.delta(ro, doh), pos, pos, scale=sh.scale, causal=True)
    tol = TOL[dtype]
    assert max_abs(host(o), ro[order]) <= tol["o"]
    gl = host(lse).transpose(1, 0, 2).reshape(hq, S)
    assert lse_err(gl, rl[:, order]) <= tol["lse"]
    assert max_abs(host(dq), rdq[order]) <= grad_tol(rdq, tol["grad"])
    assert max_abs(host(dk), rdk[order]) <= grad_tol(rdk, tol["grad"])
    assert max_abs(host(dv), rdv[order]) <= grad_tol(rdv, tol["grad"])


def test_ring_single_rank_is_plain_causal_attention(gpu_lib):
    """P = 1: one rank holds chunks 0 and 1, i.e. the whole sequence in order,
    and its one step is plain causal attention (forward and backward)."""
    S, P, hq, hkv, d = 512, 1, 4, 2, 128
    dtype = torch.bfloat16
    (qh, kh, vh, doh), (qd, kd, vd, dod), _ = _ring_inputs(S, P, hq, hkv, d, dtype, 5)
    sh = shape_for(hq, hkv, d, dtype)
    nan = float("nan")
    o = torch.full((S, hq, d), nan, device=DEV, dtype=dtype)
    lse = torch.full((hq, S), nan, device=DEV)
    dq = torch.full((S, hq, d), nan, device=DEV)
    dk = torch.full((S, hkv, d), nan, device=DEV)
    dv = torch.full_like(dk, nan)
    ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, 0, sh.dtype, True))
    cp.cp_ring_emulate(sh, S, P, 0, qd, kd, vd, None, o, lse, dod, dq, dk, dv, workspace=ws)
    torch.cuda.synchronize()
    pos = np.arange(S)
    ro, rl = A.forward(qh, kh, vh, pos, pos, scale=sh.scale, causal=True)
    rdq, rdk, rdv = A.backward(qh, kh, vh, doh, rl, A.delta(ro, doh), pos, pos, scale=sh.scale, causal=True)
    tol = TOL[dtype]
    assert max_abs(host(o), ro) <= tol["o"]
    assert lse_err(host(lse), rl) <= tol["lse"]
    assert max_abs(host(dq), rdq) <= grad_tol(rdq, tol["grad"])
    assert max_abs(host(dk), rdk) <= grad_tol(rdk, tol["grad"])
    assert max_abs(host(dv), rdv) <= grad_tol(rdv, tol["grad"])


def _layout_case(S, P, seed):
    """Packed documents and the document-balanced pairing of their chunks."""
    lens = cpinputs.lognormal_doc_lengths(S, seed=seed, median=S // 10, sigma=1.0, lo=8, hi=S)
    doc_g = cpinputs.doc_ids_from_lengths(lens)
    pairs, _ = cp.cp_balanced_pairs(S, P, doc_g)
    return doc_g, [tuple(int(x) for x in p) for p in pairs]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("layout", ["balanced", "fixed"])
def test_ring_layout_one_rank_matches_oracle(gpu_lib, dtype, layout):
    """The ring under a non-zigzag two-chunk layout (the document-balanced
    pairing of cp_balanced_pairs, or a fixed table): one rank's O, LSE, dQ and
    dK/dV contributions against the oracle's ring over the same layout."""
    S, P, hq, hkv, d = 1536, 4, 8, 2, 128
    doc_g, chunks = _layout_case(S, P, 91)
    if layout == "fixed":
        chunks = [(0, 1), (2, 5), (3, 4), (6, 7)]
    zz = [(r, 2 * P - 1 - r) for r in range(P)]
    assert sorted(chunks) != sorted(zz), "the case must differ from zigzag"
    order = Z.sharded_order(S, P, chunks)
    doc = doc_g[order]                                    # ids in this layout's sharded order
    print(f"ring layout {layout} {dtype}: chunks {chunks}", flush=True)
    (qh, kh, vh, doh), (qd, kd, vd, dod) = inputs(4400, [(S, hq, d), (S, hkv, d), (S, hkv, d), (S, hq, d)], dtype)
    doc_d = torch.from_numpy(doc).to(DEV)
    sh = shape_for(hq, hkv, d, dtype)
    n = S // P
    tol = TOL[dtype]
    for r in (0, P - 1):
        nan = float("nan")
        o = torch.full((n, hq, d), nan, device=DEV, dtype=dtype)
        lse = torch.full((hq, n), nan, device=DEV)
        dq = torch.full((n, hq, d), nan, device=DEV)
        dk = torch.full((S, hkv, d), nan, device=DEV)
        dv = torch.full_like(dk, nan)
        dout = dod[r * n:(r + 1) * n]
        ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, r, sh.dtype, True))
        cp.cp_ring_emulate_layout(sh, S, P, r, chunks, qd, kd, vd, doc_d, o, lse, dout, dq, dk, dv, workspace=ws)
        torch.cuda.synchronize()
        ro, rl, _ = Z.ring_forward(qh, kh, vh, S, P, r, scale=sh.scale, doc=doc, chunks=chunks)
        assert max_abs(host(o), ro) <= tol["o"]
        assert lse_err(host(lse), rl) <= tol["lse"]
        rdq, rdk, rdv = Z.ring_backward(qh, kh, vh, doh[r * n:(r + 1) * n], ro, rl, S, P, r,
                                        scale=sh.scale, doc=doc, chunks=chunks)
        assert max_abs(host(dq), rdq) <= grad_tol(rdq, tol["grad"])
        assert max_abs(host(dk), rdk) <= grad_tol(rdk, tol["grad"])
        assert max_abs(host(dv), rdv) <= grad_tol(rdv, tol["grad"])


def test_ring_balanced_layout_all_ranks_is_full_attention(gpu_lib):
    """Every rank of the document-balanced ring together: the outputs, in
    that layout's sharded order, equal plain document-masked causal
    attention over the sequence, and dK/dV are the full gradients."""
    S, P, hq, hkv, d = 2048, 4, 4, 2, 128
    dtype = torch.bfloat16
    doc_g, chunks = _layout_case(S, P, 93)
    order = Z.sharded_order(S, P, chunks)
    print(f"ring balanced all ranks: chunks {chunks}", flush=True)
    (qg, kg, vg, dog), _ = inputs(4500, [(S, hq, d), (S, hkv, d), (S, hkv, d), (S, hq, d)], dtype)
    qd, kd, vd, dod = (torch.from_numpy(x[order].astype(np.float32)).to(DEV).to(dtype) for x in (qg, kg, vg, dog))
    doc_d = torch.from_numpy(doc_g[order]).to(DEV)
    sh = shape_for(hq, hkv, d, dtype)
    n = S // P
    o = torch.empty(S, hq, d, device=DEV, dtype=dtype)
    lse = torch.empty(P, hq, n, device=DEV)
    dq = torch.empty(S, hq, d, device=DEV)
    dk = torch.empty(S, hkv, d, device=DEV)
    dv = torch.empty_like(dk)
    ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, -1, cp.CP_BF16, True))
    cp.cp_ring_emulate_layout(sh, S, P, -1, chunks, qd, kd, vd, doc_d, o, lse, dod, dq, dk, dv, workspace=ws)
    torch.cuda.synchronize()
    pos = np.arange(S)
    ro, rl = A.forward(qg, kg, vg, pos, pos, scale=sh.scale, causal=True, qdoc=doc_g, kdoc=doc_g)
    rdq, rdk, rdv = A.backward(qg, kg, vg, dog, rl, A.delta(ro, dog), pos, pos, scale=sh.scale, causal=True,
                               qdoc=doc_g, kdoc=doc_g)
    tol = TOL[dtype]
    assert max_abs(host(o), ro[order]) <= tol["o"]
    gl = host(lse).transpose(1, 0, 2).reshape(hq, S)
    assert lse_err(gl, rl[:, order]) <= tol["lse"]
    assert max_abs(host(dq), rdq[order]) <= grad_tol(rdq, tol["grad"])
    assert max_abs(host(dk), rdk[order]) <= grad_tol(rdk, tol["grad"])
    assert max_abs(host(dv), rdv[order]) <= grad_tol(rdv, tol["grad"])
