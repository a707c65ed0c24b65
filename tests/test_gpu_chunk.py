"""GPU parity of the chunk kernels against the fp64 oracle, through the C ABI:
forward (bf16 MFMA and fp32 paths), merge, delta, backward, tile map and an
end-to-end mask probe.  Shapes span several tiles and end in ragged tails."""
import numpy as np
import pytest
import torch

import sequence_context_parallelism_amd as cp
from gpu_util import (TOL, grad_tol, host, inputs, lse_err, max_abs, run_positions, shape_for,
                      to_dev, DEV)
from oracle import attention as A

pytestmark = pytest.mark.gpu

# (name, hq, hkv, d, q runs, k runs, causal, docs)
CASES = [
    ("causal_g4_ragged", 8, 2, 128, (0, 200), (0, 200), True, False),
    ("noncausal_g1_d64", 4, 4, 64, (0, 70), (0, 333), False, False),
    ("two_runs_g2", 4, 2, 128, (0, 96, 288, 96), (96, 96, 192, 96), True, False),
    ("docs_g8", 8, 1, 128, (0, 300), (0, 300), True, True),
    ("offset_rows_empty", 4, 2, 64, (10, 50), (40, 130), True, False),
    ("docs_two_runs_d64", 4, 2, 64, (0, 64, 192, 64), (0, 128, 128, 128), True, True),
    ("three_kv_heads", 12, 3, 64, (0, 150), (0, 150), True, False),     # groups not dividing 8
    ("sixteen_kv_heads", 64, 16, 64, (0, 70), (0, 70), True, False),    # groups a multiple of 8
    ("tiny_5x7", 4, 2, 128, (2, 5), (0, 7), True, False),               # one partial tile each way
    ("mqa_g16", 16, 1, 128, (0, 150), (0, 150), True, False),           # 16 query heads on one KV head
    ("one_row_half_one_key_block", 4, 1, 128, (0, 33), (0, 129), False, False),   # 2nd query half: 1 row
    ("all_rows_empty", 4, 2, 128, (0, 40), (100, 64), True, False),   # every key after every query
    ("no_keys", 4, 2, 64, (0, 70), (0, 0), True, False),              # empty key span
    ("causal_g1_nine_key_tiles", 2, 2, 128, (0, 1100), (0, 1100), True, False),   # partner key tiles, odd count
    ("causal_eight_kv_heads", 16, 8, 64, (0, 900), (0, 900), True, False),        # one KV head per XCD
]


def _runs(spec):
    return spec if len(spec) == 4 else (spec[0], spec[1], 0, 0)


def _docs(total_pos, seed):
    rng = np.random.default_rng(seed)
    cuts = np.sort(rng.choice(np.arange(1, total_pos), size=5, replace=False))
    return np.searchsorted(cuts, np.arange(total_pos), side="right").astype(np.int32)


def _setup(case, dtype, seed=0):
    name, hq, hkv, d, qr, kr, causal, docs = case
    qr, kr = _runs(qr), _runs(kr)
    qpos = run_positions(*qr)
    kpos = run_positions(*kr)
    Lq, Lk = len(qpos), len(kpos)
    (qh, kh, vh, doh), (qd, kd, vd, dod) = inputs(
        1000 + seed, [(Lq, hq, d), (Lk, hkv, d), (Lk, hkv, d), (Lq, hq, d)], dtype)
    qdoc = kdoc = None
    qdoc_d = kdoc_d = None
    if docs:
        allpos = _docs(int(max(qpos.max(), kpos.max())) + 1, seed)
        qdoc, kdoc = allpos[qpos], allpos[kpos]
        qdoc_d = torch.from_numpy(qdoc).to(DEV)
        kdoc_d = torch.from_numpy(kdoc).to(DEV)
    sh = shape_for(hq, hkv, d, dtype, causal)
    qs = cp.make_span(qr[0], qr[1], qr[2], qr[3], qdoc_d)
    ks = cp.make_span(kr[0], kr[1], kr[2], kr[3], kdoc_d)
    return dict(sh=sh, qs=qs, ks=ks, qh=qh, kh=kh, vh=vh, doh=doh, qd=qd, kd=kd, vd=vd, dod=dod,
                qpos=qpos, kpos=kpos, qdoc=qdoc, kdoc=kdoc, hq=hq, hkv=hkv, d=d, causal=causal,
                keep=(qdoc_d, kdoc_d))


def _gpu_fwd(c, o_dtype):
    Lq = len(c["qpos"])
    o = torch.empty(Lq, c["hq"], c["d"], device=DEV, dtype=o_dtype)
    lse = torch.empty(c["hq"], Lq, device=DEV, dtype=torch.float32)
    cp.cp_attn_chunk_fwd(c["sh"], c["qd"], c["qs"], c["kd"], c["vd"], c["ks"], o, lse)
    torch.cuda.synchronize()
    return o, lse


def _oracle_fwd(c):
    return A.forward(c["qh"], c["kh"], c["vh"], c["qpos"], c["kpos"], scale=c["sh"].scale,
                     causal=c["causal"], qdoc=c["qdoc"], kdoc=c["kdoc"])


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunk_forward_parity(gpu_lib, case, dtype):
    print(f"case {case[0]} {dtype}", flush=True)
    c = _setup(case, dtype)
    o, lse = _gpu_fwd(c, torch.float32)
    ro, rl = _oracle_fwd(c)
    tol = TOL[dtype]
    assert max_abs(host(o), ro) <= tol["o"]
    assert lse_err(host(lse), rl) <= tol["lse"]
    if dtype == torch.bfloat16:   # final bf16 output: the same up to one bf16 rounding
        ob, _ = _gpu_fwd(c, torch.bfloat16)
        assert max_abs(host(ob), ro) <= tol["o"]


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
@pytest.mark.parametrize("case", CASES, ids=[c[0] for c in CASES])
def test_chunk_backward_parity(gpu_lib, case, dtype):
    print(f"case {case[0]} {dtype}", flush=True)
    c = _setup(case, dtype, seed=1)
    Lq, Lk = len(c["qpos"]), len(c["kpos"])
    o, lse = _gpu_fwd(c, dtype)
    delta = torch.empty(c["hq"], Lq, device=DEV, dtype=torch.float32)
    cp.cp_attn_delta(o, c["dod"], delta)
    dq = torch.zeros(Lq, c["hq"], c["d"], device=DEV)
    dk = torch.zeros(Lk, c["hkv"], c["d"], device=DEV)
    dv = torch.zeros_like(dk)
    cp.cp_attn_chunk_bwd(c["sh"], c["qd"], c["qs"], c["kd"], c["vd"], c["ks"], c["dod"], lse, delta,
                         dq, dk, dv)
    torch.cuda.synchronize()
    ro, rl = _oracle_fwd(c)
    rdq, rdk, rdv = A.backward(c["qh"], c["kh"], c["vh"], c["doh"], rl, A.delta(ro, c["doh"]),
                               c["qpos"], c["kpos"], scale=c["sh"].scale, causal=c["causal"],
                               qdoc=c["qdoc"], kdoc=c["kdoc"])
    tol = TOL[dtype]["grad"]
    assert max_abs(host(delta), A.delta(ro, c["doh"])) <= grad_tol(A.delta(ro, c["doh"]), tol)
    assert max_abs(host(dq), rdq) <= grad_tol(rdq, tol)
    assert max_abs(host(dk), rdk) <= grad_tol(rdk, tol)
    assert max_abs(host(dv), rdv) <= grad_tol(rdv, tol)


@pytest.mark.parametrize("d", [64, 128])
def test_merge_parity_and_empty_identity(gpu_lib, d):
    rows, h = 77, 6
    rng = np.random.default_rng(d)
    oa = rng.standard_normal((rows, h, d)).astype(np.float32)
    ob = rng.standard_normal((rows, h, d)).astype(np.float32)
    la = rng.normal(3, 2, (h, rows)).astype(np.float32)
    lb = rng.normal(3, 2, (h, rows)).astype(np.float32)
    la[0, :10] = -np.inf              # acc empty
    lb[1, :10] = -np.inf              # part empty
    la[2, :5] = -np.inf
    lb[2, :5] = -np.inf               # both empty
    oa[:10, 0] = 0
    ob[:10, 1] = 0
    oa[:5, 2] = 0
    ob[:5, 2] = 0
    ro, rl = A.merge(oa, la, ob, lb)
    to, tl = (torch.from_numpy(x).to(DEV) for x in (oa, la))
    po, pl = (torch.from_numpy(x).to(DEV) for x in (ob, lb))
    cp.cp_lse_merge(to, tl, po, pl)
    torch.cuda.synchronize()
    go, gl = to.cpu().numpy(), tl.cpu().numpy()
    assert lse_err(gl, rl) <= 1e-6
    assert max_abs(go, ro) <= 1e-5
    # -inf is the identity, bit for bit
    assert np.array_equal(go[:10, 0], ob[:10, 0]) and np.array_equal(gl[0, :10], lb[0, :10])
    assert np.array_equal(go[:10, 1], oa[:10, 1]) and np.array_equal(gl[1, :10], la[1, :10])
    assert np.all(go[:5, 2] == 0) and np.all(np.isneginf(gl[2, :5]))


TILE_CASES = [
    ((0, 300), (0, 300), True, True, 64, 64),
    ((0, 96, 288, 96), (96, 96, 192, 96), True, False, 64, 128),
    ((0, 100, 250, 37), (0, 200, 300, 90), True, True, 32, 48),
    ((5, 77), (0, 123), False, True, 16, 16),
]


@pytest.mark.parametrize("qr,kr,causal,docs,bq,bk", TILE_CASES)
def test_tile_map_bit_exact(gpu_lib, qr, kr, causal, docs, bq, bk):
    qr, kr = _runs(qr), _runs(kr)
    qpos, kpos = run_positions(*qr), run_positions(*kr)
    qdoc = kdoc = None
    qdd = kdd = None
    if docs:
        allpos = _docs(int(max(qpos.max(), kpos.max())) + 1, 3)
        qdoc, kdoc = allpos[qpos], allpos[kpos]
        qdd, kdd = torch.from_numpy(qdoc).to(DEV), torch.from_numpy(kdoc).to(DEV)
    want = A.tile_classes(qpos, kpos, causal, bq, bk, qdoc, kdoc)
    out = torch.full(want.shape, -1, dtype=torch.int8, device=DEV)
    sh = shape_for(4, 2, 128, torch.bfloat16, causal)
    cp.cp_tile_map(sh, cp.make_span(*qr, qdd), cp.make_span(*kr, kdd), bq, bk, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), want)


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32], ids=["bf16", "f32"])
def test_mask_probe_recovers_mask_exactly(gpu_lib, dtype):
    """Q = 0 and V_j = one-hot(j): every allowed score is 0, so O_i * |J_i|
    is row i of the mask and exp(LSE_i) = |J_i|.  Checks the kernel's masking
    (causal, documents, two runs, ragged tiles) entry by entry."""
    qr, kr = (0, 40, 100, 50), (20, 60, 90, 40)
    qpos, kpos = run_positions(*qr), run_positions(*kr)
    Lq, Lk, d = len(qpos), len(kpos), 128
    allpos = _docs(200, 9)
    qdoc, kdoc = allpos[qpos], allpos[kpos]
    mask = A.allowed_mask(qpos, kpos, True, qdoc, kdoc)
    q = torch.zeros(Lq, 2, d, device=DEV, dtype=dtype)
    k = torch.randn(Lk, 1, d, device=DEV).to(dtype)
    v = torch.zeros(Lk, 1, d, device=DEV, dtype=dtype)
    v[torch.arange(Lk), 0, torch.arange(Lk)] = 1
    o = torch.empty(Lq, 2, d, device=DEV)
    lse = torch.empty(2, Lq, device=DEV)
    sh = shape_for(2, 1, d, dtype, True)
    qdd, kdd = torch.from_numpy(qdoc).to(DEV), torch.from_numpy(kdoc).to(DEV)
    cp.cp_attn_chunk_fwd(sh, q, cp.make_span(*qr, qdd), k, v, cp.make_span(*kr, kdd), o, lse)
    torch.cuda.synchronize()
    cnt = mask.sum(axis=1)
    on = o.cpu().numpy()
    ln = lse.cpu().numpy()
    for h in range(2):
        rec = np.rint(on[:, h, :Lk] * np.maximum(cnt, 1)[:, None]).astype(int)
        assert np.array_equal(rec.astype(bool), mask)
        live = cnt > 0
        assert np.array_equal(np.rint(np.exp(ln[h, live])).astype(int), cnt[live])
        assert np.all(np.isneginf(ln[h, ~live]))


def test_backward_deterministic_and_split_equals_combined(gpu_lib):
    """The backward uses no atomics: two runs are bitwise identical, and the
    dK/dV and dQ halves called separately give the same bits as the whole."""
    c = _setup(CASES[0], torch.bfloat16, seed=4)
    Lq, Lk = len(c["qpos"]), len(c["kpos"])
    o, lse = _gpu_fwd(c, torch.bfloat16)
    delta = torch.empty(c["hq"], Lq, device=DEV)
    cp.cp_attn_delta(o, c["dod"], delta)
    outs = []
    for _ in range(2):
        dq = torch.zeros(Lq, c["hq"], c["d"], device=DEV)
        dk = torch.zeros(Lk, c["hkv"], c["d"], device=DEV)
        dv = torch.zeros_like(dk)
        cp.cp_attn_chunk_bwd(c["sh"], c["qd"], c["qs"], c["kd"], c["vd"], c["ks"], c["dod"], lse, delta,
                             dq, dk, dv)
        outs.append((dq, dk, dv))
    dq = torch.zeros(Lq, c["hq"], c["d"], device=DEV)
    dk = torch.zeros(Lk, c["hkv"], c["d"], device=DEV)
    dv = torch.zeros_like(dk)
    cp.cp_attn_chunk_bwd_dkdv(c["sh"], c["qd"], c["qs"], c["kd"], c["vd"], c["ks"], c["dod"], lse, delta, dk, dv)
    cp.cp_attn_chunk_bwd_dq(c["sh"], c["qd"], c["qs"], c["kd"], c["vd"], c["ks"], c["dod"], lse, delta, dq)
    outs.append((dq, dk, dv))
    torch.cuda.synchronize()
    for x, y in zip(outs[0], outs[1]):
        assert torch.equal(x, y)
    for x, y in zip(outs[0], outs[2]):
        assert torch.equal(x, y)


@pytest.mark.parametrize("causal", [True, False])
def test_forward_exact_fallback_on_growing_scores(gpu_lib, causal):
    """Scores that rise by ~100 (natural-log units) along the keys: the first
    tile's max is far below later scores, the row sums pass 2^64 and the
    kernel must redo the rows with the exact online softmax."""
    L, hq, hkv, d = 256, 4, 2, 128
    rng = np.random.default_rng(17)
    beta = np.linspace(0.0, 10.0, L).astype(np.float32)          # grows along the keys
    qh = np.ones((L, hq, d), np.float32)
    kh = np.repeat(beta[:, None, None], hkv, axis=1) * np.ones((1, 1, d), np.float32)
    vh = rng.standard_normal((L, hkv, d)).astype(np.float32)
    q, k, v = (to_dev(x, torch.bfloat16) for x in (qh, kh, vh))
    qx, kx, vx = (t.to(torch.float64).cpu().numpy() for t in (q, k, v))   # exact bf16 values
    pos = np.arange(L)
    ro, rl = A.forward(qx, kx, vx, pos, pos, scale=1 / np.sqrt(d), causal=causal)
    sh = shape_for(hq, hkv, d, torch.bfloat16, causal)
    o = torch.empty(L, hq, d, device=DEV)
    lse = torch.empty(hq, L, device=DEV)
    cp.cp_attn_chunk_fwd(sh, q, cp.make_span(0, L), k, v, cp.make_span(0, L), o, lse)
    torch.cuda.synchronize()
    assert np.all(np.isfinite(host(o)))
    assert max_abs(host(o), ro) <= 2e-2
    assert lse_err(host(lse), rl) <= 1e-3
