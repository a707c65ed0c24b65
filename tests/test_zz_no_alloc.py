"""cp_ulysses_share_noalloc -- the Ulysses share for callers that cannot
allocate device memory -- against cp_ulysses_share (the same kernels with a
caller workspace) and the oracle.  Two calls in a row on the same GPU, the
second with a smaller share, so the built-in scratch is reused with
different sizes; the results must equal the workspace entry point's bit for
bit and meet the oracle tolerances."""
import numpy as np
import pytest
import torch

import sequence_context_parallelism_amd as cp
from gpu_util import DEV, TOL, grad_tol, host, inputs, lse_err, max_abs, shape_for
from oracle import attention as A
from oracle import schedule as Z

pytestmark = pytest.mark.gpu

CASES = [   # (S, layer hq, layer hkv, d, dtype, sp, rank, docs): second smaller than the first
    (4096, 16, 4, 128, torch.bfloat16, 2, 1, False),
    (1536, 8, 2, 64, torch.bfloat16, 1, 0, True),
    (512, 8, 4, 128, torch.float32, 2, 0, False),
]


def _outputs(S, hq, hkv, d, dtype):
    nan = float("nan")
    return (torch.full((S, hq, d), nan, device=DEV, dtype=dtype), torch.full((hq, S), nan, device=DEV),
            torch.full((S, hq, d), nan, device=DEV), torch.full((S, hkv, d), nan, device=DEV),
            torch.full((S, hkv, d), nan, device=DEV))


def test_noalloc_equals_workspace_entry_point(gpu_lib):
    for i, (S, HQ, HKV, d, dtype, sp, r, docs) in enumerate(CASES):
        print(f"noalloc call {i}: S={S} heads {HQ}/{HKV} d={d} {dtype} sp={sp} rank={r} docs={docs}", flush=True)
        (qh, kh, vh), (qd, kd, vd) = inputs(900 + i, [(S, HQ, d), (S, HKV, d), (S, HKV, d)], dtype)
        hq, hkv = HQ // sp, HKV // sp
        (doh,), (dod,) = inputs(950 + i, [(S, hq, d)], dtype)
        doc = None
        if docs:
            doc = np.repeat(np.arange(3, dtype=np.int32), [S // 3, S // 3, S - 2 * (S // 3)])
        doc_d = None if doc is None else torch.from_numpy(doc).to(DEV)
        sh = shape_for(HQ, HKV, d, dtype)
        ref = _outputs(S, hq, hkv, d, dtype)
        ws = cp.workspace(cp.cp_ulysses_workspace_bytes(sh, S, sp, True))
        cp.cp_ulysses_share(sh, S, sp, r, qd, kd, vd, doc_d, ref[0], ref[1], dod, *ref[2:], workspace=ws)
        got = _outputs(S, hq, hkv, d, dtype)
        cp.cp_ulysses_share_noalloc(sh, S, sp, r, qd, kd, vd, doc_d, got[0], got[1], dod, *got[2:])
        torch.cuda.synchronize()
        for name, a, b in zip(("o", "lse", "dq", "dk", "dv"), got, ref):
            assert torch.equal(a, b), f"call {i}: {name} differs from cp_ulysses_share"
        # and the oracle's values for the share
        (h0, h1), (g0, g1) = Z.head_slice(HQ, HKV, sp, r)
        pos = np.arange(S)
        ro, rl = A.forward(qh[:, h0:h1], kh[:, g0:g1], vh[:, g0:g1], pos, pos, scale=sh.scale, causal=True,
                           qdoc=doc, kdoc=doc)
        rdq, rdk, rdv = A.backward(qh[:, h0:h1], kh[:, g0:g1], vh[:, g0:g1], doh, rl, A.delta(ro, doh), pos, pos,
                                   scale=sh.scale, causal=True, qdoc=doc, kdoc=doc)
        tol = TOL[dtype]
        assert max_abs(host(got[0]), ro) <= tol["o"]
        assert lse_err(host(got[1]), rl) <= tol["lse"]
        assert max_abs(host(got[2]), rdq) <= grad_tol(rdq, tol["grad"])
        assert max_abs(host(got[3]), rdk) <= grad_tol(rdk, tol["grad"])
        assert max_abs(host(got[4]), rdv) <= grad_tol(rdv, tol["grad"])


def test_noalloc_forward_only_and_oversize_refused(gpu_lib):
    S, HQ, HKV, d = 1024, 8, 2, 128
    (_, _, _), (qd, kd, vd) = inputs(990, [(S, HQ, d), (S, HKV, d), (S, HKV, d)], torch.bfloat16)
    sh = shape_for(HQ, HKV, d, torch.bfloat16)
    o = torch.empty(S, HQ, d, device=DEV, dtype=torch.bfloat16)
    lse = torch.empty(HQ, S, device=DEV)
    cp.cp_ulysses_share_noalloc(sh, S, 1, 0, qd, kd, vd, None, o, lse)        # no backward: no scratch use
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    cp.cp_ulysses_share(sh, S, 1, 0, qd, kd, vd, None, o2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)
