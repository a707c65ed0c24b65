"""Document-id validation at the boundary (siliconandsystems.com, "Llama 3
parallelism", section "네 병렬화는 서로 다른 자원을 확보하는 방식": packed
documents must keep their mask under context parallelism).  With CP_CHECK_DOCS
set, every entry point that takes ids refuses negative or decreasing ones with
CP_ERR_DOCS before enqueueing anything: the outputs keep the NaN they were
filled with.  Valid ids pass and give the same result as an unchecked call."""
import numpy as np
import pytest
import torch

import sequence_context_parallelism_amd as cp
from gpu_util import DEV, inputs, shape_for

pytestmark = pytest.mark.gpu

BAD = {"negative": lambda d: _set(d, 70, -3), "decreasing": lambda d: _set(d, 200, 0)}


def _set(d, i, val):
    d = d.copy()
    d[i] = val
    return d


def _docs(S):
    return np.repeat(np.arange(4, dtype=np.int32), S // 4)        # four documents in order


def _untouched(*ts):
    return all(bool(torch.isnan(t.float()).all()) for t in ts)


@pytest.mark.parametrize("bad", sorted(BAD))
def test_chunk_calls_refuse_bad_ids(gpu_lib, bad):
    S, hq, hkv, d = 256, 4, 2, 64
    print(f"docs check chunk: {bad}", flush=True)
    (_, _, _, _), (q, k, v, do) = inputs(5, [(S, hq, d), (S, hkv, d), (S, hkv, d), (S, hq, d)], torch.bfloat16)
    good = torch.from_numpy(_docs(S)).to(DEV)
    wrong = torch.from_numpy(BAD[bad](_docs(S))).to(DEV)
    sh = shape_for(hq, hkv, d, torch.bfloat16)
    sh.flags = cp.CP_CHECK_DOCS
    nan = float("nan")
    o = torch.full((S, hq, d), nan, device=DEV)
    lse = torch.full((hq, S), nan, device=DEV)
    for qdoc, kdoc in ((wrong, good), (good, wrong)):
        with pytest.raises(cp.CpError) as e:
            cp.cp_attn_chunk_fwd(sh, q, cp.make_span(0, S, 0, 0, qdoc), k, v, cp.make_span(0, S, 0, 0, kdoc), o, lse)
        assert e.value.status == cp.CP_ERR_DOCS
        torch.cuda.synchronize()
        assert _untouched(o, lse)
    delta = torch.zeros(hq, S, device=DEV)
    dq = torch.full((S, hq, d), nan, device=DEV)
    dk = torch.full((S, hkv, d), nan, device=DEV)
    dv = torch.full_like(dk, nan)
    with pytest.raises(cp.CpError) as e:
        cp.cp_attn_chunk_bwd(sh, q, cp.make_span(0, S, 0, 0, wrong), k, v, cp.make_span(0, S, 0, 0, wrong), do,
                             lse, delta, dq, dk, dv)
    assert e.value.status == cp.CP_ERR_DOCS
    torch.cuda.synchronize()
    assert _untouched(dq, dk, dv)
    with pytest.raises(cp.CpError) as e:
        cp.cp_check_docs(wrong)
    assert e.value.status == cp.CP_ERR_DOCS
    cp.cp_check_docs(good)
    # valid ids: the checked call runs and equals the unchecked one bit for bit
    cp.cp_attn_chunk_fwd(sh, q, cp.make_span(0, S, 0, 0, good), k, v, cp.make_span(0, S, 0, 0, good), o, lse)
    o2, lse2 = torch.empty_like(o), torch.empty_like(lse)
    sh2 = shape_for(hq, hkv, d, torch.bfloat16)
    cp.cp_attn_chunk_fwd(sh2, q, cp.make_span(0, S, 0, 0, good), k, v, cp.make_span(0, S, 0, 0, good), o2, lse2)
    torch.cuda.synchronize()
    assert torch.equal(o, o2) and torch.equal(lse, lse2)


@pytest.mark.parametrize("bad", sorted(BAD))
def test_drivers_refuse_bad_ids(gpu_lib, bad):
    S, P, hq, hkv, d = 512, 2, 4, 2, 128
    print(f"docs check drivers: {bad}", flush=True)
    (_, _, _, _), (q, k, v, do) = inputs(6, [(S, hq, d), (S, hkv, d), (S, hkv, d), (S, hq, d)], torch.bfloat16)
    wrong = torch.from_numpy(BAD[bad](_docs(S))).to(DEV)
    sh = shape_for(hq, hkv, d, torch.bfloat16)
    sh.flags = cp.CP_CHECK_DOCS
    nan = float("nan")
    o = torch.full((S, hq, d), nan, device=DEV, dtype=torch.bfloat16)
    lse = torch.full((hq, S), nan, device=DEV)
    dq = torch.full((S, hq, d), nan, device=DEV)
    dk = torch.full((S, hkv, d), nan, device=DEV)
    dv = torch.full_like(dk, nan)
    ws = cp.workspace(cp.cp_ulysses_workspace_bytes(sh, S, 1, True))
    with pytest.raises(cp.CpError) as e:
        cp.cp_ulysses_share(sh, S, 1, 0, q, k, v, wrong, o, lse, do, dq, dk, dv, workspace=ws)
    assert e.value.status == cp.CP_ERR_DOCS
    n = S // P
    o_r = torch.full((n, hq, d), nan, device=DEV, dtype=torch.bfloat16)
    lse_r = torch.full((hq, n), nan, device=DEV)
    dq_r = torch.full((n, hq, d), nan, device=DEV)
    wsr = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, 0, cp.CP_BF16, True))
    with pytest.raises(cp.CpError) as e:
        cp.cp_ring_emulate(sh, S, P, 0, q, k, v, wrong, o_r, lse_r, do[:n], dq_r, dk, dv, workspace=wsr)
    assert e.value.status == cp.CP_ERR_DOCS
    with pytest.raises(cp.CpError) as e:
        cp.cp_ring_emulate_layout(sh, S, P, 0, [(0, 1), (2, 3)], q, k, v, wrong, o_r, lse_r, do[:n], dq_r, dk, dv,
                                  workspace=wsr)
    assert e.value.status == cp.CP_ERR_DOCS
    wsa = cp.workspace(cp.cp_allgather_workspace_bytes(sh, S, P, True, True))
    with pytest.raises(cp.CpError) as e:
        cp.cp_allgather_share(sh, S, P, 0, q[:n], k, v, wrong, o_r, lse_r, do[:n], dq_r, dk, dv, workspace=wsa)
    assert e.value.status == cp.CP_ERR_DOCS
    torch.cuda.synchronize()
    assert _untouched(o, lse, dq, dk, dv, o_r, lse_r, dq_r)


def test_ring_check_reads_ids_in_global_order(gpu_lib):
    """Ring ids come in sharded order, which is not sorted (rank 0 holds the
    first and the last chunk); the check must put them back in global order
    and accept them."""
    S, P, hq, hkv, d = 512, 2, 4, 2, 128
    from oracle import schedule as Z
    doc_g = _docs(S)
    order = Z.sharded_order(S, P)
    doc_sh = doc_g[order]
    assert np.any(np.diff(doc_sh) < 0)                    # sharded order is not sorted ...
    (_, _, _, _), (q, k, v, do) = inputs(8, [(S, hq, d), (S, hkv, d), (S, hkv, d), (S, hq, d)], torch.bfloat16)
    sh = shape_for(hq, hkv, d, torch.bfloat16)
    sh.flags = cp.CP_CHECK_DOCS
    n = S // P
    o = torch.empty(n, hq, d, device=DEV, dtype=torch.bfloat16)
    lse = torch.empty(hq, n, device=DEV)
    ws = cp.workspace(cp.cp_ring_workspace_bytes(sh, S, P, 0, cp.CP_BF16, False))
    cp.cp_ring_emulate(sh, S, P, 0, q, k, v, torch.from_numpy(doc_sh).to(DEV), o, lse, workspace=ws)   # ... yet valid
    torch.cuda.synchronize()
    assert torch.isfinite(o.float()).all()
