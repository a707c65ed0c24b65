"""CPU tests of the C ABI: the library loads, exports every symbol the header
declares, and its host-only logic (zigzag layout, ring schedule, argument
validation) matches the oracle bit for bit.  No kernel is launched."""
import ctypes
import os
import re

import numpy as np
import pytest

import sequence_context_parallelism_amd as cp
from oracle import schedule as Z

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "cpattn.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(cp_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    return cp.load()


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert len(names) >= 13
    assert set(names) == set(cp.EXPORTED)
    for n in names:
        assert hasattr(lib, n), n
    assert cp.cp_abi_version() == 2


@pytest.mark.parametrize("S,P", [(16, 2), (256, 2), (131072, 8), (1048576, 4), (96, 6), (8, 1)])
def test_zigzag_and_schedule_bit_exact(S, P):
    for r in range(P):
        assert cp.cp_zigzag_layout(S, P, r) == tuple(tuple(x) for x in Z.zigzag_layout(S, P, r))
        for s in range(P):
            src, kinds = cp.cp_ring_schedule(S, P, r, s)
            osrc, okinds = Z.ring_schedule(S, P, r, s)
            assert (src, kinds) == (osrc, okinds)


@pytest.mark.parametrize("args", [(10, 3, 0), (16, 2, 2), (16, 0, 0), (16, 2, -1), (0, 1, 0)])
def test_zigzag_rejects_bad_sizes(args):
    with pytest.raises(cp.CpError) as e:
        cp.cp_zigzag_layout(*args)
    assert e.value.status == cp.CP_ERR_ARG
    with pytest.raises(ValueError):
        Z.zigzag_layout(*args)


def test_schedule_rejects_bad_step():
    with pytest.raises(cp.CpError):
        cp.cp_ring_schedule(16, 2, 0, 2)


def _shape(**kw):
    base = dict(hq=8, hkv=2, d=128, q_stride=8 * 128, kv_stride=2 * 128, scale=0.088,
                causal=True, dtype=cp.CP_BF16)
    base.update(kw)
    return cp.make_shape(**base)


def _fwd_status(lib, shape, qs=None, ks=None, ptr=0x10000):
    qs = qs or cp.make_span(0, 64)
    ks = ks or cp.make_span(0, 64)
    p = ctypes.c_void_p(ptr)
    return lib.cp_attn_chunk_fwd(ctypes.byref(shape), p, qs, p, p, ks, p, cp.CP_F32, p, None)


@pytest.mark.parametrize("kw,status", [
    (dict(d=96), cp.CP_ERR_UNSUPPORTED),
    (dict(hq=6, hkv=2), cp.CP_ERR_UNSUPPORTED),       # group of 3
    (dict(hq=7, hkv=2), cp.CP_ERR_ARG),
    (dict(q_stride=100), cp.CP_ERR_ARG),
    (dict(q_stride=8 * 128 + 4), cp.CP_ERR_ALIGN),
    (dict(scale=-1.0), cp.CP_ERR_ARG),
    (dict(hkv=0), cp.CP_ERR_ARG),
    (dict(q_stride=(1 << 23) + 8), cp.CP_ERR_UNSUPPORTED),  # > 16 MiB between tokens
    (dict(kv_stride=(1 << 23) + 8), cp.CP_ERR_UNSUPPORTED),
])
def test_validation_errors_before_launch(lib, kw, status):
    assert _fwd_status(lib, _shape(**kw)) == status
    assert lib.cp_last_error().decode() != ""


def test_span_and_pointer_errors(lib):
    sh = _shape()
    bad_runs = cp.make_span(0, 64, 10, 8)                  # second run overlaps the first
    assert _fwd_status(lib, sh, qs=bad_runs) == cp.CP_ERR_ARG
    assert _fwd_status(lib, sh, qs=cp.make_span(0, -1)) == cp.CP_ERR_ARG
    assert _fwd_status(lib, sh, ptr=0x10008) == cp.CP_ERR_ALIGN
    one_doc = cp.cp_span()
    one_doc.len[0] = 64
    one_doc.doc = 0x1000
    assert _fwd_status(lib, sh, qs=one_doc) == cp.CP_ERR_DOCS
    # spans past 2^29 tokens: per-token rows are addressed with 32-bit byte offsets
    assert _fwd_status(lib, sh, ks=cp.make_span(0, (1 << 29) + 64)) == cp.CP_ERR_UNSUPPORTED
    assert _fwd_status(lib, sh, qs=cp.make_span(0, 1 << 28, 1 << 28, (1 << 28) + 64)) == cp.CP_ERR_UNSUPPORTED
    # empty query span: nothing to do, success without touching memory
    assert _fwd_status(lib, sh, qs=cp.make_span(0, 0)) == cp.CP_OK


def test_ring_and_ulysses_argument_errors(lib):
    sh = _shape()
    P = ctypes.c_void_p(0x10000)
    st = lib.cp_ring_emulate(ctypes.byref(sh), 1000, 8, 0, P, P, P, None, P, cp.CP_BF16, P,
                             None, None, None, None, None, None, None, 0, None)
    assert st == cp.CP_ERR_ARG                                  # 1000 % 16 != 0
    st = lib.cp_ring_emulate(ctypes.byref(sh), (1 << 29) + 16, 8, 0, P, P, P, None, P, cp.CP_BF16, P,
                             None, None, None, None, None, None, None, 0, None)
    assert st == cp.CP_ERR_UNSUPPORTED                          # above 2^29 tokens
    st = lib.cp_ulysses_share(ctypes.byref(sh), (1 << 29) + 16, 2, 0, P, P, P, None, P, cp.CP_BF16, P,
                              None, None, None, None, None, 0, None)
    assert st == cp.CP_ERR_UNSUPPORTED
    st = lib.cp_ring_emulate(ctypes.byref(sh), 1024, 8, 0, P, P, P, None, P, cp.CP_BF16, P,
                             None, None, None, None, None, None, None, 0, None)
    assert st == cp.CP_ERR_WORKSPACE
    need = cp.cp_ring_workspace_bytes(sh, 1024, 8, 0, cp.CP_BF16, False)
    assert need > 0 and need % 256 == 0
    st = lib.cp_ulysses_share(ctypes.byref(sh), 1024, 4, 0, P, P, P, None, P, cp.CP_BF16, P,
                              None, None, None, None, None, 0, None)
    assert st == cp.CP_ERR_ARG                                  # sp=4 does not divide hkv=2
    assert cp.cp_ulysses_workspace_bytes(sh, 1024, 2, True) == 4 * 1024 * 4
    # the traffic emulation: one rank only, a distinct copy stream, its own workspace
    S1 = ctypes.c_void_p(0x20000)
    st = lib.cp_ring_emulate_overlap(ctypes.byref(sh), 1024, 8, -1, P, P, P, None, P, cp.CP_BF16, P,
                                     None, None, None, None, None, 0, None, S1)
    assert st == cp.CP_ERR_ARG                                  # rank -1
    st = lib.cp_ring_emulate_overlap(ctypes.byref(sh), 1024, 8, 0, P, P, P, None, P, cp.CP_BF16, P,
                                     None, None, None, None, None, 0, S1, S1)
    assert st == cp.CP_ERR_ARG                                  # same stream twice
    st = lib.cp_ring_emulate_overlap(ctypes.byref(sh), 1024, 8, 0, P, P, P, None, P, cp.CP_BF16, P,
                                     None, None, None, None, None, 0, None, S1)
    assert st == cp.CP_ERR_WORKSPACE
    plain = cp.cp_ring_workspace_bytes(sh, 1024, 8, 0, cp.CP_BF16, True)
    over = cp.cp_ring_overlap_workspace_bytes(sh, 1024, 8, cp.CP_BF16, True)
    n, kvrow = 1024 // 8, sh.hkv * sh.d
    assert over % 256 == 0 and over >= plain + 2 * (2 * n * kvrow * 2) + 2 * n * kvrow * 4
    assert cp.cp_ring_overlap_workspace_bytes(sh, 1000, 8, cp.CP_BF16, True) == 0


def _docs(S, seed, median):
    import cpinputs
    lens = cpinputs.lognormal_doc_lengths(S, seed=seed, median=median, sigma=1.0, lo=1, hi=S)
    return cpinputs.doc_ids_from_lengths(lens)


@pytest.mark.parametrize("S,P,docs", [(512, 1, False), (512, 2, True), (768, 3, True), (1024, 4, True), (1024, 4, False)])
def test_chunk_work_matches_mask_count(lib, S, P, docs):
    doc = _docs(S, 11 + S + P, S // 8) if docs else None
    got = cp.cp_chunk_work(S, P, doc)
    assert np.array_equal(got, Z.chunk_work(S, P, doc))


@pytest.mark.parametrize("P,seed", [(2, 1), (3, 2), (4, 3), (4, 4), (5, 5)])
def test_balanced_pairs_are_optimal(lib, P, seed):
    S = 2 * P * 64
    doc = _docs(S, seed, 40)
    pairs, rw = cp.cp_balanced_pairs(S, P, doc)
    work = Z.chunk_work(S, P, doc)
    assert sorted(pairs.ravel().tolist()) == list(range(2 * P))          # every chunk exactly once
    assert np.all(pairs[:, 0] < pairs[:, 1])
    assert np.array_equal(rw, work[pairs[:, 0]] + work[pairs[:, 1]])
    assert rw.max() == Z.best_pairing(work)                                # min-max is attained


def test_balanced_pairs_without_docs_is_zigzag(lib):
    S, P = 4096, 8
    pairs, rw = cp.cp_balanced_pairs(S, P)
    got = {tuple(p) for p in pairs.tolist()}
    want = {tuple(int(x) // (S // (2 * P)) for x in (Z.zigzag_layout(S, P, r)[0])) for r in range(P)}
    assert got == want
    assert rw.min() == rw.max()          # causal work is exactly balanced by zigzag


def test_doc_aware_layout_beats_zigzag_on_packed_documents(lib):
    import cpinputs
    S, P = 131072, 8
    doc = cpinputs.doc_ids_from_lengths(cpinputs.lognormal_doc_lengths(S))
    work = cp.cp_chunk_work(S, P, doc)
    zz = np.array([work[r] + work[2 * P - 1 - r] for r in range(P)])
    _, rw = cp.cp_balanced_pairs(S, P, doc)
    assert rw.sum() == zz.sum() == work.sum()
    assert rw.max() <= zz.max()


def test_chunk_work_rejects_bad_docs(lib):
    with pytest.raises(cp.CpError):
        cp.cp_chunk_work(8, 2, np.array([0, 0, 1, 0, 1, 1, 1, 1], dtype=np.int32))
    with pytest.raises(cp.CpError):
        cp.cp_chunk_work(10, 2)


# ---- document ids (Llama 3 page, section "네 병렬화는 서로 다른 자원을 확보하는
# 방식": packed documents must keep their mask) ----------------------------------

@pytest.mark.parametrize("ids,ok", [
    ([0, 0, 1, 1, 5, 5, 9], True),
    ([], True),
    ([3], True),
    ([0, 0, -1, 2], False),          # negative
    ([-4, -4, -4], False),
    ([0, 1, 2, 1, 3], False),        # decreasing
    ([5, 4], False),
])
def test_check_docs_on_host_copy(lib, ids, ok):
    arr = np.array(ids, dtype=np.int32)
    if ok:
        cp.cp_check_docs(arr)
    else:
        with pytest.raises(cp.CpError) as e:
            cp.cp_check_docs(arr)
        assert e.value.status == cp.CP_ERR_DOCS
        assert "index" in lib.cp_last_error().decode()


def test_check_docs_argument_errors(lib):
    assert lib.cp_check_docs(None, 4, 1, None) == cp.CP_ERR_ARG
    assert lib.cp_check_docs(None, -1, 1, None) == cp.CP_ERR_ARG
    assert lib.cp_check_docs(None, 0, 1, None) == cp.CP_OK


def test_unknown_flag_bits_are_refused(lib):
    assert _fwd_status(lib, _shape(flags=2)) == cp.CP_ERR_ARG
    # the one defined bit passes the shape check (an empty query span then returns before any launch)
    assert _fwd_status(lib, _shape(flags=cp.CP_CHECK_DOCS), qs=cp.make_span(0, 0)) == cp.CP_OK


@pytest.mark.parametrize("chunks,status", [
    ([0, 7, 1, 6, 2, 5, 3, 4], cp.CP_ERR_WORKSPACE),      # zigzag table: valid, then the missing workspace
    ([0, 1, 2, 3, 4, 5, 6, 7], cp.CP_ERR_WORKSPACE),      # any pairing with a < b is valid
    ([1, 0, 2, 3, 4, 5, 6, 7], cp.CP_ERR_ARG),            # a > b
    ([0, 1, 1, 2, 4, 5, 6, 7], cp.CP_ERR_ARG),            # chunk 1 twice
    ([0, 1, 2, 3, 4, 5, 6, 8], cp.CP_ERR_ARG),            # out of range
])
def test_ring_layout_table_checks(lib, chunks, status):
    sh = _shape()
    P = ctypes.c_void_p(0x10000)
    tab = np.array(chunks, dtype=np.int32)
    st = lib.cp_ring_emulate_layout(ctypes.byref(sh), 1024, 4, 0, tab.ctypes.data_as(ctypes.c_void_p),
                                    P, P, P, None, P, cp.CP_BF16, P, None, None, None, None, None, 0, None)
    assert st == status, lib.cp_last_error().decode()
    st = lib.cp_ring_emulate_layout(ctypes.byref(sh), 1024, 4, 0, None, P, P, P, None, P, cp.CP_BF16, P,
                                    None, None, None, None, None, 0, None)
    assert st == cp.CP_ERR_ARG


def test_ulysses_noalloc_refusals_before_launch(lib):
    """The no-allocation Ulysses share refuses, before touching the GPU, a
    backward whose Delta rows exceed the built-in scratch and the checked
    document mode (which would copy to the host and wait)."""
    sh = _shape()
    P = ctypes.c_void_p(0x10000)
    big = cp.NOALLOC_SCRATCH_BYTES // (4 * sh.hq) + 64
    st = lib.cp_ulysses_share_noalloc(ctypes.byref(sh), big, 1, 0, P, P, P, None, P, cp.CP_BF16, P,
                                      P, P, P, P, None)
    assert st == cp.CP_ERR_WORKSPACE, lib.cp_last_error().decode()
    shc = _shape(flags=cp.CP_CHECK_DOCS)
    st = lib.cp_ulysses_share_noalloc(ctypes.byref(shc), 1024, 1, 0, P, P, P, None, P, cp.CP_BF16, P,
                                      P, P, P, P, None)
    assert st == cp.CP_ERR_ARG
    st = lib.cp_ulysses_share_noalloc(ctypes.byref(sh), 1024, 4, 0, P, P, P, None, P, cp.CP_BF16, P,
                                      P, P, P, P, None)
    assert st == cp.CP_ERR_ARG                                   # sp=4 does not divide hkv=2
