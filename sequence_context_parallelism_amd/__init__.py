"""Python binding of libcpattn: one GPU's share of context-parallel attention
on MI355X.

Argument marshalling only.  Every step of the path runs in the HIP kernels of
``libcpattn.so``; PyTorch supplies device memory and the stream.  Each
function has the name of the C entry point it wraps (see include/cpattn.h for
layouts, ownership and error behaviour) and raises ``CpError`` on any status
other than CP_OK.  There is no fallback: if the library is missing, ``load``
raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcpattn.so")

CP_OK, CP_ERR_ARG, CP_ERR_UNSUPPORTED, CP_ERR_ALIGN, CP_ERR_DOCS, CP_ERR_WORKSPACE, CP_ERR_HIP = \
    0, -1, -2, -3, -4, -5, -6
CP_BF16, CP_F32 = 0, 1
CP_CHECK_DOCS = 1

EXPORTED = (
    "cp_attn_chunk_fwd", "cp_lse_merge", "cp_attn_delta", "cp_attn_chunk_bwd",
    "cp_attn_chunk_bwd_dkdv", "cp_attn_chunk_bwd_dq",
    "cp_zigzag_layout", "cp_ring_schedule", "cp_ring_workspace_bytes", "cp_ring_emulate",
    "cp_ring_emulate_layout",
    "cp_ring_overlap_workspace_bytes", "cp_ring_emulate_overlap",
    "cp_ulysses_workspace_bytes", "cp_ulysses_share", "cp_ulysses_share_noalloc",
    "cp_allgather_workspace_bytes", "cp_allgather_share",
    "cp_check_docs", "cp_chunk_work", "cp_balanced_pairs",
    "cp_a2a_tokens_to_heads", "cp_a2a_heads_to_tokens",
    "cp_tile_map", "cp_last_error", "cp_abi_version",
)


class CpError(RuntimeError):
    def __init__(self, status, message):
        super().__init__(f"cpattn status {status}: {message}")
        self.status = status


class cp_span(ctypes.Structure):
    _fields_ = [("pos", ctypes.c_int64 * 2), ("len", ctypes.c_int32 * 2),
                ("doc", ctypes.c_void_p)]


class cp_shape(ctypes.Structure):
    _fields_ = [("hq", ctypes.c_int32), ("hkv", ctypes.c_int32), ("d", ctypes.c_int32),
                ("q_stride", ctypes.c_int64), ("kv_stride", ctypes.c_int64),
                ("scale", ctypes.c_float), ("causal", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


_lib = None


def load(path: str = LIB_PATH):
    """Load libcpattn.so (once).  Raises if it is not built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(f"{path} is not built; run `python -m sequence_context_parallelism_amd.build`")
    lib = ctypes.CDLL(path)
    P, I32, I64, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    SH = ctypes.POINTER(cp_shape)
    sig = {
        "cp_attn_chunk_fwd": (I32, [SH, P, cp_span, P, P, cp_span, P, I32, P, P]),
        "cp_lse_merge": (I32, [I64, I32, I32, P, P, P, P, P]),
        "cp_attn_delta": (I32, [I64, I32, I32, P, I32, P, I32, P, P]),
        "cp_attn_chunk_bwd": (I32, [SH, P, cp_span, P, P, cp_span, P, P, P, P, P, P, P]),
        "cp_attn_chunk_bwd_dkdv": (I32, [SH, P, cp_span, P, P, cp_span, P, P, P, P, P, P]),
        "cp_attn_chunk_bwd_dq": (I32, [SH, P, cp_span, P, P, cp_span, P, P, P, P, P]),
        "cp_zigzag_layout": (I32, [I64, I32, I32, ctypes.POINTER(ctypes.c_int64),
                                   ctypes.POINTER(ctypes.c_int32)]),
        "cp_ring_schedule": (I32, [I64, I32, I32, I32, ctypes.POINTER(ctypes.c_int32),
                                   ctypes.POINTER(ctypes.c_int8)]),
        "cp_ring_workspace_bytes": (SZ, [SH, I64, I32, I32, I32, I32]),
        "cp_ring_overlap_workspace_bytes": (SZ, [SH, I64, I32, I32, I32]),
        "cp_ring_emulate_overlap": (I32, [SH, I64, I32, I32, P, P, P, P, P, I32, P, P, P, P, P,
                                          P, SZ, P, P]),
        "cp_ring_emulate": (I32, [SH, I64, I32, I32, P, P, P, P, P, I32, P, P, P, P, P, P, P,
                                  P, SZ, P]),
        "cp_ring_emulate_layout": (I32, [SH, I64, I32, I32, P, P, P, P, P, P, I32, P, P, P, P, P,
                                         P, SZ, P]),
        "cp_ulysses_workspace_bytes": (SZ, [SH, I64, I32, I32]),
        "cp_ulysses_share": (I32, [SH, I64, I32, I32, P, P, P, P, P, I32, P, P, P, P, P, P,
                                   SZ, P]),
        "cp_ulysses_share_noalloc": (I32, [SH, I64, I32, I32, P, P, P, P, P, I32, P, P, P, P, P, P]),
        "cp_allgather_workspace_bytes": (SZ, [SH, I64, I32, I32, I32]),
        "cp_allgather_share": (I32, [SH, I64, I32, I32, P, P, P, P, P, I32, P, P, P, P, P, P, SZ, P]),
        "cp_check_docs": (I32, [P, I64, I32, P]),
        "cp_chunk_work": (I32, [I64, I32, P, P]),
        "cp_balanced_pairs": (I32, [I64, I32, P, P, P]),
        "cp_a2a_tokens_to_heads": (I32, [I64, I32, I32, I32, I32, I32, P, I64, P, P]),
        "cp_a2a_heads_to_tokens": (I32, [I64, I32, I32, I32, I32, I32, P, P, I64, P]),
        "cp_tile_map": (I32, [SH, cp_span, cp_span, I32, I32, P, P]),
        "cp_last_error": (ctypes.c_char_p, []),
        "cp_abi_version": (I32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status):
    if status != CP_OK:
        raise CpError(status, _lib.cp_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _arg_error(msg):
    raise CpError(CP_ERR_ARG, msg)


def _dense(name, t, shape=None):
    """An output (or dout/lse/delta) tensor must be contiguous, on the GPU,
    and, when ``shape`` is given, of exactly that shape: the library reads it
    with the documented dense layout and cannot see strides."""
    if t is None:
        return
    if not t.is_cuda:
        _arg_error(f"{name} must be a GPU tensor")
    if shape is not None and tuple(t.shape) != tuple(shape):
        _arg_error(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.numel() == 0:
        return
    if not t.is_contiguous():
        _arg_error(f"{name} must be contiguous (shape {tuple(t.shape)}, strides {tuple(t.stride())})")


def _tokens(name, t, stride):
    """q, k, v: token-major with ``stride`` elements between tokens (a head
    slice of a wider tensor is fine) and each head row contiguous."""
    if t is None:
        return
    if not t.is_cuda:
        _arg_error(f"{name} must be a GPU tensor")
    if t.numel() == 0:                     # an empty span: nothing is read
        return
    if t.dim() >= 2 and t.shape[0] > 1 and t.stride(0) != stride:
        _arg_error(f"{name} token stride {t.stride(0)} differs from the shape's {stride}")
    if t.stride(-1) != 1 or (t.dim() == 3 and t.shape[1] > 1 and t.stride(1) != t.shape[2]):
        _arg_error(f"{name} must have contiguous head rows (strides {tuple(t.stride())})")


def _stream(stream):
    if stream is not None:
        return ctypes.c_void_p(getattr(stream, "cuda_stream", stream))   # torch stream or raw handle
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    import torch
    if t.dtype == torch.bfloat16:
        return CP_BF16
    if t.dtype == torch.float32:
        return CP_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def make_span(pos0, len0, pos1=0, len1=0, doc=None):
    """A cp_span of up to two runs of global positions; ``doc`` is an int32
    device tensor or None."""
    s = cp_span()
    s.pos[0], s.pos[1] = int(pos0), int(pos1)
    s.len[0], s.len[1] = int(len0), int(len1)
    s.doc = None if doc is None else doc.data_ptr()
    return s


def make_shape(hq, hkv, d, q_stride, kv_stride, scale, causal, dtype, flags=0):
    sh = cp_shape()
    sh.hq, sh.hkv, sh.d = hq, hkv, d
    sh.q_stride, sh.kv_stride = q_stride, kv_stride
    sh.scale, sh.causal, sh.dtype = scale, int(bool(causal)), dtype
    sh.flags = int(flags)
    return sh


def _span_len(s):
    return int(s.len[0]) + int(s.len[1])


def cp_abi_version():
    return load().cp_abi_version()


def cp_attn_chunk_fwd(shape, q, qs, k, v, ks, o, lse, stream=None):
    lib = load()
    _tokens("q", q, shape.q_stride)
    _tokens("k", k, shape.kv_stride)
    _tokens("v", v, shape.kv_stride)
    _dense("o", o, (_span_len(qs), shape.hq, shape.d))
    _dense("lse", lse, (shape.hq, _span_len(qs)))
    _check(lib.cp_attn_chunk_fwd(ctypes.byref(shape), _ptr(q), qs, _ptr(k), _ptr(v), ks,
                                 _ptr(o), _dtype_code(o), _ptr(lse), _stream(stream)))


def cp_lse_merge(o_acc, lse_acc, o_part, lse_part, stream=None):
    """o_* [rows, h, d] fp32, lse_* [h, rows] fp32; acc updated in place."""
    lib = load()
    rows, h, d = o_acc.shape
    for name, t, shp in (("o_acc", o_acc, (rows, h, d)), ("o_part", o_part, (rows, h, d)),
                         ("lse_acc", lse_acc, (h, rows)), ("lse_part", lse_part, (h, rows))):
        _dense(name, t, shp)
    _check(lib.cp_lse_merge(rows, h, d, _ptr(o_acc), _ptr(lse_acc), _ptr(o_part),
                            _ptr(lse_part), _stream(stream)))


def cp_attn_delta(o, dout, delta, stream=None):
    lib = load()
    rows, h, d = o.shape
    _dense("o", o, (rows, h, d))
    _dense("dout", dout, (rows, h, d))
    _dense("delta", delta, (h, rows))
    _check(lib.cp_attn_delta(rows, h, d, _ptr(o), _dtype_code(o), _ptr(dout), _dtype_code(dout),
                             _ptr(delta), _stream(stream)))


def cp_attn_chunk_bwd(shape, q, qs, k, v, ks, dout, lse, delta, dq, dk, dv, stream=None):
    lib = load()
    _tokens("q", q, shape.q_stride)
    _tokens("k", k, shape.kv_stride)
    _tokens("v", v, shape.kv_stride)
    lq, lk = _span_len(qs), _span_len(ks)
    _dense("dout", dout, (lq, shape.hq, shape.d))
    _dense("lse", lse, (shape.hq, lq))
    _dense("delta", delta, (shape.hq, lq))
    _dense("dq", dq, (lq, shape.hq, shape.d))
    _dense("dk", dk, (lk, shape.hkv, shape.d))
    _dense("dv", dv, (lk, shape.hkv, shape.d))
    _check(lib.cp_attn_chunk_bwd(ctypes.byref(shape), _ptr(q), qs, _ptr(k), _ptr(v), ks,
                                 _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq), _ptr(dk),
                                 _ptr(dv), _stream(stream)))


def cp_attn_chunk_bwd_dkdv(shape, q, qs, k, v, ks, dout, lse, delta, dk, dv, stream=None):
    lib = load()
    _tokens("q", q, shape.q_stride)
    _tokens("k", k, shape.kv_stride)
    _tokens("v", v, shape.kv_stride)
    lq, lk = _span_len(qs), _span_len(ks)
    _dense("dout", dout, (lq, shape.hq, shape.d))
    _dense("lse", lse, (shape.hq, lq))
    _dense("delta", delta, (shape.hq, lq))
    _dense("dk", dk, (lk, shape.hkv, shape.d))
    _dense("dv", dv, (lk, shape.hkv, shape.d))
    _check(lib.cp_attn_chunk_bwd_dkdv(ctypes.byref(shape), _ptr(q), qs, _ptr(k), _ptr(v), ks,
                                      _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dk), _ptr(dv),
                                      _stream(stream)))


def cp_attn_chunk_bwd_dq(shape, q, qs, k, v, ks, dout, lse, delta, dq, stream=None):
    lib = load()
    _tokens("q", q, shape.q_stride)
    _tokens("k", k, shape.kv_stride)
    _tokens("v", v, shape.kv_stride)
    lq, lk = _span_len(qs), _span_len(ks)
    _dense("dout", dout, (lq, shape.hq, shape.d))
    _dense("lse", lse, (shape.hq, lq))
    _dense("delta", delta, (shape.hq, lq))
    _dense("dq", dq, (lq, shape.hq, shape.d))
    _check(lib.cp_attn_chunk_bwd_dq(ctypes.byref(shape), _ptr(q), qs, _ptr(k), _ptr(v), ks,
                                    _ptr(dout), _ptr(lse), _ptr(delta), _ptr(dq), _stream(stream)))


def cp_zigzag_layout(S, P, rank):
    lib = load()
    pos = (ctypes.c_int64 * 2)()
    ln = (ctypes.c_int32 * 2)()
    _check(lib.cp_zigzag_layout(S, P, rank, pos, ln))
    return (pos[0], pos[1]), (ln[0], ln[1])


def cp_ring_schedule(S, P, rank, step):
    lib = load()
    src = ctypes.c_int32()
    kind = (ctypes.c_int8 * 4)()
    _check(lib.cp_ring_schedule(S, P, rank, step, ctypes.byref(src), kind))
    return src.value, [kind[i] for i in range(4)]


def _ring_checks(shape, S, P, rank, q, k, v, o, lse, dout, dq, dk, dv):
    rows = S if rank < 0 else S // P
    _tokens("q", q, shape.q_stride)
    _tokens("k", k, shape.kv_stride)
    _tokens("v", v, shape.kv_stride)
    _dense("o", o, (rows, shape.hq, shape.d))
    _dense("lse", lse)
    if lse is not None and lse.numel() != shape.hq * rows:
        _arg_error(f"lse has {lse.numel()} elements, expected {shape.hq * rows}")
    _dense("dout", dout, (rows, shape.hq, shape.d))
    _dense("dq", dq, (rows, shape.hq, shape.d))
    _dense("dk", dk, (S, shape.hkv, shape.d))
    _dense("dv", dv, (S, shape.hkv, shape.d))


def cp_ring_workspace_bytes(shape, S, P, rank, o_dtype, backward):
    return load().cp_ring_workspace_bytes(ctypes.byref(shape), S, P, rank, o_dtype, int(bool(backward)))


def cp_ring_emulate(shape, S, P, rank, q, k, v, doc, o, lse, dout=None, dq=None, dk=None, dv=None,
                    step_o=None, step_lse=None, workspace=None, stream=None):
    lib = load()
    _ring_checks(shape, S, P, rank, q, k, v, o, lse, dout, dq, dk, dv)
    _dense("step_o", step_o, (P, S // P, shape.hq, shape.d))
    _dense("step_lse", step_lse, (P, shape.hq, S // P))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.cp_ring_emulate(ctypes.byref(shape), S, P, rank, _ptr(q), _ptr(k), _ptr(v), _ptr(doc),
                               _ptr(o), _dtype_code(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                               _ptr(dv), _ptr(step_o), _ptr(step_lse), _ptr(workspace), ws_bytes,
                               _stream(stream)))


def cp_ring_emulate_layout(shape, S, P, rank, chunks, q, k, v, doc, o, lse, dout=None, dq=None, dk=None, dv=None,
                           workspace=None, stream=None):
    """cp_ring_emulate under an explicit layout: ``chunks`` is a host int
    sequence of P pairs (a, b), a < b (e.g. the first result of
    cp_balanced_pairs); inputs are in that layout's sharded order."""
    import numpy as np
    lib = load()
    _ring_checks(shape, S, P, rank, q, k, v, o, lse, dout, dq, dk, dv)
    tab = np.ascontiguousarray(np.asarray(chunks, dtype=np.int32).reshape(-1))
    if tab.size != 2 * P:
        _arg_error(f"chunks holds {tab.size} entries, expected 2P={2 * P}")
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.cp_ring_emulate_layout(ctypes.byref(shape), S, P, rank, tab.ctypes.data_as(ctypes.c_void_p),
                                      _ptr(q), _ptr(k), _ptr(v), _ptr(doc), _ptr(o), _dtype_code(o), _ptr(lse),
                                      _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes,
                                      _stream(stream)))


def cp_ring_overlap_workspace_bytes(shape, S, P, o_dtype, backward):
    return load().cp_ring_overlap_workspace_bytes(ctypes.byref(shape), S, P, o_dtype, int(bool(backward)))


def cp_ring_emulate_overlap(shape, S, P, rank, q, k, v, doc, o, lse, dout=None, dq=None, dk=None, dv=None,
                            workspace=None, stream=None, copy_stream=None):
    lib = load()
    _ring_checks(shape, S, P, rank, q, k, v, o, lse, dout, dq, dk, dv)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.cp_ring_emulate_overlap(ctypes.byref(shape), S, P, rank, _ptr(q), _ptr(k), _ptr(v), _ptr(doc),
                                       _ptr(o), _dtype_code(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                       _ptr(dv), _ptr(workspace), ws_bytes, _stream(stream),
                                       _stream(copy_stream)))


def cp_ulysses_workspace_bytes(shape, S, sp, backward):
    return load().cp_ulysses_workspace_bytes(ctypes.byref(shape), S, sp, int(bool(backward)))


def cp_ulysses_share(shape, S, sp, sp_rank, q, k, v, doc, o, lse, dout=None, dq=None, dk=None,
                     dv=None, workspace=None, stream=None):
    lib = load()
    hq, hkv = shape.hq // sp, shape.hkv // sp
    _tokens("q", q, shape.q_stride)
    _tokens("k", k, shape.kv_stride)
    _tokens("v", v, shape.kv_stride)
    _dense("o", o, (S, hq, shape.d))
    _dense("lse", lse, (hq, S))
    _dense("dout", dout, (S, hq, shape.d))
    _dense("dq", dq, (S, hq, shape.d))
    _dense("dk", dk, (S, hkv, shape.d))
    _dense("dv", dv, (S, hkv, shape.d))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.cp_ulysses_share(ctypes.byref(shape), S, sp, sp_rank, _ptr(q), _ptr(k), _ptr(v),
                                _ptr(doc), _ptr(o), _dtype_code(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                _ptr(dk), _ptr(dv), _ptr(workspace), ws_bytes, _stream(stream)))


NOALLOC_SCRATCH_BYTES = 32 << 20       # CP_NOALLOC_SCRATCH_BYTES


def cp_ulysses_share_noalloc(shape, S, sp, sp_rank, q, k, v, doc, o, lse, dout=None, dq=None, dk=None, dv=None,
                             stream=None):
    """cp_ulysses_share without a workspace: Delta lives in the library's
    built-in per-GPU scratch (NOALLOC_SCRATCH_BYTES); calls that overlap on
    one GPU race."""
    lib = load()
    hq, hkv = shape.hq // sp, shape.hkv // sp
    _tokens("q", q, shape.q_stride)
    _tokens("k", k, shape.kv_stride)
    _tokens("v", v, shape.kv_stride)
    _dense("o", o, (S, hq, shape.d))
    _dense("lse", lse, (hq, S))
    _dense("dout", dout, (S, hq, shape.d))
    _dense("dq", dq, (S, hq, shape.d))
    _dense("dk", dk, (S, hkv, shape.d))
    _dense("dv", dv, (S, hkv, shape.d))
    _check(lib.cp_ulysses_share_noalloc(ctypes.byref(shape), S, sp, sp_rank, _ptr(q), _ptr(k), _ptr(v),
                                        _ptr(doc), _ptr(o), _dtype_code(o), _ptr(lse), _ptr(dout), _ptr(dq),
                                        _ptr(dk), _ptr(dv), _stream(stream)))


def cp_allgather_workspace_bytes(shape, S, P, has_doc, backward):
    return load().cp_allgather_workspace_bytes(ctypes.byref(shape), S, P, int(bool(has_doc)), int(bool(backward)))


def cp_allgather_share(shape, S, P, rank, q, k, v, doc, o, lse, dout=None, dq=None, dk=None, dv=None,
                       workspace=None, stream=None):
    lib = load()
    n = S // P
    _tokens("q", q, shape.q_stride)
    _tokens("k", k, shape.kv_stride)
    _tokens("v", v, shape.kv_stride)
    _dense("o", o, (n, shape.hq, shape.d))
    _dense("lse", lse, (shape.hq, n))
    _dense("dout", dout, (n, shape.hq, shape.d))
    _dense("dq", dq, (n, shape.hq, shape.d))
    _dense("dk", dk, (S, shape.hkv, shape.d))
    _dense("dv", dv, (S, shape.hkv, shape.d))
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib.cp_allgather_share(ctypes.byref(shape), S, P, rank, _ptr(q), _ptr(k), _ptr(v), _ptr(doc),
                                  _ptr(o), _dtype_code(o), _ptr(lse), _ptr(dout), _ptr(dq), _ptr(dk),
                                  _ptr(dv), _ptr(workspace), ws_bytes, _stream(stream)))


def _host_doc(doc):
    import numpy as np
    if doc is None:
        return None, None
    d = np.ascontiguousarray(doc, dtype=np.int32)
    return d, d.ctypes.data_as(ctypes.c_void_p)


def cp_check_docs(doc, stream=None):
    """Checks document ids (>= 0, non-decreasing): ``doc`` is a GPU int32
    tensor (copied to the host on the stream, which the call waits for) or a
    host array.  Raises CpError (CP_ERR_DOCS) naming the first bad index."""
    import numpy as np
    lib = load()
    if hasattr(doc, "is_cuda") and doc.is_cuda:
        import torch
        if doc.dtype != torch.int32 or not doc.is_contiguous():
            _arg_error("doc must be a contiguous int32 tensor")
        _check(lib.cp_check_docs(_ptr(doc), doc.numel(), 0, _stream(stream)))
        return
    d, dp = _host_doc(doc)
    _check(lib.cp_check_docs(dp, 0 if d is None else d.size, 1, None))


def cp_chunk_work(S, P, doc=None):
    """Live (query, key) pairs per chunk of S/(2P) tokens; doc: host int32 ids or None."""
    import numpy as np
    lib = load()
    d, dp = _host_doc(doc)
    w = np.zeros(2 * P, dtype=np.int64)
    _check(lib.cp_chunk_work(S, P, dp, w.ctypes.data_as(ctypes.c_void_p)))
    return w


def cp_balanced_pairs(S, P, doc=None):
    """(chunks [P, 2], rank_work [P]) of the document-aware two-chunk layout."""
    import numpy as np
    lib = load()
    d, dp = _host_doc(doc)
    ch = np.zeros(2 * P, dtype=np.int32)
    rw = np.zeros(P, dtype=np.int64)
    _check(lib.cp_balanced_pairs(S, P, dp, ch.ctypes.data_as(ctypes.c_void_p), rw.ctypes.data_as(ctypes.c_void_p)))
    return ch.reshape(P, 2), rw


def cp_a2a_tokens_to_heads(x, sp, rank, y, stream=None):
    """x [S, h, d] (token stride x.stride(0)) -> y [S, h_out, d] for `rank`."""
    lib = load()
    S, h, d = x.shape
    _check(lib.cp_a2a_tokens_to_heads(S, h, d, x.element_size(), sp, rank, _ptr(x), x.stride(0), _ptr(y),
                                      _stream(stream)))


def cp_a2a_heads_to_tokens(o, sp, rank, z, stream=None):
    """o [S, h/sp, d] of `rank` -> its heads of z [S, h, d] (token stride z.stride(0))."""
    lib = load()
    S, h, d = z.shape
    _check(lib.cp_a2a_heads_to_tokens(S, h, d, z.element_size(), sp, rank, _ptr(o), _ptr(z), z.stride(0),
                                      _stream(stream)))


def cp_tile_map(shape, qs, ks, bq, bk, out, stream=None):
    lib = load()
    _check(lib.cp_tile_map(ctypes.byref(shape), qs, ks, bq, bk, _ptr(out), _stream(stream)))


def workspace(nbytes, device="cuda"):
    """A caller-owned scratch buffer (torch allocations are 256-byte aligned)."""
    import torch
    return torch.empty(max(int(nbytes), 1), dtype=torch.uint8, device=device)
