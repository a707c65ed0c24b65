"""Helpers for the GPU parity tests: seeded host inputs, device copies, and
error measures.  Holds none of the attention arithmetic."""
import math

import numpy as np
import torch

import cpinputs
import sequence_context_parallelism_amd as cp

DEV = "cuda"


def bf16_round(x):
    """Round float32 host values to bf16 (nearest even) and return them as
    float64, i.e. the exact values the device will see."""
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def to_dev(x, dtype):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(DEV).to(dtype)


def inputs(seed, shapes, dtype):
    """Host N(0,1) arrays (rounded to bf16 if dtype is bf16) and their device copies."""
    host = cpinputs.normal_host(seed, shapes)
    if dtype == torch.bfloat16:
        host = [bf16_round(h) for h in host]
    else:
        host = [h.astype(np.float64) for h in host]
    return host, [to_dev(h, dtype) for h in host]


def run_positions(pos0, len0, pos1=0, len1=0):
    return np.concatenate([np.arange(pos0, pos0 + len0), np.arange(pos1, pos1 + len1)]).astype(np.int64)


def max_abs(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if a.size == 0:
        return 0.0
    return float(np.max(np.abs(a - b)))


def lse_err(gpu, ref):
    """Max |difference| over finite entries; -inf entries must match exactly."""
    gpu = np.asarray(gpu, np.float64)
    ref = np.asarray(ref, np.float64)
    assert np.array_equal(np.isneginf(gpu), np.isneginf(ref)), "empty-row (-inf) pattern differs"
    fin = np.isfinite(ref)
    return float(np.max(np.abs(gpu[fin] - ref[fin]), initial=0.0))


def grad_tol(ref, base):
    return base * max(1.0, float(np.max(np.abs(ref), initial=0.0)))


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def shape_for(hq, hkv, d, dtype, causal=True, q_stride=None, kv_stride=None, scale=None):
    return cp.make_shape(hq, hkv, d, q_stride or hq * d, kv_stride or hkv * d,
                         scale if scale is not None else 1.0 / math.sqrt(d), causal,
                         cp.CP_BF16 if dtype == torch.bfloat16 else cp.CP_F32)


TOL = {torch.bfloat16: dict(o=2e-2, lse=1e-3, grad=2e-2),
       torch.float32: dict(o=1e-5, lse=1e-6, grad=1e-5)}
