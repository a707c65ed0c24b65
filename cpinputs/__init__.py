"""Seeded synthetic inputs shared by the tests, the smoke check and the
benchmark.  This module draws random numbers and builds integer layouts; it
holds none of the attention arithmetic and imports neither the oracle nor the
library.

Input recipe (the workloads are synthetic; no dataset is involved):

* Q, K, V and dO are i.i.d. N(0, 1) float32 drawn in that order from one seed,
  then rounded to bf16 (round to nearest even) when the workload is bf16.  The
  softmax scale is 1/sqrt(d); the inputs themselves are not pre-scaled.
* Packed documents: lengths drawn lognormal with median 4096 and sigma 1.0
  (natural-log units), rounded to the nearest integer and clipped to
  [128, 32768], drawn until they cover S; the last document is cut to fill S.
  Document ids are 0, 1, 2, ... in order (int32, non-decreasing).
"""
from __future__ import annotations

import numpy as np

SEEDS = {"tiny_ring": 1001, "ulysses_64k": 1002, "ring_128k": 1003,
         "docs_128k": 1004, "usp_1m": 1005}
DOC_SEED = 2004


def normal_host(seed, shapes):
    """float32 N(0,1) arrays of the given shapes, drawn in order from one
    numpy generator."""
    rng = np.random.default_rng(seed)
    return [rng.standard_normal(s, dtype=np.float32) for s in shapes]


def normal_torch(seed, shapes, device, dtype):
    """N(0,1) tensors drawn in float32 in order from one torch generator on
    ``device``, then cast to ``dtype`` (round to nearest even for bf16)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    out = []
    for s in shapes:
        t = torch.randn(s, generator=g, device=device, dtype=torch.float32)
        out.append(t.to(dtype) if dtype != torch.float32 else t)
    return out


def lognormal_doc_lengths(S, seed=DOC_SEED, median=4096, sigma=1.0,
                          lo=128, hi=32768):
    """Document lengths covering exactly S tokens (see module docstring)."""
    rng = np.random.default_rng(seed)
    lens = []
    total = 0
    while total < S:
        x = int(np.clip(np.rint(rng.lognormal(np.log(median), sigma)), lo, hi))
        x = min(x, S - total)
        lens.append(x)
        total += x
    return np.array(lens, dtype=np.int64)


def doc_ids_from_lengths(lengths):
    """Per-token document ids 0, 1, 2, ... (int32)."""
    return np.repeat(np.arange(len(lengths), dtype=np.int32), lengths)


def random_doc_ids(L, rng, max_docs=6):
    """Small random non-decreasing doc-id vector for tests (int32)."""
    cuts = np.sort(rng.choice(np.arange(1, max(L, 2)), size=min(max_docs - 1, max(L - 1, 0)),
                              replace=False)) if L > 1 else np.array([], dtype=np.int64)
    ids = np.zeros(L, dtype=np.int32)
    for c in cuts:
        ids[c:] += 1
    return ids
