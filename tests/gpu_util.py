"""Shared helpers of the GPU parity tests: device availability, the
acceptance checks, and a per-query oracle for full-size workloads."""
from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import workloads as W
from oracle import csa2_oracle as O

# Acceptance bars: Top-K index sets bit-exact on integer indexer inputs; on
# N(0,1) inputs an aggregate overlap of at least 99.9 %, every disagreement a
# near-tie of the fp64 scores; attention outputs within 2e-3 absolute of the
# fp64 oracle evaluated over the GPU's own selection; LSE within 1e-4
# relative.
OVERLAP_MIN = 0.999
OUT_ATOL = 2e-3
LSE_RTOL = 1e-4
# fp32 accumulation of 128 exact FP8 products and <= 16 weighted heads: the
# relative rounding of the score is below ~2^-24 * 150; 1e-5 of the
# magnitude of the score bounds a near-tie generously.
TIE_RTOL = 1e-5


def have_gpu() -> bool:
    try:
        return torch.cuda.is_available()
    except Exception:
        return False


def need_gpu():
    if not have_gpu():
        pytest.skip("no GPU")
    from fp4_kv_cache_layer_amd import _lib
    _lib.load()          # fail loudly if the HIP library is missing


def say(msg: str) -> None:
    print(msg, flush=True)


def overlap_stats(gpu_idx, gpu_cnt, ora_idx, ora_cnt):
    tot = inter = 0
    worst = 1.0
    for gi, gc, oi, oc in zip(gpu_idx, gpu_cnt, ora_idx, ora_cnt):
        assert gc == oc, (gc, oc)
        a, b = set(gi[:gc].tolist()), set(oi[:oc].tolist())
        n = len(a & b)
        tot += oc
        inter += n
        if oc:
            worst = min(worst, n / oc)
    return (inter / tot if tot else 1.0), worst


def check_selection_valid(gi, gc, oi, oc, scores, k):
    """The GPU row must be ascending, padded with -1, and any entry it holds
    instead of an oracle entry must be a near-tie in the fp64 scores."""
    assert gc == oc
    row = gi[:gc]
    assert (np.diff(row) > 0).all(), "selection not strictly ascending"
    assert (gi[gc:] == -1).all()
    extra = sorted(set(row.tolist()) - set(oi[:oc].tolist()))
    missing = sorted(set(oi[:oc].tolist()) - set(row.tolist()))
    assert len(extra) == len(missing)
    if extra:
        top_missing = max(scores[t] for t in missing)
        low_extra = min(scores[t] for t in extra)
        tol = TIE_RTOL * max(1.0, abs(top_missing), abs(low_extra))
        assert top_missing - low_extra <= tol, (extra[:4], missing[:4], top_missing, low_extra)


def single_seq_cache(spec: W.CaseSpec, s: int, vis: int, gen_device: str):
    """An oracle cache holding sequence s's first vis indexer rows (encoded by
    the oracle) in in-order 64-entry pages; main-KV rows are added on demand."""
    ps = 64
    npg = (vis + ps - 1) // ps
    cache = O.Cache.empty(npg, ps, np.arange(npg, dtype=np.int32)[None], [vis])
    ik = W.idxk_rows(spec, s, gen_device)[:vis].cpu().numpy().view(np.uint16)
    flat = cache.idx_k.reshape(-1, 128)
    for a in range(0, vis, 1 << 18):
        b = min(vis, a + (1 << 18))
        flat[a:b] = O.quantize_idxk_rows(O.bf16_to_f64(ik[a:b]))
    return cache


def add_kv_rows(cache, spec: W.CaseSpec, s: int, rows, gen_device: str):
    rows = np.asarray(sorted(set(int(t) for t in rows if t >= 0)), dtype=np.int64)
    if rows.size == 0:
        return
    kv = W.kv_rows(spec, s, gen_device)
    sel = kv[torch.from_numpy(rows).to(kv.device)].cpu().numpy().view(np.uint16)
    cache.kv.reshape(-1, 272)[rows] = O.quantize_kv_rows(O.bf16_to_f64(sel))
