"""Glue between the seeded workloads and the fp64 oracle (tests only).

``OracleCase`` holds the host copies of one workload's raw inputs and an
oracle cache filled with the cached entries (encoded by the oracle's own
encoders).  ``run_group`` runs the workload's layer group through the oracle.
"""
from __future__ import annotations

import dataclasses
from typing import Dict, List

import numpy as np

import workloads as W
from oracle import csa2_oracle as O


@dataclasses.dataclass
class LayerInputs:
    mode: int
    q_idx: np.ndarray      # [nq][h_idx][128] uint8
    w: np.ndarray          # [nq][h_idx] float32
    q: np.ndarray          # [nq][h][512] uint16 (bf16 bits)


@dataclasses.dataclass
class OracleCase:
    spec: W.CaseSpec
    page_table: np.ndarray
    kv_src: List[np.ndarray]      # per sequence: [seq_len_after][512] bf16 bits
    ik_src: List[np.ndarray]      # per sequence: [seq_len_after][128] bf16 bits
    layers: List[LayerInputs]
    new_slots: np.ndarray         # [n_rows_new] physical slots of the appended rows
    new_kv: np.ndarray            # [n_rows_new][512]
    new_ik: np.ndarray            # [n_rows_new][128]

    def fresh_cache(self) -> O.Cache:
        """Oracle cache holding the cached (pre-step) entries only."""
        spec = self.spec
        cache = O.Cache.empty(spec.total_pages(), spec.page_size, self.page_table,
                              [spec.seq_len_after(s) for s in range(spec.num_seqs)])
        for s in range(spec.num_seqs):
            c = spec.cached[s]
            if c:
                O.append_quant_fp4(cache, W.slots_for(spec, self.page_table, s, 0, c),
                                   self.kv_src[s][:c], self.ik_src[s][:c])
        return cache


def build(spec: W.CaseSpec, device="cpu") -> OracleCase:
    pt = W.page_table(spec)
    kv_src, ik_src = [], []
    ns, nk, ni = [], [], []
    for s in range(spec.num_seqs):
        kv = W.kv_rows(spec, s, device).cpu().numpy().view(np.uint16)
        ik = W.idxk_rows(spec, s, device).cpu().numpy().view(np.uint16)
        kv_src.append(kv)
        ik_src.append(ik)
        c = spec.cached[s]
        if spec.n_new:
            ns.append(W.slots_for(spec, pt, s, c, c + spec.n_new))
            nk.append(kv[c:c + spec.n_new])
            ni.append(ik[c:c + spec.n_new])
    layers = []
    for li, mode in enumerate(spec.modes):
        qi, w, q = W.layer_queries(spec, li, device)
        layers.append(LayerInputs(mode, qi.cpu().numpy(), w.cpu().numpy(), q.cpu().numpy().view(np.uint16)))
    cat = (lambda xs, shape: np.concatenate(xs) if xs else np.zeros(shape, np.uint16))
    return OracleCase(spec, pt, kv_src, ik_src, layers,
                      np.concatenate(ns).astype(np.int32) if ns else np.zeros(0, np.int32),
                      cat(nk, (0, 512)), cat(ni, (0, 128)))


def run_group(case: OracleCase) -> List[Dict[str, np.ndarray]]:
    """The workload's layer group through the oracle.  Reindex and Reuse layers
    read the preceding Full layer's cache; Reuse reads that layer's indices.
    With spec.pool_k, the Full layer's Top-pool_k is the pool (returned with
    its results) and Reindex layers select among it."""
    spec = case.spec
    q_seq, q_vis = spec.q_seq(), spec.q_vis()
    results = []
    cache = None
    full_idx = full_cnt = None
    pool = pool_cnt = None
    for L in case.layers:
        if L.mode == O.FULL:
            cache = case.fresh_cache()
            idx, cnt, o, lse = O.layer_step(O.FULL, cache, L.q, q_seq, q_vis, spec.k, spec.sm_scale,
                                            q_idx=L.q_idx, w=L.w, new_slots=case.new_slots,
                                            new_kv=case.new_kv, new_idxk=case.new_ik)
            full_idx, full_cnt = idx, cnt
            if spec.pool_k:
                pool, pool_cnt = O.index_topk(cache, L.q_idx, L.w, q_seq, q_vis, spec.pool_k)
                results.append(dict(idx=idx, cnt=cnt, out=o, lse=lse, pool=pool, pool_cnt=pool_cnt))
                continue
        elif L.mode == O.REINDEX and spec.pool_k:
            idx, cnt = O.pool_index_topk(cache, L.q_idx, L.w, q_seq, pool, pool_cnt, spec.k)
            o, lse = O.sparse_attn(cache, L.q, q_seq, idx, cnt, spec.sm_scale)
        elif L.mode == O.REINDEX:
            idx, cnt, o, lse = O.layer_step(O.REINDEX, cache, L.q, q_seq, q_vis, spec.k, spec.sm_scale,
                                            q_idx=L.q_idx, w=L.w)
        else:
            idx, cnt, o, lse = O.layer_step(O.REUSE, cache, L.q, q_seq, q_vis, spec.k, spec.sm_scale,
                                            idx=full_idx, cnt=full_cnt)
        results.append(dict(idx=idx, cnt=cnt, out=o, lse=lse))
    return results
