"""Pins for the oracle's layer modes and cache layout (CPU only).

Reuse hands on the earlier layer's indices bit for bit; Reindex with the Full
layer's own indexer query reproduces the Full layer's selection; the physical
page layout and the batch order do not change any result; the decode append
is visible to the step that appends it.
"""
import dataclasses

import numpy as np

import workloads as W
from oracle import csa2_oracle as O
from tests import casebuild as CB


def _small(seed=11, **kw):
    base = dict(cached=[200, 37, 513, 64], n_new=1, h_idx=4, h=8, k=64)
    base.update(kw)
    return W.small_case("modes", seed, **base)


def test_reuse_returns_source_indices_bit_for_bit():
    case = CB.build(_small())
    res = CB.run_group(case)
    assert [L.mode for L in case.layers] == [O.FULL, O.REINDEX, O.REUSE, O.REUSE]
    for r in res[2:]:
        assert np.array_equal(r["idx"], res[0]["idx"]) and np.array_equal(r["cnt"], res[0]["cnt"])


def test_reindex_with_full_query_reproduces_full_selection():
    case = CB.build(_small(seed=12))
    case.layers[1] = dataclasses.replace(case.layers[1], q_idx=case.layers[0].q_idx, w=case.layers[0].w)
    res = CB.run_group(case)
    assert np.array_equal(res[1]["idx"], res[0]["idx"])


def test_page_layout_does_not_matter():
    a = CB.run_group(CB.build(_small(seed=13, shuffle_pages=True, page_size=16)))
    b = CB.run_group(CB.build(_small(seed=13, shuffle_pages=False, page_size=64, extra_pages=0)))
    for ra, rb in zip(a, b):
        for key in ("idx", "cnt", "out", "lse"):
            assert np.array_equal(ra[key], rb[key]), key


def test_batch_order_permutes_results():
    spec = _small(seed=14)
    case = CB.build(spec)
    res = CB.run_group(case)
    perm = np.array([2, 0, 3, 1])
    cache = case.fresh_cache()
    O.append_quant_fp4(cache, case.new_slots, case.new_kv, case.new_ik)
    L = case.layers[0]
    q_seq, q_vis = spec.q_seq()[perm], spec.q_vis()[perm]
    idx, cnt = O.index_topk(cache, L.q_idx[perm], L.w[perm], q_seq, q_vis, spec.k)
    o, lse = O.sparse_attn(cache, L.q[perm], q_seq, idx, cnt, spec.sm_scale)
    assert np.array_equal(idx, res[0]["idx"][perm])
    assert np.array_equal(o, res[0]["out"][perm]) and np.array_equal(lse, res[0]["lse"][perm])


def test_appended_entry_is_visible_and_short_sequences_pad():
    spec = _small(seed=15, integer_indexer=True)
    case = CB.build(spec)
    res = CB.run_group(case)
    for i, s in enumerate(spec.q_seq()):
        v = spec.seq_len_after(int(s))
        kp = min(spec.k, v)
        assert res[0]["cnt"][i] == kp
        assert (res[0]["idx"][i, kp:] == -1).all()
        assert (res[0]["idx"][i, :kp] < v).all()
    # sequence 1 has 38 visible entries < k: every entry, including the appended one, is selected
    assert list(res[0]["idx"][1, :38]) == list(range(38))


def test_full_mode_writes_the_appended_rows():
    spec = _small(seed=16)
    case = CB.build(spec)
    cache = case.fresh_cache()
    L = case.layers[0]
    O.layer_step(O.FULL, cache, L.q, spec.q_seq(), spec.q_vis(), spec.k, spec.sm_scale,
                 q_idx=L.q_idx, w=L.w, new_slots=case.new_slots, new_kv=case.new_kv, new_idxk=case.new_ik)
    for s in range(spec.num_seqs):
        t = spec.cached[s]
        row = cache.kv_rows(s, [t])[0]
        assert np.array_equal(row, O.quantize_kv_rows(O.bf16_to_f64(case.kv_src[s][t])[None])[0])


def test_prefill_is_causal():
    spec = W.small_case("prefill", 17, cached=[300], n_new=40, h_idx=4, h=4, k=32,
                        modes=(O.FULL,), prefill=True)
    case = CB.build(spec)
    res = CB.run_group(case)
    vis = spec.q_vis()
    assert list(vis[:3]) == [301, 302, 303]
    for i in range(spec.nq):
        sel = res[0]["idx"][i, :res[0]["cnt"][i]]
        assert (sel < vis[i]).all()
