"""Full-size workloads on the GPU, in the launch configuration the benchmark
times, checked against the fp64 oracle on sampled queries (each sampled
query is scored over its whole visible context by the oracle)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import csa2_oracle as O
from tests.gpu_util import (LSE_RTOL, OUT_ATOL, OVERLAP_MIN, add_kv_rows, check_selection_valid, need_gpu,
                            overlap_stats, say, single_seq_cache)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _check_sampled(spec, sample, exact=False):
    from fp4_kv_cache_layer_amd import runner
    say(f"[fullsize] {spec.name}: building ({spec.num_seqs} seqs, {sum(spec.cached)} cached entries)")
    dc = runner.DeviceCase(spec, gen_device="cuda")
    say(f"[fullsize] {spec.name}: running group {spec.modes}")
    dc.run_group()
    got = dc.results_host()
    q_seq, q_vis = spec.q_seq(), spec.q_vis()
    full_idx = got[0]["idx"]
    if spec.pool_k:
        pool, pool_cnt = dc.pool.cpu().numpy(), dc.pool_cnt.cpu().numpy()
    inter = total = 0
    for i in sample:
        s, vis = int(q_seq[i]), int(q_vis[i])
        say(f"  query {i} seq {s} vis {vis}")
        cache = single_seq_cache(spec, s, vis, "cuda")
        sel_rows = set()
        for li, mode in enumerate(spec.modes):
            g = got[li]
            qi, w, q = (x.cpu().numpy() for x in dc.inputs[li])
            if mode == O.FULL and spec.pool_k:
                # the pool: this layer's Top-pool_k
                sc = O.index_scores(cache, 0, vis, qi[i], w[i])
                pi, pc = O.select_topk(sc, spec.pool_k)
                if exact:
                    assert pool_cnt[i] == pc and np.array_equal(pool[i, :pc], pi[:pc])
                else:
                    check_selection_valid(pool[i], pool_cnt[i], pi, pc, sc, spec.pool_k)
            if mode == O.REINDEX and spec.pool_k:
                # Top-k of the GPU's pool: exact on integer inputs, else valid up to near-ties
                oi, oc = O.pool_index_topk(cache, qi[i:i + 1], w[i:i + 1], np.zeros(1, np.int32), pool[i:i + 1],
                                           pool_cnt[i:i + 1], spec.k)
                oi, oc = oi[0], int(oc[0])
                full = O.index_scores(cache, 0, vis, qi[i], w[i])
                sc = np.full(full.shape, -np.inf)
                sc[pool[i, :pool_cnt[i]]] = full[pool[i, :pool_cnt[i]]]
                if exact:
                    assert g["cnt"][i] == oc and np.array_equal(g["idx"][i], oi)
                else:
                    check_selection_valid(g["idx"][i], g["cnt"][i], oi, oc, sc, spec.k)
            elif mode != O.REUSE:
                sc = O.index_scores(cache, 0, vis, qi[i], w[i])
                oi, oc = O.select_topk(sc, spec.k)
                if exact:
                    assert g["cnt"][i] == oc and np.array_equal(g["idx"][i], oi)
                else:
                    ov, _ = overlap_stats(g["idx"][i:i + 1], g["cnt"][i:i + 1], oi[None], [oc])
                    say(f"    layer {li}: overlap {ov:.5f}")
                    inter += round(ov * oc)
                    total += oc
                    check_selection_valid(g["idx"][i], g["cnt"][i], oi, oc, sc, spec.k)
            else:
                assert np.array_equal(g["idx"][i], full_idx[i])
            sel_rows |= set(g["idx"][i, :g["cnt"][i]].tolist())
        add_kv_rows(cache, spec, s, sel_rows, "cuda")
        for li, mode in enumerate(spec.modes):
            g = got[li]
            q = dc.inputs[li][2].cpu().numpy().view(np.uint16)
            o, lse = O.attend(cache, 0, q[i], g["idx"][i], int(g["cnt"][i]), spec.sm_scale)
            err = np.abs(g["out"][i] - o).max()
            lerr = np.max(np.abs(g["lse"][i] - lse) / np.maximum(1, np.abs(lse)))
            say(f"    layer {li}: max|dO| {err:.2e} lse rel {lerr:.1e}")
            assert err <= OUT_ATOL and lerr <= LSE_RTOL
    if total:
        say(f"  aggregate overlap {inter / total:.6f}")
        assert inter / total >= OVERLAP_MIN
    del dc
    torch.cuda.empty_cache()


def test_config1_decode_b32_64k_group():
    _check_sampled(W.config(1), sample=[0, 17, 31])


def test_config1_integer_exact():
    _check_sampled(W.config(1, integer_indexer=True), sample=[5, 30], exact=True)


def test_config1_hierarchical_indexer_integer_exact():
    """The decode workload with a 2,048-entry pool: the Full layer's pool and
    selection and the Reindex layer's selection in the pool, bit-exact."""
    import dataclasses
    _check_sampled(dataclasses.replace(W.config(1, integer_indexer=True), pool_k=2048), sample=[3, 28], exact=True)


def test_config1_hierarchical_indexer_gaussian():
    import dataclasses
    _check_sampled(dataclasses.replace(W.config(1), pool_k=2048), sample=[0, 31])


def test_config2_prefill_sampled_rows():
    _check_sampled(W.config(2), sample=[0, 1, 2047, 4095])


def test_config3_decode_1m():
    _check_sampled(W.config(3), sample=[0, 7])


def test_config4_ragged_paged():
    spec = W.config(4)
    lens = np.array(spec.cached)
    sample = sorted({int(lens.argmin()), int(lens.argmax()), int(np.argsort(lens)[len(lens) // 2])})
    _check_sampled(spec, sample=sample)


def test_config3_decode_1m_integer_exact():
    """The 1M-entry decode workload on integer indexer inputs: the scan over
    512 chunks per query, the chip-wide collect and the bitonic output path
    (contexts past 262,144 entries), bit-exact against the oracle."""
    _check_sampled(W.config(3, integer_indexer=True), sample=[0, 7], exact=True)


def test_config4_ragged_paged_integer_exact():
    """The ragged paged group on integer indexer inputs, bit-exact, on the
    shortest and the longest sequence."""
    spec = W.config(4, integer_indexer=True)
    lens = np.array(spec.cached)
    _check_sampled(spec, sample=sorted({int(lens.argmin()), int(lens.argmax())}), exact=True)


def test_config2_prefill_integer_exact():
    """The full prefill chunk through the dense indexer on integer inputs,
    bit-exact on the first, second, middle and last rows."""
    _check_sampled(W.config(2, integer_indexer=True), sample=[0, 1, 2047, 4095], exact=True)


@pytest.mark.parametrize("k", [500, 2048])
def test_long_context_bitonic_output_integer_exact(k):
    """One query over about 300K entries (past the 262,144-entry bitmap, so
    the select sorts its output bitonically) with integer indexer inputs, at
    a k that is not a power of two (padding) and at the largest k."""
    spec = W.small_case("bitonic", 90 + k, [300007], n_new=1, h_idx=8, h=16, k=k, modes=(O.FULL,),
                        integer_indexer=True, page_size=4096, shuffle_pages=True)
    _check_sampled(spec, sample=[0], exact=True)


def test_config1_group_step_equals_layer_calls():
    """The benchmark's group step (Reuse attentions on an auxiliary stream)
    against the per-layer calls on the full decode workload: identical bits."""
    from fp4_kv_cache_layer_amd import runner
    spec = W.config(1)
    say(f"[fullsize] {spec.name}: group step vs layer calls")
    dc = runner.DeviceCase(spec, gen_device="cuda", group=1)
    dc.run_layers()
    want = dc.results_host()
    for rep in range(2):
        dc.run_group()
        got = dc.results_host()
        for li, (x, y) in enumerate(zip(got, want)):
            for key in ("idx", "cnt", "out", "lse"):
                assert np.array_equal(x[key], y[key]), (rep, li, key)
    del dc
    torch.cuda.empty_cache()


def test_prefill_sized_merge_and_fake_quant_sampled():
    """Branch merge and FP4 fake quantisation at the benchmark's prefill size
    (262,144 rows of 512), checked against the oracle on sampled rows."""
    from fp4_kv_cache_layer_amd import ops
    rows, dim = 4096 * 64, 512
    g = torch.Generator(device="cuda").manual_seed(12)
    oa = torch.randn(rows, dim, generator=g, device="cuda")
    ob = torch.randn(rows, dim, generator=g, device="cuda") * 2
    la = torch.randn(rows, generator=g, device="cuda") * 20
    lb = torch.randn(rows, generator=g, device="cuda") * 20
    say(f"[fullsize] merge and fake quant, {rows} rows of {dim}")
    o, lse = ops.csa2_lse_merge(oa, la, ob, lb)
    fq = ops.csa2_fake_quant_fp4(oa)
    fqb = ops.csa2_fake_quant_fp4(ob.to(torch.bfloat16))
    sample = torch.tensor([0, 1, 77, rows // 2, rows - 2, rows - 1], device="cuda")
    sa, sb = oa[sample].cpu().numpy(), ob[sample].cpu().numpy()
    ro, rl = O.lse_merge(sa, la[sample].cpu().numpy(), sb, lb[sample].cpu().numpy())
    got_o = o[sample].cpu().numpy()
    assert (np.abs(got_o - ro) <= 2e-6 * np.maximum(np.abs(sa), np.abs(sb)) + 1e-7).all()
    assert np.allclose(lse[sample].cpu().numpy(), rl, rtol=2e-7, atol=2e-7)
    want_fq = O.fake_quant_e2m1(sa.astype(np.float64)).astype(np.float32)
    assert np.array_equal(fq[sample].cpu().numpy().view(np.uint32), want_fq.view(np.uint32))
    sbb = ob.to(torch.bfloat16)[sample].float().cpu().numpy()
    want_fqb = O.fake_quant_e2m1(sbb.astype(np.float64)).astype(np.float32)
    assert np.array_equal(fqb[sample].float().cpu().numpy().view(np.uint32), want_fqb.view(np.uint32))
