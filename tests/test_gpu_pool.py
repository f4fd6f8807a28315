"""GPU parity of the hierarchical indexer: the pool scoring and Top-k of
csa2_pool_index_topk, and layer steps with CSA2_STEP_POOL, against the fp64
oracle (integer indexer inputs: bit-exact) and against the exhaustive indexer
(pools that hold every entry: bit-identical on N(0,1) inputs)."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import csa2_oracle as O
from tests import casebuild as CB
from tests.gpu_util import (LSE_RTOL, OUT_ATOL, OVERLAP_MIN, check_selection_valid, need_gpu, overlap_stats, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _ops():
    from fp4_kv_cache_layer_amd import ops, runner
    return ops, runner


def _oracle_cache_after_step(case):
    c = case.fresh_cache()
    if case.new_slots.size:
        O.append_quant_fp4(c, case.new_slots, case.new_kv, case.new_ik)
    return c


def _random_pools(rng, vis, p, counts):
    """Ascending random subsets of [0, vis) of the given sizes, -1 padded to p."""
    pool = np.full((len(vis), p), -1, dtype=np.int32)
    for i, (v, c) in enumerate(zip(vis, counts)):
        pool[i, :c] = np.sort(rng.choice(v, size=c, replace=False))
    return pool, np.asarray(counts, dtype=np.int32)


def _check_attn(spec, ocache, L, g):
    q_seq = spec.q_seq()
    o_ref, lse_ref = O.sparse_attn(ocache, L.q, q_seq, g["idx"], g["cnt"], spec.sm_scale)
    err = np.abs(g["out"] - o_ref).max()
    assert err <= OUT_ATOL, err
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(g["lse"]), fin)
    lerr = np.abs(g["lse"][fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
    assert lerr.size == 0 or lerr.max() <= LSE_RTOL, lerr.max()
    return err


@pytest.mark.parametrize("seed,cached,k,pool_k,h_idx", [
    (61, [3000, 777, 1500, 0, 5000], 256, 1024, 8),
    (62, [9000, 2100], 512, 2048, 16),
    (63, [700, 64, 2047], 64, 100, 4),
    (64, [4000], 300, 300, 1),
])
def test_pool_group_integer_exact(seed, cached, k, pool_k, h_idx):
    """Full keeps its Top-pool_k as the pool; Reindex layers select in it; one
    group step gives the same bits as the per-layer calls."""
    _, runner = _ops()
    spec = W.small_case("pool_int", seed, cached, n_new=1, h_idx=h_idx, h=16, k=k, integer_indexer=True,
                        modes=(W.FULL, W.REINDEX, W.REUSE, W.REINDEX), pool_k=pool_k)
    say(f"[pool group] seed={seed} cached={cached} k={k} pool_k={pool_k} h_idx={h_idx}")
    dc = runner.DeviceCase(spec, gen_device="cpu", group=2)
    dc.run_layers()
    got = dc.results_host()
    pool, pool_cnt = dc.pool.cpu().numpy(), dc.pool_cnt.cpu().numpy()
    case = CB.build(spec)
    ref = CB.run_group(case)
    assert np.array_equal(pool_cnt, ref[0]["pool_cnt"])
    for i in range(spec.nq):
        assert np.array_equal(pool[i, :pool_cnt[i]], ref[0]["pool"][i, :pool_cnt[i]]), f"pool row {i}"
    ocache = _oracle_cache_after_step(case)
    for li, (g, r, L) in enumerate(zip(got, ref, case.layers)):
        assert np.array_equal(g["cnt"], r["cnt"]), f"layer {li} cnt"
        bad = np.nonzero((g["idx"] != r["idx"]).any(1))[0]
        assert bad.size == 0, f"layer {li}: {bad.size} queries differ, first {bad[:3]}"
        err = _check_attn(spec, ocache, L, g)
        say(f"  layer {li} mode {L.mode}: max|dO| {err:.2e}")
    dc.run_group()
    for g, h in zip(dc.results_host(), got):
        for key in ("idx", "cnt", "out", "lse"):
            assert np.array_equal(g[key], h[key]), f"group step differs in {key}"


@pytest.mark.parametrize("p,k,counts", [
    (1024, 256, [1024, 0, 200, 1, 1024]),
    (1000, 512, [1000, 999, 513, 512, 17]),
    (64, 64, [64, 63, 1, 0, 64]),
    (2048, 2048, [2048, 1, 2000, 1500, 0]),
])
def test_pool_index_direct_integer_exact(p, k, counts):
    """csa2_pool_index_topk on arbitrary ascending pools (ragged counts,
    empty pools, pools narrower than k) against the oracle, bit-exact."""
    ops, runner = _ops()
    cached = [3000, 2100, 2500, 40, 4100]
    spec = W.small_case("pool_direct", 65, cached, n_new=1, h_idx=8, h=16, k=k, integer_indexer=True,
                        modes=(W.FULL,))
    say(f"[pool direct] p={p} k={k} counts={counts}")
    dc = runner.DeviceCase(spec, gen_device="cpu")
    dc.run_layers()                                   # appends the new rows
    vis = spec.q_vis()
    rng = np.random.default_rng(p + k)
    pool, cnt = _random_pools(rng, vis, p, [min(c, int(v)) for c, v in zip(counts, vis)])
    qi, w, _ = dc.inputs[0]
    gi, gc = ops.csa2_pool_index_topk(dc.cache, qi, w, dc.q_seq, torch.from_numpy(pool).cuda(),
                                      torch.from_numpy(cnt).cuda(), k)
    torch.cuda.synchronize()
    case = CB.build(spec)
    ocache = _oracle_cache_after_step(case)
    ri, rc = O.pool_index_topk(ocache, case.layers[0].q_idx, case.layers[0].w, spec.q_seq(), pool, cnt, k)
    assert np.array_equal(gc.cpu().numpy(), rc)
    assert np.array_equal(gi.cpu().numpy(), ri)


@pytest.mark.parametrize("seed,cached", [(66, [2000, 1000, 1500, 300]), (67, [2047])])
def test_pool_of_every_entry_matches_exhaustive_indexer(seed, cached):
    """On N(0,1) inputs: a pool holding every visible entry scores each entry
    with the exhaustive scan's bits, so the selection is bit-identical."""
    ops, runner = _ops()
    spec = W.small_case("pool_all", seed, cached, n_new=1, h_idx=8, h=16, k=512, integer_indexer=False,
                        modes=(W.FULL,))
    dc = runner.DeviceCase(spec, gen_device="cpu")
    dc.run_layers()
    vis = spec.q_vis()
    p = 2048
    pool = np.full((spec.nq, p), -1, dtype=np.int32)
    for i, v in enumerate(vis):
        pool[i, :v] = np.arange(v)
    qi, w, _ = dc.inputs[0]
    gi, gc = ops.csa2_pool_index_topk(dc.cache, qi, w, dc.q_seq, torch.from_numpy(pool).cuda(),
                                      torch.from_numpy(vis.astype(np.int32)).cuda(), spec.k)
    ws = ops.workspace(ops.FULL, spec.nq, dc.max_vis, spec.h_idx, spec.h, spec.k)
    ei, ec = ops.csa2_index_topk(dc.cache, qi, w, dc.q_seq, dc.q_vis, spec.k, dc.max_vis, ws)
    torch.cuda.synchronize()
    assert torch.equal(gc, ec) and torch.equal(gi, ei)


@pytest.mark.parametrize("seed,cached,pool_k", [(68, [1500, 900, 2000], 2048), (69, [6000, 3000, 777], 1024)])
def test_pool_layers_gaussian(seed, cached, pool_k):
    """N(0,1) inputs.  The Full layer's selection is bit-identical with and
    without the pool; the pool is a valid Top-pool_k; Reindex selections are
    valid Top-k of the pool the GPU chose (near-ties aside) and, when the pool
    holds every entry, bit-identical to the exhaustive Reindex."""
    _, runner = _ops()
    modes = (W.FULL, W.REINDEX, W.REUSE)
    base = W.small_case("pool_gauss", seed, cached, n_new=1, h_idx=8, h=32, k=512, integer_indexer=False,
                        modes=modes)
    spec = W.small_case("pool_gauss", seed, cached, n_new=1, h_idx=8, h=32, k=512, integer_indexer=False,
                        modes=modes, pool_k=pool_k)
    say(f"[pool gauss] seed={seed} cached={cached} pool_k={pool_k}")
    dp = runner.DeviceCase(spec, gen_device="cpu")
    dp.run_layers()
    got = dp.results_host()
    pool, pool_cnt = dp.pool.cpu().numpy(), dp.pool_cnt.cpu().numpy()
    db = runner.DeviceCase(base, gen_device="cpu")
    db.run_layers()
    plain = db.results_host()
    for key in ("idx", "cnt", "out", "lse"):
        assert np.array_equal(got[0][key], plain[0][key]), f"Full layer differs with the pool in {key}"
    every = all(int(v) <= pool_k for v in spec.q_vis())
    if every:
        for key in ("idx", "cnt", "out", "lse"):
            assert np.array_equal(got[1][key], plain[1][key]), f"Reindex differs in {key}"
    case = CB.build(spec)
    ocache = _oracle_cache_after_step(case)
    q_seq, q_vis = spec.q_seq(), spec.q_vis()
    L0, L1 = case.layers[0], case.layers[1]
    ri, rc = O.index_topk(ocache, L0.q_idx, L0.w, q_seq, q_vis, pool_k)
    ov, worst = overlap_stats(pool, pool_cnt, ri, rc)
    say(f"  pool overlap {ov:.6f} worst {worst:.4f}")
    assert ov >= OVERLAP_MIN
    for i in range(spec.nq):
        sc = O.index_scores(ocache, int(q_seq[i]), int(q_vis[i]), L0.q_idx[i], L0.w[i])
        check_selection_valid(pool[i], pool_cnt[i], ri[i], rc[i], sc, pool_k)
    # Reindex: against the oracle's Top-k of the GPU's pool
    oi, oc = O.pool_index_topk(ocache, L1.q_idx, L1.w, q_seq, pool, pool_cnt, spec.k)
    ov, worst = overlap_stats(got[1]["idx"], got[1]["cnt"], oi, oc)
    say(f"  reindex overlap {ov:.6f} worst {worst:.4f}")
    assert ov >= OVERLAP_MIN
    for i in range(spec.nq):
        full = O.index_scores(ocache, int(q_seq[i]), int(q_vis[i]), L1.q_idx[i], L1.w[i])
        sc = np.full(full.shape, -np.inf)
        sc[pool[i, :pool_cnt[i]]] = full[pool[i, :pool_cnt[i]]]
        check_selection_valid(got[1]["idx"][i], got[1]["cnt"][i], oi[i], oc[i], sc, spec.k)
        assert set(got[1]["idx"][i, :got[1]["cnt"][i]].tolist()) <= set(pool[i, :pool_cnt[i]].tolist())
    for li in range(3):
        _check_attn(spec, ocache, case.layers[li], got[li])


@pytest.mark.parametrize("seed,cached,n_new,k,pool_k", [(71, [700], 37, 64, 256), (72, [3000], 130, 128, 512)])
def test_pool_prefill_dense_integer_exact(seed, cached, n_new, k, pool_k):
    """Prefill chunk through the dense indexer with the hierarchical indexer:
    the Full layer's dense Top-pool_k is the pool, the Reindex layer rescores
    only the pool (its dense flag has no effect); bit-exact against the
    oracle on integer inputs."""
    _, runner = _ops()
    spec = W.small_case("pool_prefill", seed, cached, n_new=n_new, h_idx=8, h=16, k=k, integer_indexer=True,
                        modes=(W.FULL, W.REINDEX, W.REUSE), prefill=True, pool_k=pool_k)
    say(f"[pool prefill] seed={seed} cached={cached} n_new={n_new} k={k} pool_k={pool_k}")
    dc = runner.DeviceCase(spec, gen_device="cpu")
    assert dc.dense
    dc.run_layers()
    got = dc.results_host()
    pool, pool_cnt = dc.pool.cpu().numpy(), dc.pool_cnt.cpu().numpy()
    case = CB.build(spec)
    ref = CB.run_group(case)
    assert np.array_equal(pool_cnt, ref[0]["pool_cnt"])
    for i in range(spec.nq):
        assert np.array_equal(pool[i, :pool_cnt[i]], ref[0]["pool"][i, :pool_cnt[i]]), f"pool row {i}"
    ocache = _oracle_cache_after_step(case)
    for li, (g, r, L) in enumerate(zip(got, ref, case.layers)):
        assert np.array_equal(g["cnt"], r["cnt"]), f"layer {li} cnt"
        bad = np.nonzero((g["idx"] != r["idx"]).any(1))[0]
        assert bad.size == 0, f"layer {li}: {bad.size} queries differ, first {bad[:3]}"
        _check_attn(spec, ocache, L, g)
