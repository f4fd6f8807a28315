"""Pins of the oracle's block-level pruning (block_bounds, block_score_bound,
prune_threshold, pruned_index_topk) against brute force: every row's score
against its block's bound, the bound attained at the box's worst corner, and
the pruned Top-K against the exhaustive one."""
import numpy as np
import pytest

import workloads as W
from oracle import csa2_oracle as O


def _cache_of(spec):
    pt = W.page_table(spec)
    cache = O.Cache.empty(spec.total_pages(), spec.page_size, pt, [spec.seq_len_after(s) for s in range(spec.num_seqs)])
    for s in range(spec.num_seqs):
        n = spec.seq_len_after(s)
        slots = W.slots_for(spec, pt, s, 0, n)
        O.append_quant_fp4(cache, slots, W.kv_rows(spec, s).numpy().view(np.uint16),
                           W.idxk_rows(spec, s).numpy().view(np.uint16))
    return cache


def _random_e4m3(rng, shape):
    b = rng.integers(0, 256, size=shape, dtype=np.uint8)
    return np.where((b & 0x7F) == 0x7F, b & 0xF0, b).astype(np.uint8)      # no NaN codes


def test_bound_holds_for_every_row():
    rng = np.random.default_rng(5)
    nb = 40
    cache = O.Cache.empty(nb, O.PRUNE_BLOCK, np.arange(nb, dtype=np.int32)[None], [nb * O.PRUNE_BLOCK])
    cache.idx_k[:] = _random_e4m3(rng, cache.idx_k.shape)
    bmax, bmin = O.block_bounds(cache)
    for trial in range(6):
        qi = _random_e4m3(rng, (8, O.D_INDEX))
        w = rng.normal(size=8)                                              # negative weights included
        sc = O.index_scores(cache, 0, nb * O.PRUNE_BLOCK, qi, w)
        ub = O.block_score_bound(qi, w, bmax, bmin)
        per_block = sc.reshape(nb, O.PRUNE_BLOCK).max(axis=1)
        assert (per_block <= ub + 1e-9 * np.abs(ub)).all(), trial


def test_bound_is_exact_for_a_constant_block():
    rng = np.random.default_rng(6)
    cache = O.Cache.empty(1, O.PRUNE_BLOCK, np.zeros((1, 1), np.int32), [O.PRUNE_BLOCK])
    cache.idx_k[0, :] = _random_e4m3(rng, (1, O.D_INDEX))
    bmax, bmin = O.block_bounds(cache)
    qi = _random_e4m3(rng, (4, O.D_INDEX))
    w = np.array([1.5, -0.75, 2.0, -3.0])
    sc = O.index_scores(cache, 0, O.PRUNE_BLOCK, qi, w)
    assert np.allclose(sc, sc[0], rtol=0, atol=0)
    assert O.block_score_bound(qi, w, bmax[0], bmin[0]) == pytest.approx(sc[0], rel=1e-12, abs=1e-12)


@pytest.mark.parametrize("weight", [1.0, -1.0])
def test_bound_is_attained_at_the_worst_corner(weight):
    """One head: the bound equals the score of the box corner that takes the
    upper end of every dimension where q_d >= 0 (lower end elsewhere) for a
    positive weight, the other way round for a negative one."""
    rng = np.random.default_rng(7 if weight > 0 else 8)
    cache = O.Cache.empty(2, O.PRUNE_BLOCK, np.arange(2, dtype=np.int32)[None], [2 * O.PRUNE_BLOCK])
    cache.idx_k[0] = _random_e4m3(rng, (O.PRUNE_BLOCK, O.D_INDEX))
    bmax, bmin = O.block_bounds(cache)
    kmax = cache.idx_k[0][np.argmax(O.e4m3fn_decode(cache.idx_k[0]), axis=0), np.arange(O.D_INDEX)]
    kmin = cache.idx_k[0][np.argmin(O.e4m3fn_decode(cache.idx_k[0]), axis=0), np.arange(O.D_INDEX)]
    for _ in range(5):
        qi = _random_e4m3(rng, (1, O.D_INDEX))
        q = O.e4m3fn_decode(qi)[0]
        up = (q >= 0) if weight > 0 else (q < 0)
        cache.idx_k[1, 0] = np.where(up, kmax, kmin)                       # the corner row
        corner = O.index_scores(cache, 0, O.PRUNE_BLOCK + 1, qi, [weight])[O.PRUNE_BLOCK]
        assert O.block_score_bound(qi, [weight], bmax[0], bmin[0]) == pytest.approx(corner, rel=1e-12, abs=1e-12)


def _check_pruned(spec, seeds, expect_pruning):
    cache = _cache_of(spec)
    qi, w, _ = W.layer_queries(spec, 0)
    qi, w = qi.numpy(), w.numpy()
    q_seq, q_vis = spec.q_seq(), spec.q_vis()
    ref_idx, ref_cnt = O.index_topk(cache, qi, w, q_seq, q_vis, spec.k)
    seed, seed_cnt = seeds(cache, qi, w, q_seq, q_vis, ref_idx, ref_cnt)
    idx, cnt, masks = O.pruned_index_topk(cache, qi, w, q_seq, q_vis, seed, seed_cnt, spec.k)
    assert np.array_equal(idx, ref_idx) and np.array_equal(cnt, ref_cnt)
    frac = np.mean(np.concatenate(masks))
    if expect_pruning:
        assert frac > 0.3, frac
    else:
        assert frac == 0.0, frac
    # the threshold never exceeds the k-th largest score
    for i in range(len(q_seq)):
        sc = O.index_scores(cache, int(q_seq[i]), int(q_vis[i]), qi[i], w[i])
        thr = O.prune_threshold(cache, int(q_seq[i]), int(q_vis[i]), qi[i], w[i], seed[i][:seed_cnt[i]], spec.k)
        if int(q_vis[i]) >= spec.k:
            assert thr <= np.sort(sc)[::-1][spec.k - 1]
    return frac


def _exact_seed(cache, qi, w, q_seq, q_vis, ref_idx, ref_cnt):
    return ref_idx, ref_cnt


def _random_seed(cache, qi, w, q_seq, q_vis, ref_idx, ref_cnt):
    rng = np.random.default_rng(9)
    k = ref_idx.shape[1]
    seed = np.stack([rng.choice(int(v), size=k, replace=False) for v in q_vis]).astype(np.int32)
    return seed, np.full(len(q_vis), k, np.int32)


def _messy_seed(cache, qi, w, q_seq, q_vis, ref_idx, ref_cnt):
    """The exact Top-K with duplicates, negative and out-of-range entries
    mixed in: only its distinct visible entries count."""
    k = ref_idx.shape[1]
    seed = ref_idx.copy()
    seed[:, 1::7] = seed[:, 0:1]                       # duplicates
    seed[:, 2::11] = -5
    seed[:, 3::13] = np.asarray(q_vis)[:, None] + 3    # past the visible range
    return seed, np.full(len(q_vis), k, np.int32)


def _short_seed(cache, qi, w, q_seq, q_vis, ref_idx, ref_cnt):
    return ref_idx, np.full(len(q_vis), ref_idx.shape[1] - 1, np.int32)


@pytest.mark.parametrize("integer", [True, False])
def test_pruned_topk_is_exact_and_prunes_clustered_blocks(integer):
    spec = W.small_case("prune_clustered", 21 if integer else 22, [6000, 3500], k=128, clustered=True,
                        integer_indexer=integer, modes=(W.FULL,), page_size=128)
    _check_pruned(spec, _exact_seed, expect_pruning=True)


@pytest.mark.parametrize("seeds", [_random_seed, _messy_seed])
def test_pruned_topk_is_exact_with_other_seeds(seeds):
    spec = W.small_case("prune_seeds", 23, [5000, 2600], k=128, clustered=True, integer_indexer=True,
                        modes=(W.FULL,), page_size=64)
    cache = _cache_of(spec)
    qi, w, _ = W.layer_queries(spec, 0)
    qi, w = qi.numpy(), w.numpy()
    ref_idx, ref_cnt = O.index_topk(cache, qi, w, spec.q_seq(), spec.q_vis(), spec.k)
    seed, seed_cnt = seeds(cache, qi, w, spec.q_seq(), spec.q_vis(), ref_idx, ref_cnt)
    idx, cnt, _ = O.pruned_index_topk(cache, qi, w, spec.q_seq(), spec.q_vis(), seed, seed_cnt, spec.k)
    assert np.array_equal(idx, ref_idx) and np.array_equal(cnt, ref_cnt)


def test_short_seed_prunes_nothing():
    spec = W.small_case("prune_short", 24, [3000], k=128, clustered=True, integer_indexer=True,
                        modes=(W.FULL,), page_size=64)
    _check_pruned(spec, _short_seed, expect_pruning=False)


def test_unclustered_gaussian_blocks_are_not_pruned():
    """N(0,1) rows: every 64-row box is wide, so even the exact Top-K as seed
    prunes nothing (the bench workload's situation)."""
    spec = W.small_case("prune_gauss", 25, [4000, 2000], k=128, modes=(W.FULL,), page_size=64)
    _check_pruned(spec, _exact_seed, expect_pruning=False)
