"""Pins of the oracle's hierarchical indexer (Reindex restricted to the
candidate pool an earlier indexer chose): a pool of every visible entry gives
the exhaustive Top-K; the same query over its own Top-P pool gives its Top-K;
rank counting with Python integers on small pools; short pools."""
import numpy as np
import pytest

from oracle import csa2_oracle as O
from tests.test_oracle_select_attend import _tiny_cache


def _q(rng, nq, h, integer=True):
    qi = rng.integers(-8, 9, size=(nq, h, 128)) if integer else rng.standard_normal((nq, h, 128))
    return O.e4m3fn_encode(qi.astype(np.float64)), qi


@pytest.mark.parametrize("seed", range(3))
def test_pool_of_everything_is_exhaustive_topk(seed):
    rng = np.random.default_rng(40 + seed)
    n = int(rng.integers(20, 200))
    cache, _ = _tiny_cache(rng, n, integer=False)
    qb, _ = _q(rng, 1, 4, integer=False)
    w = rng.standard_normal((1, 4))
    k = int(rng.integers(1, 40))
    want = O.index_topk(cache, qb, w, [0], [n], k)
    pool = np.arange(n, dtype=np.int32)[None]
    got = O.pool_index_topk(cache, qb, w, [0], pool, [n], k)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_own_topP_pool_gives_own_topk():
    rng = np.random.default_rng(50)
    n = 300
    cache, _ = _tiny_cache(rng, n)
    qb, _ = _q(rng, 2, 8)
    w = rng.integers(1, 3, size=(2, 8)).astype(np.float64)
    pool, pcnt = O.index_topk(cache, qb, w, [0, 0], [n, 250], 64)
    got = O.pool_index_topk(cache, qb, w, [0, 0], pool, pcnt, 16)
    want = O.index_topk(cache, qb, w, [0, 0], [n, 250], 16)
    assert np.array_equal(got[0], want[0]) and np.array_equal(got[1], want[1])


def test_pool_matches_rank_counting_with_integers():
    rng = np.random.default_rng(51)
    n, H = 120, 3
    cache, ik = _tiny_cache(rng, n)
    qb, qi = _q(rng, 1, H)
    w = rng.integers(-2, 3, size=(1, H))
    pool = np.sort(rng.choice(n, size=40, replace=False)).astype(np.int32)
    k = 7
    got, cnt = O.pool_index_topk(cache, qb, w.astype(np.float64), [0], pool[None], [40], k)
    score = {int(t): sum(int(w[0, h]) * max(0, sum(int(qi[0, h, d]) * int(ik[t, d]) for d in range(128)))
                         for h in range(H)) for t in pool}
    rank = {t: sum(1 for u in pool if (score[int(u)], -int(u)) > (score[t], -t)) for t in score}
    want = sorted(t for t in score if rank[t] < k)
    assert cnt[0] == k and list(got[0]) == want


def test_short_pool_takes_everything():
    rng = np.random.default_rng(52)
    cache, _ = _tiny_cache(rng, 50)
    qb, _ = _q(rng, 1, 2)
    pool = np.array([[3, 9, 30, -1, -1]], dtype=np.int32)
    idx, cnt = O.pool_index_topk(cache, qb, np.ones((1, 2)), [0], pool, [3], 8)
    assert cnt[0] == 3 and list(idx[0]) == [3, 9, 30, -1, -1, -1, -1, -1]
