"""Pins for the oracle's scoring, Top-K selection and attention (CPU only).

Scoring is checked against exact Python-integer arithmetic; Top-K against
brute-force subset enumeration (L <= 16) and pairwise rank counting (L <= 64);
attention against torch's own scaled_dot_product_attention in float64 when
k >= V (dense attention), and against closed forms at k = 1.
"""
import itertools

import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O


def _beats(s, a, b):
    """a is ranked ahead of b: higher score, or equal score and lower index."""
    return s[a] > s[b] or (s[a] == s[b] and a < b)


@pytest.mark.parametrize("seed", range(12))
def test_topk_matches_subset_enumeration(seed):
    rng = np.random.default_rng(seed)
    L = int(rng.integers(1, 17))
    s = rng.integers(-3, 4, size=L).astype(np.float64)       # many ties
    for k in sorted({1, 2, 3, L // 2 + 1, L, L + 3}):
        kp = min(k, L)
        winners = []
        for sub in itertools.combinations(range(L), kp):
            inside = set(sub)
            if all(_beats(s, a, b) for a in inside for b in range(L) if b not in inside):
                winners.append(sub)
        assert len(winners) == 1
        idx, cnt = O.select_topk(s, k)
        assert cnt == kp
        assert list(idx[:kp]) == list(winners[0])
        assert (idx[kp:] == -1).all()


@pytest.mark.parametrize("seed", range(8))
def test_topk_matches_rank_counting(seed):
    rng = np.random.default_rng(100 + seed)
    L = int(rng.integers(17, 65))
    s = rng.integers(-5, 6, size=L).astype(np.float64) * rng.choice([0.5, 1.0, 3.0])
    for k in (1, 7, 32, 64, 100):
        kp = min(k, L)
        rank = [sum(_beats(s, u, t) for u in range(L)) for t in range(L)]
        want = [t for t in range(L) if rank[t] < kp]
        idx, cnt = O.select_topk(s, k)
        assert cnt == kp and list(idx[:kp]) == want


def test_topk_all_equal_and_short():
    idx, cnt = O.select_topk(np.zeros(100), 10)
    assert cnt == 10 and list(idx) == list(range(10))
    idx, cnt = O.select_topk(np.ones(5), 512)
    assert cnt == 5 and list(idx[:5]) == list(range(5)) and (idx[5:] == -1).all()
    idx, cnt = O.select_topk(np.zeros(0), 4)
    assert cnt == 0 and (idx == -1).all()


def _tiny_cache(rng, n, integer=True, page_size=16, shuffle=True):
    npages = (n + page_size - 1) // page_size + 2
    perm = rng.permutation(npages).astype(np.int32) if shuffle else np.arange(npages, dtype=np.int32)
    mp = (n + page_size - 1) // page_size
    pt = perm[:mp][None, :]
    cache = O.Cache.empty(npages, page_size, pt, [n])
    t = np.arange(n)
    slots = pt[0, t // page_size].astype(np.int64) * page_size + t % page_size
    kv = rng.standard_normal((n, 512)).astype(np.float32)
    kv_bits = (kv.view(np.uint32) >> 16).astype(np.uint16)
    if integer:
        ik = rng.integers(-8, 9, size=(n, 128)).astype(np.float32)
    else:
        ik = rng.standard_normal((n, 128)).astype(np.float32)
    ik_bits = (ik.view(np.uint32) >> 16).astype(np.uint16)
    O.append_quant_fp4(cache, slots, kv_bits, ik_bits)
    return cache, ik


def test_scores_exact_against_python_integers():
    rng = np.random.default_rng(7)
    n, H = 40, 5
    cache, ik = _tiny_cache(rng, n)
    qi = rng.integers(-8, 9, size=(H, 128))
    w = rng.integers(-2, 3, size=H)
    q_bytes = O.e4m3fn_encode(qi.astype(np.float64))
    got = O.index_scores(cache, 0, n, q_bytes, w.astype(np.float64))
    for t in range(n):
        tot = 0
        for h in range(H):
            d = sum(int(qi[h, j]) * int(ik[t, j]) for j in range(128))
            tot += int(w[h]) * max(0, d)
        assert got[t] == tot
        if tot == 0:
            assert not np.signbit(got[t])       # zero scores are +0


def test_negative_weight_zero_score_is_plus_zero():
    rng = np.random.default_rng(8)
    cache, ik = _tiny_cache(rng, 8)
    qi = np.zeros((2, 128))
    s = O.index_scores(cache, 0, 8, O.e4m3fn_encode(qi), np.array([-1.0, -2.0]))
    assert (s == 0).all() and not np.signbit(s).any()
    idx, cnt = O.select_topk(s, 3)
    assert list(idx) == [0, 1, 2]


def test_index_topk_visibility_prefix():
    """A query sees only entries 0..vis-1."""
    rng = np.random.default_rng(9)
    cache, ik = _tiny_cache(rng, 50)
    qi = O.e4m3fn_encode(rng.integers(-8, 9, size=(1, 4, 128)).astype(np.float64))
    w = np.ones((1, 4))
    idx, cnt = O.index_topk(cache, qi, w, [0], [20], 64)
    assert cnt[0] == 20 and list(idx[0, :20]) == list(range(20))


def _torch_dense(q, x, scale):
    qt = torch.from_numpy(q)[:, None, :]                          # [H][1][512]: one query per head
    xt = torch.from_numpy(x)[None].expand(q.shape[0], -1, -1)     # [H][n][512]: K = V = X
    o = torch.nn.functional.scaled_dot_product_attention(qt, xt, xt, scale=scale)[:, 0]
    lse = torch.logsumexp(scale * (torch.from_numpy(q) @ torch.from_numpy(x).T), dim=1)
    return o.numpy(), lse.numpy()


@pytest.mark.parametrize("seed", range(4))
def test_attention_with_k_ge_V_is_dense_attention(seed):
    rng = np.random.default_rng(20 + seed)
    n = int(rng.integers(1, 90))
    cache, _ = _tiny_cache(rng, n)
    H = 6
    q = rng.standard_normal((H, 512)).astype(np.float32)
    q_bits = (q.view(np.uint32) >> 16).astype(np.uint16)
    scale = 1 / np.sqrt(512)
    qi = O.e4m3fn_encode(rng.integers(-8, 9, size=(1, 3, 128)).astype(np.float64))
    idx, cnt = O.index_topk(cache, qi, np.ones((1, 3)), [0], [n], 128)
    o, lse = O.attend(cache, 0, q_bits, idx[0], int(cnt[0]), scale)
    x = O.dequantize_kv_rows(cache.kv_rows(0, np.arange(n)))
    ro, rl = _torch_dense(O.bf16_to_f64(q_bits), x, scale)
    np.testing.assert_allclose(o, ro, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, rl, rtol=1e-13, atol=1e-13)


def test_attention_k1_is_the_row():
    rng = np.random.default_rng(30)
    cache, _ = _tiny_cache(rng, 30)
    q_bits = (rng.standard_normal((4, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    idx = np.array([17] + [-1] * 7, dtype=np.int32)
    o, lse = O.attend(cache, 0, q_bits, idx, 1, 0.1)
    x = O.dequantize_kv_rows(cache.kv_rows(0, [17]))[0]
    assert np.array_equal(o, np.broadcast_to(x, o.shape))
    np.testing.assert_allclose(lse, 0.1 * (O.bf16_to_f64(q_bits) @ x), rtol=1e-15)


def test_attention_output_within_row_hull():
    rng = np.random.default_rng(31)
    cache, _ = _tiny_cache(rng, 64)
    q_bits = (rng.standard_normal((8, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    sel = np.sort(rng.choice(64, 20, replace=False)).astype(np.int32)
    o, lse = O.attend(cache, 0, q_bits, sel, 20, 1 / np.sqrt(512))
    x = O.dequantize_kv_rows(cache.kv_rows(0, sel))
    assert (o >= x.min(0) - 1e-12).all() and (o <= x.max(0) + 1e-12).all()


def test_sparse_attention_over_a_selection_is_dense_attention_over_its_rows():
    """Several sequences in shuffled pages, selections shorter than k in
    arbitrary order with -1 padding: every query's output equals torch's
    dense attention over exactly its selected rows, located here through the
    workload's own slot arithmetic (page table row, page size) rather than
    the oracle's cache walk."""
    import workloads as W
    from tests import casebuild as CB
    spec = W.small_case("attn_subset", 33, [700, 1500, 90], n_new=0, h=4, k=128, modes=(O.FULL,), page_size=64)
    case = CB.build(spec)
    cache = case.fresh_cache()
    rng = np.random.default_rng(34)
    q_seq, q_vis = spec.q_seq(), spec.q_vis()
    nq, k = len(q_seq), spec.k
    idx = np.full((nq, k), -1, dtype=np.int32)
    cnt = np.zeros(nq, dtype=np.int32)
    for i in range(nq):
        c = int(rng.integers(1, min(k, int(q_vis[i])) + 1))
        idx[i, :c] = rng.choice(int(q_vis[i]), size=c, replace=False)
        cnt[i] = c
    q = case.layers[0].q                                              # [nq][H][512] bf16 bits
    scale = spec.sm_scale
    out, lse = O.sparse_attn(cache, q, q_seq, idx, cnt, scale)
    flat = cache.kv.reshape(-1, O.KV_ROW_BYTES)
    for i in range(nq):
        s = int(q_seq[i])
        slots = np.array([W.slots_for(spec, case.page_table, s, int(t), int(t) + 1)[0] for t in idx[i, :cnt[i]]])
        x = O.dequantize_kv_rows(flat[slots])
        ro, rl = _torch_dense(O.bf16_to_f64(q[i]), x, scale)
        np.testing.assert_allclose(out[i], ro, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse[i], rl, rtol=1e-13, atol=1e-13)
