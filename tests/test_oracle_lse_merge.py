"""Pins of the oracle's merge of the global (CSA2) branch with the local
sliding-window branch: a hand-worked example, the defining property (the
merge of two disjoint key sets' softmaxes is the softmax over their union,
checked against torch's dense attention), empty sides, symmetry and
associativity."""
import os

import numpy as np
import torch

from oracle import csa2_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "lse_merge_example.txt")


def test_worked_example():
    row = np.loadtxt(GOLDEN)
    o, lse = O.lse_merge(row[None, 0:4], row[None, 4], row[None, 5:9], row[None, 9])
    np.testing.assert_allclose(o[0], row[10:14], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], row[14], rtol=1e-15)


def _dense(q, x, scale):
    """torch's dense attention of H queries over rows x (K = V = x)."""
    qt = torch.from_numpy(q)[:, None, :]
    xt = torch.from_numpy(x)[None].expand(q.shape[0], -1, -1)
    o = torch.nn.functional.scaled_dot_product_attention(qt, xt, xt, scale=scale)[:, 0].numpy()
    lse = torch.logsumexp(scale * (torch.from_numpy(q) @ torch.from_numpy(x).T), dim=1).numpy()
    return o, lse


def test_merge_of_two_key_sets_is_attention_over_their_union():
    rng = np.random.default_rng(3)
    for trial in range(6):
        H, d = 5, 64
        na, nb = int(rng.integers(1, 40)), int(rng.integers(1, 40))
        q = rng.standard_normal((H, d))
        x = rng.standard_normal((na + nb, d)) * (1 + 3 * trial)    # wider logit spreads as trials go
        scale = 1 / np.sqrt(d)
        oa, la = _dense(q, x[:na], scale)
        ob, lb = _dense(q, x[na:], scale)
        ou, lu = _dense(q, x, scale)
        o, lse = O.lse_merge(oa, la, ob, lb)
        np.testing.assert_allclose(o, ou, rtol=0, atol=1e-10 * max(1.0, np.abs(ou).max()))
        np.testing.assert_allclose(lse, lu, rtol=1e-12, atol=1e-12)


def test_empty_sides():
    rng = np.random.default_rng(4)
    oa = rng.standard_normal((3, 8))
    la = rng.standard_normal(3)
    z = np.zeros((3, 8))
    ninf = np.full(3, -np.inf)
    o, lse = O.lse_merge(oa, la, z, ninf)
    assert np.array_equal(o, oa) and np.array_equal(lse, la)
    o, lse = O.lse_merge(z, ninf, oa, la)
    assert np.array_equal(o, oa) and np.array_equal(lse, la)
    o, lse = O.lse_merge(z, ninf, z, ninf)
    assert np.array_equal(o, z) and np.isneginf(lse).all()


def test_symmetric_and_associative():
    rng = np.random.default_rng(5)
    o = [rng.standard_normal((4, 16)) for _ in range(3)]
    l = [rng.standard_normal(4) * 30 for _ in range(3)]
    a1, b1 = O.lse_merge(o[0], l[0], o[1], l[1])
    a2, b2 = O.lse_merge(o[1], l[1], o[0], l[0])
    np.testing.assert_allclose(a1, a2, rtol=0, atol=1e-14)
    np.testing.assert_allclose(b1, b2, rtol=1e-15)
    x1, y1 = O.lse_merge(*O.lse_merge(o[0], l[0], o[1], l[1]), o[2], l[2])
    x2, y2 = O.lse_merge(o[0], l[0], *O.lse_merge(o[1], l[1], o[2], l[2]))
    np.testing.assert_allclose(x1, x2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(y1, y2, rtol=1e-14)


def test_huge_lse_gap_keeps_the_dominant_side():
    oa, ob = np.full((1, 4), 2.0), np.full((1, 4), -7.0)
    o, lse = O.lse_merge(oa, np.array([1000.0]), ob, np.array([-1000.0]))
    assert np.array_equal(o, oa) and lse[0] == 1000.0
