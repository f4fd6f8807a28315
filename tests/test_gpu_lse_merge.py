"""GPU parity of csa2_lse_merge (the merge of the global branch with the
local sliding-window branch) against the oracle, plus the end-to-end property
that merging the attention over two disjoint selections equals the attention
over their union."""
import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _ops():
    from fp4_kv_cache_layer_amd import ops
    return ops


def _lse(rng, rows, kind):
    if kind == "normal":
        return rng.standard_normal(rows) * 10
    if kind == "wide":
        return rng.uniform(-300, 300, rows)
    l = rng.standard_normal(rows) * 5
    l[rng.random(rows) < 0.3] = -np.inf
    return l


@pytest.mark.parametrize("rows,dim,ka,kb", [
    (1, 4, "normal", "normal"),
    (7, 512, "normal", "inf"),
    (2051, 512, "wide", "normal"),
    (300, 1028, "inf", "inf"),
    (64 * 32, 512, "normal", "normal"),
])
def test_lse_merge_matches_oracle(rows, dim, ka, kb):
    ops = _ops()
    say(f"[lse_merge] rows={rows} dim={dim} lse kinds={ka},{kb}")
    rng = np.random.default_rng(rows * 7 + dim)
    oa = rng.standard_normal((rows, dim)).astype(np.float32)
    ob = (rng.standard_normal((rows, dim)) * 3).astype(np.float32)
    la, lb = _lse(rng, rows, ka).astype(np.float32), _lse(rng, rows, kb).astype(np.float32)
    both = np.isneginf(la) & np.isneginf(lb)
    oa[np.isneginf(la)] = 0.0                  # an empty branch's output is 0 (csa2_sparse_attn's convention)
    ob[np.isneginf(lb)] = 0.0
    t = lambda a: torch.from_numpy(a).cuda()
    o, lse = ops.csa2_lse_merge(t(oa), t(la), t(ob), t(lb))
    o, lse = o.cpu().numpy(), lse.cpu().numpy()
    ro, rl = O.lse_merge(oa, la, ob, lb)
    bound = 2e-6 * np.maximum(np.abs(oa), np.abs(ob)) + 1e-7
    assert (np.abs(o - ro) <= bound).all(), np.abs(o - ro).max()
    fin = np.isfinite(rl)
    assert np.array_equal(np.isfinite(lse), fin) and np.isneginf(lse[both]).all()
    assert (np.abs(lse[fin] - rl[fin]) <= 2e-7 * np.maximum(1.0, np.abs(rl[fin]))).all()
    assert (o[both] == 0).all()


def test_lse_merge_in_place():
    ops = _ops()
    rng = np.random.default_rng(11)
    oa = torch.from_numpy(rng.standard_normal((50, 512)).astype(np.float32)).cuda()
    ob = torch.from_numpy(rng.standard_normal((50, 512)).astype(np.float32)).cuda()
    la = torch.from_numpy(rng.standard_normal(50).astype(np.float32)).cuda()
    lb = torch.from_numpy(rng.standard_normal(50).astype(np.float32)).cuda()
    want, wl = ops.csa2_lse_merge(oa, la, ob, lb)
    got, gl = ops.csa2_lse_merge(oa, la, ob, lb, out=oa)
    assert got.data_ptr() == oa.data_ptr()
    assert torch.equal(got, want) and torch.equal(gl, wl)


def test_merge_of_two_selections_is_attention_over_their_union():
    """Attention over rows A, attention over rows B (disjoint), merged: the
    attention over A and B together, all on the GPU path."""
    from fp4_kv_cache_layer_amd import runner
    import workloads as W
    ops = _ops()
    spec = W.small_case("merge_e2e", 71, [3000, 1200], n_new=1, h_idx=8, h=32, k=512)
    dc = runner.DeviceCase(spec, gen_device="cpu")
    dc.run_group()                              # appends the new rows, so every visible entry is written
    rng = np.random.default_rng(72)
    nq, h = spec.nq, spec.h
    vis = spec.q_vis()
    ia = np.full((nq, spec.k), -1, np.int32)
    ib = np.full((nq, spec.k), -1, np.int32)
    iu = np.full((nq, spec.k), -1, np.int32)
    ca, cb, cu = np.zeros(nq, np.int32), np.zeros(nq, np.int32), np.zeros(nq, np.int32)
    for i in range(nq):
        pick = np.sort(rng.choice(int(vis[i]), size=300, replace=False))
        a, b = pick[:170], pick[170:]          # e.g. a far, global part and a recent, local part
        ia[i, :a.size], ib[i, :b.size], iu[i, :pick.size] = a, b, pick
        ca[i], cb[i], cu[i] = a.size, b.size, pick.size
    q = dc.inputs[0][2]
    outs = []
    for idx, cnt in ((ia, ca), (ib, cb), (iu, cu)):
        o = torch.empty((nq, h, 512), dtype=torch.float32, device="cuda")
        l = torch.empty((nq, h), dtype=torch.float32, device="cuda")
        ops.csa2_sparse_attn(dc.cache, q, dc.q_seq, torch.from_numpy(idx).cuda(), torch.from_numpy(cnt).cuda(),
                             spec.sm_scale, o, l)
        outs.append((o, l))
    mo, ml = ops.csa2_lse_merge(outs[0][0], outs[0][1], outs[1][0], outs[1][1])
    err = (mo - outs[2][0]).abs().max().item()
    lerr = ((ml - outs[2][1]).abs() / outs[2][1].abs().clamp(min=1.0)).max().item()
    say(f"[lse_merge e2e] max|dO| {err:.2e} max rel dLSE {lerr:.2e}")
    assert err <= 1e-5 and lerr <= 1e-6
