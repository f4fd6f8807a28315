"""GPU parity of block-level pruning (csa2_idxk_bounds_build, CSA2_STEP_PRUNE)
through the C ABI: the block-level representation against the oracle's, and
pruned layer groups against the oracle and against the same group without
pruning (bit for bit), with seeds that prune much, nothing, or only part."""
import numpy as np
import pytest
import torch

import workloads as W
from oracle import csa2_oracle as O
from tests import casebuild as CB
from tests.gpu_util import say
from tests.test_gpu_parity import _check_against_oracle

pytestmark = pytest.mark.gpu


def _ops():
    from fp4_kv_cache_layer_amd import ops, runner
    return ops, runner


def _mask_fraction(dc, ws) -> float:
    """Share of the visible 64-entry blocks the prune pass of the last call on
    ws marked."""
    ops, _ = _ops()
    return ops.pruned_block_fraction(ops.workspace_prune_masks(ws, dc.spec.nq, dc.max_vis), dc.spec.q_vis())


def _run_layers(dc):
    """The layers as separate calls; returns the pruned share of every Full
    and Reindex layer (read before the next call reuses the workspace)."""
    ops, _ = _ops()
    fracs = []
    for li, c in enumerate(dc.calls):
        if dc.poison_ws:
            dc._poison(dc.ws)
        c()
        if dc.spec.modes[li] != ops.REUSE:
            fracs.append(_mask_fraction(dc, dc.ws))
    return fracs


def _decode_bounds(raw):
    b = raw.reshape(-1, 2, O.D_INDEX)
    return O.e4m3fn_decode(b[:, 0]), O.e4m3fn_decode(b[:, 1])


@pytest.mark.parametrize("clustered,integer", [(True, True), (False, False)])
def test_bounds_match_the_oracle(clustered, integer):
    spec = W.small_case("bounds", 31, [3000, 1111], clustered=clustered, integer_indexer=integer, page_size=128,
                        modes=(W.FULL,), k=128)
    _, runner = _ops()
    dc = runner.DeviceCase(spec, gen_device="cpu", prune=True)
    case = CB.build(spec)
    ocache = case.fresh_cache()
    gmax, gmin = _decode_bounds(dc.cache.bounds.cpu().numpy())
    omax, omin = O.block_bounds(ocache)
    assert np.array_equal(gmax, omax) and np.array_equal(gmin, omin)
    # a Full layer step refreshes the blocks of the rows it appends
    dc.run_layers()
    O.append_quant_fp4(ocache, case.new_slots, case.new_kv, case.new_ik)
    gmax, gmin = _decode_bounds(dc.cache.bounds.cpu().numpy())
    omax, omin = O.block_bounds(ocache)
    assert np.array_equal(gmax, omax) and np.array_equal(gmin, omin)


def _two_steps(spec, **kw):
    """The group twice: the first call has no seed (nothing pruned), the
    second takes each layer's first selection as its seed."""
    _, runner = _ops()
    dc = runner.DeviceCase(spec, gen_device="cpu", prune=True, poison_ws=True, **kw)
    f1 = _run_layers(dc)
    first = dc.results_host()
    f2 = _run_layers(dc)
    assert all(f == 0.0 for f in f1), f1
    return f2, first, dc.results_host()


@pytest.mark.parametrize("integer,page_size", [(True, 64), (True, 256), (False, 128)])
def test_pruned_group_is_exact_and_prunes(integer, page_size):
    spec = W.small_case("prune_group", 32 + page_size, [9000, 5000, 2100], clustered=True,
                        integer_indexer=integer, page_size=page_size, k=128)
    say(f"[prune] int={integer} page={page_size}")
    fracs, first, second = _two_steps(spec)
    say(f"  pruned blocks per indexer layer {fracs}")
    assert min(fracs) > 0.3, fracs
    plain = _plain(spec)
    for li, (a, b, c) in enumerate(zip(first, second, plain)):
        for key in ("idx", "cnt", "out", "lse"):
            assert np.array_equal(a[key], c[key]), (li, key)            # nothing pruned on the first call
            assert np.array_equal(b[key], c[key]), (li, key)            # pruned: the same bits
    _check_against_oracle(spec, second, exact_topk=integer)


def _plain(spec):
    _, runner = _ops()
    dc = runner.DeviceCase(spec, gen_device="cpu")
    dc.run_layers()
    return dc.results_host()


def test_unclustered_gaussian_prunes_nothing():
    spec = W.small_case("prune_gauss", 41, [8000, 3000], k=256)
    fracs, _, second = _two_steps(spec)
    assert fracs == [0.0, 0.0], fracs
    for a, b in zip(second, _plain(spec)):
        for key in ("idx", "cnt", "out", "lse"):
            assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("kind", ["random", "messy", "short", "shuffled_exact"])
def test_other_seeds_keep_the_selection(kind):
    """Seeds that are not the exact previous selection: random visible
    entries, the selection with duplicates and out-of-range entries mixed in,
    one entry short of k, and the exact selection in shuffled order (sorted
    by the kernel before use)."""
    ops, runner = _ops()
    spec = W.small_case("prune_seeds", 42, [7000, 2600], clustered=True, integer_indexer=True, page_size=64,
                        modes=(W.FULL, W.REINDEX), k=128)
    plain = _plain(spec)
    dc = runner.DeviceCase(spec, gen_device="cpu", prune=True, poison_ws=True)
    rng = np.random.default_rng(43)
    nq, k = spec.nq, spec.k
    for li in range(len(spec.modes)):
        ref = plain[li]["idx"]
        if kind == "random":
            seed = np.stack([rng.choice(int(v), size=k, replace=False) for v in spec.q_vis()])
            cnt = np.full(nq, k)
        elif kind == "messy":
            seed = ref.copy()
            seed[:, 1::7] = seed[:, 0:1]
            seed[:, 2::11] = -5
            seed[:, 3::13] = spec.q_vis()[:, None] + 3
            cnt = np.full(nq, k)
        elif kind == "short":
            seed, cnt = ref.copy(), np.full(nq, k - 1)
        else:
            seed = np.stack([rng.permutation(r) for r in ref])
            cnt = np.full(nq, k)
        dc.outputs[li]["idx"].copy_(torch.from_numpy(seed.astype(np.int32)))
        dc.outputs[li]["cnt"].copy_(torch.from_numpy(cnt.astype(np.int32)))
    fracs = _run_layers(dc)
    say(f"[prune seeds] {kind}: pruned {fracs}")
    if kind == "shuffled_exact":
        assert min(fracs) > 0.3, fracs
    elif kind in ("short", "messy"):
        assert fracs == [0.0, 0.0], fracs                 # fewer than k distinct visible entries
    got = dc.results_host()
    for li, (a, b) in enumerate(zip(got, plain)):
        for key in ("idx", "cnt", "out", "lse"):
            assert np.array_equal(a[key], b[key]), (kind, li, key)


@pytest.mark.parametrize("k", [128, 512])
def test_pruning_when_one_chunk_holds_the_topk(k):
    """Clustered integer rows, with indexer-K rows 2,048..4,095 of sequence 0
    pointing along its query's weighted heads: that chunk holds all of the
    Full layer's Top-k, keeps only its local top entries, and pruning removes
    nearly every other block, so the select starts with fewer than k
    candidates and must take the rest from the threshold alone.  Pruned,
    unpruned and oracle selections agree bit for bit."""
    ops, runner = _ops()
    spec = W.small_case("prune_hot", 91 + k, [20000, 7000], n_new=1, h_idx=8, h=16, k=k,
                        modes=(W.FULL, W.REINDEX), integer_indexer=True, clustered=True, page_size=128)
    qi, w, _ = W.layer_queries(spec, 0, "cpu")
    qv = qi[0].view(torch.float8_e4m3fn).float().numpy()
    u = (w[0].numpy()[:, None] * qv).sum(0)
    rng = np.random.default_rng(k)
    hot = (np.where(u >= 0, 1.0, -1.0)[None, :] * rng.integers(4, 9, (2048, 128))).astype(np.float32)
    hot_bits = torch.from_numpy((hot.view(np.uint32) >> 16).astype(np.uint16).view(np.int16))
    say(f"[prune hot chunk] k={k}")
    pt = W.page_table(spec)
    slots = torch.from_numpy(W.slots_for(spec, pt, 0, 2048, 4096)).cuda()
    kv_bits = W.kv_rows(spec, 0, "cpu")[2048:4096].contiguous().cuda()
    results = {}
    for prune in (False, True):
        dc = runner.DeviceCase(spec, gen_device="cpu", prune=prune, poison_ws=True)
        ops.csa2_append_quant_fp4(dc.cache, slots, kv_bits, hot_bits.cuda())
        if prune:
            dc.cache.build_bounds()
            _run_layers(dc)                                   # no seed yet
        fr = _run_layers(dc)
        results[prune] = dc.results_host()
        if prune:
            say(f"  pruned blocks {fr}")
            assert fr[0] > 0.5, fr
    case = CB.build(spec)
    case.ik_src[0] = case.ik_src[0].copy()
    case.ik_src[0][2048:4096] = hot_bits.numpy().view(np.uint16)
    ref = CB.run_group(case)
    assert int(((ref[0]["idx"][0] >= 2048) & (ref[0]["idx"][0] < 4096)).sum()) == k   # all in the hot chunk
    for li in range(2):
        for key in ("idx", "cnt"):
            assert np.array_equal(results[True][li][key], ref[li][key]), (li, key)
            assert np.array_equal(results[False][li][key], ref[li][key]), (li, key)
        for key in ("out", "lse"):
            assert np.array_equal(results[True][li][key], results[False][li][key]), (li, key)
