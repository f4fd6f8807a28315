"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Small cases span several tiles and ragged tails; every input is drawn on the
host by the shared seeded generators so both sides see the same bytes.
"""
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


# ---------------------------------------------------------------------------
# quantize-on-append: bit-exact bytes
# ---------------------------------------------------------------------------

def _finite_bf16_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = O.bf16_to_f64(bits)
    return bits[np.isfinite(x)]


@pytest.mark.parametrize("arrangement", ["shuffled", "sorted", "alone"])
def test_append_bit_exact_every_bf16(arrangement):
    ops, _ = _ops()
    say(f"[append] every finite bf16, {arrangement}")
    pats = _finite_bf16_patterns()
    rng = np.random.default_rng(3)
    if arrangement == "shuffled":
        pats = rng.permutation(pats)
    elif arrangement == "alone":
        # each value leads a block of tiny companions, so it sets the block scale alone
        blocks = np.full((pats.size, 32), 0x0001, dtype=np.uint16)
        blocks[:, 0] = pats
        blocks[:, 1::2] |= 0x8000
        pats = blocks.reshape(-1)
    n = (pats.size + 511) // 512
    kv = np.zeros(n * 512, dtype=np.uint16)
    kv[:pats.size] = pats
    kv = kv.reshape(n, 512)
    ik = np.resize(pats, n * 128).reshape(n, 128)
    ps = 64
    npg = (n + ps - 1) // ps + 1
    cache = ops.Cache(npg, ps, torch.arange(npg, dtype=torch.int32)[None])
    slots = torch.from_numpy(np.random.default_rng(4).permutation(npg * ps)[:n].astype(np.int32)).cuda()
    ops.csa2_append_quant_fp4(cache, slots, torch.from_numpy(kv.view(np.int16)).cuda(),
                              torch.from_numpy(ik.view(np.int16)).cuda())
    torch.cuda.synchronize()
    got_kv = cache.kv.reshape(-1, 272)[slots.long()].cpu().numpy()
    got_ik = cache.idx_k.reshape(-1, 128)[slots.long()].cpu().numpy()
    want_kv = O.quantize_kv_rows(O.bf16_to_f64(kv))
    want_ik = O.quantize_idxk_rows(O.bf16_to_f64(ik))
    bad = np.nonzero((got_kv != want_kv).any(1))[0]
    assert bad.size == 0, f"{bad.size} kv rows differ; first {bad[:3]}"
    assert np.array_equal(got_ik, want_ik)


# ---------------------------------------------------------------------------
# indexer + Top-K
# ---------------------------------------------------------------------------

def _run_case(spec, dense=None, poison_ws=True, **kw):
    """Runs the case's layer group (workspaces poisoned before every call
    unless told otherwise) and returns the device case and its results."""
    _, runner = _ops()
    dc = runner.DeviceCase(spec, gen_device="cpu", dense=dense, poison_ws=poison_ws, **kw)
    dc.run_group()
    return dc, dc.results_host()


def _compare_group(spec, exact_topk: bool, dense=None, group: int = 0):
    say(f"[group] {spec.name} seed={spec.seed} seqs={spec.num_seqs} cached={spec.cached[:6]} "
        f"n_new={spec.n_new} h_idx={spec.h_idx} h={spec.h} k={spec.k} int={spec.integer_indexer} dense={dense} "
        f"group={group}")
    dc, got = _run_case(spec, dense, group=group)
    ref = _check_against_oracle(spec, got, exact_topk)
    return dc, got, ref


def _check_against_oracle(spec, got, exact_topk: bool):
    """Every layer's selection (bit-exact, or valid up to near-ties) and its
    attention over the GPU's own selection against the fp64 oracle."""
    case = CB.build(spec)
    ref = CB.run_group(case)
    # oracle cache after the Full layer's append, to evaluate attention over the GPU's selection
    ocache = case.fresh_cache()
    if case.new_slots.size:
        O.append_quant_fp4(ocache, case.new_slots, case.new_kv, case.new_ik)
    q_seq, q_vis = spec.q_seq(), spec.q_vis()
    for li, (g, r, L) in enumerate(zip(got, ref, case.layers)):
        if L.mode != O.REUSE:
            if exact_topk:
                assert np.array_equal(g["cnt"], r["cnt"]), f"layer {li} cnt"
                bad = np.nonzero((g["idx"] != r["idx"]).any(1))[0]
                assert bad.size == 0, f"layer {li}: {bad.size} queries differ, first {bad[:3]}"
            else:
                ov, worst = overlap_stats(g["idx"], g["cnt"], r["idx"], r["cnt"])
                say(f"  layer {li} overlap {ov:.6f} worst {worst:.4f}")
                assert ov >= OVERLAP_MIN
                for i in range(spec.nq):
                    sc = O.index_scores(ocache, int(q_seq[i]), int(q_vis[i]), L.q_idx[i], L.w[i])
                    check_selection_valid(g["idx"][i], g["cnt"][i], r["idx"][i], r["cnt"][i], sc, spec.k)
        else:
            assert np.array_equal(g["idx"], got[0]["idx"])
        o_ref, lse_ref = O.sparse_attn(ocache, L.q, q_seq, g["idx"], g["cnt"], spec.sm_scale)
        err = np.abs(g["out"] - o_ref).max()
        say(f"  layer {li} mode {L.mode}: max|dO| {err:.2e}")
        assert err <= OUT_ATOL
        fin = np.isfinite(lse_ref)
        assert np.array_equal(np.isfinite(g["lse"]), fin)
        lerr = np.abs(g["lse"][fin] - lse_ref[fin]) / np.maximum(1.0, np.abs(lse_ref[fin]))
        assert lerr.size == 0 or lerr.max() <= LSE_RTOL, lerr.max()
    return ref


@pytest.mark.parametrize("n_aux", [1, 2])
def test_group_step_against_oracle(n_aux):
    """The group step (Reuse attentions on auxiliary streams) checked against
    the oracle directly, not only against the per-layer calls."""
    spec = W.small_case("group_oracle", 64, [3000, 1200, 5000, 64], n_new=1, h_idx=8, h=64, k=512,
                        integer_indexer=True)
    _compare_group(spec, exact_topk=True, group=n_aux)


def test_graph_replay_against_oracle_and_eager():
    """The group's per-layer calls captured in one HIP graph: every replay,
    with eager work (outputs clobbered) and synchronisations between replays,
    gives exactly the eager results, which match the oracle."""
    spec = W.small_case("graph", 65, [4096, 900, 2500], n_new=1, h_idx=8, h=64, k=512, integer_indexer=True)
    say("[graph] capture and replay")
    dc, eager = _run_case(spec)
    _check_against_oracle(spec, eager, exact_topk=True)
    dc.poison_ws = False                     # no fill kernels inside the captured graph
    dc.capture_graph()
    for rep in range(3):
        for o in dc.outputs:
            o["out"].fill_(float("nan"))
            o["lse"].fill_(float("nan"))
            o["idx"].fill_(-7)
            o["cnt"].fill_(-7)
        torch.cuda.synchronize()
        dc.replay_graph()
        got = dc.results_host()
        for li, (x, y) in enumerate(zip(got, eager)):
            for key in ("idx", "cnt", "out", "lse"):
                assert np.array_equal(x[key], y[key]), (rep, li, key)
    _check_against_oracle(spec, got, exact_topk=True)


@pytest.mark.parametrize("seed,cached,h_idx,k", [
    (21, [4096], 4, 512),
    (22, [600, 37, 2048 + 5, 5000, 511, 0, 1], 8, 512),
    (23, [3000, 777], 16, 64),
    (24, [2500, 130], 1, 128),
    (25, [9000], 8, 2048),
])
def test_group_integer_exact(seed, cached, h_idx, k):
    spec = W.small_case("int_group", seed, cached, n_new=1, h_idx=h_idx, h=16, k=k, integer_indexer=True)
    _compare_group(spec, exact_topk=True)


@pytest.mark.parametrize("seed,cached,n_new", [
    (26, [2047, 4095, 1], 1),              # an appended row ending a full chunk; a one-row chunk
    (27, [2046, 6143, 300], 3),            # appended rows across a chunk boundary
    (28, [700] * 30, 3),                   # 90 appended rows: more than one launch carries
])
def test_full_layer_append_positions(seed, cached, n_new):
    """Appended rows at chunk ends, across chunk boundaries and in numbers
    past what the scan launch carries itself: every layer's selection
    bit-exact against the oracle, and the appended rows' cache bytes equal to
    the oracle's encoding."""
    spec = W.small_case("append_pos", seed, cached, n_new=n_new, h_idx=8, h=16, k=128, integer_indexer=True)
    dc, got, ref = _compare_group(spec, exact_topk=True)
    case = CB.build(spec)
    kv = dc.cache.kv.reshape(-1, O.KV_ROW_BYTES)[torch.from_numpy(case.new_slots.astype(np.int64)).cuda()].cpu().numpy()
    ik = dc.cache.idx_k.reshape(-1, 128)[torch.from_numpy(case.new_slots.astype(np.int64)).cuda()].cpu().numpy()
    assert np.array_equal(kv, O.quantize_kv_rows(O.bf16_to_f64(case.new_kv)))
    assert np.array_equal(ik, O.quantize_idxk_rows(O.bf16_to_f64(case.new_ik)))


@pytest.mark.parametrize("seed,cached,h", [
    (31, [4096, 1500, 700], 64),
    (32, [3000, 200], 24),
    (33, [2100], 128),
])
def test_group_gaussian(seed, cached, h):
    spec = W.small_case("gauss_group", seed, cached, n_new=1, h_idx=8, h=h, k=512, integer_indexer=False)
    _compare_group(spec, exact_topk=False)


def test_config0_exact():
    spec = W.config(0)
    _compare_group(spec, exact_topk=True)


@pytest.mark.parametrize("dense", [True, False])
def test_prefill_small_causal(dense):
    spec = W.small_case("prefill", 41, [1500], n_new=300, h_idx=8, h=32, k=256, modes=(O.FULL,), prefill=True,
                        integer_indexer=True)
    _compare_group(spec, exact_topk=True, dense=dense)


@pytest.mark.parametrize("seed,cached,n_new,h_idx,k", [
    (42, [2000], 37, 12, 512),       # one query per A tile, ragged query block
    (43, [700], 130, 3, 128),        # short context: most entries causal-masked for early queries
])
def test_prefill_dense_integer_exact(seed, cached, n_new, h_idx, k):
    spec = W.small_case("prefill_int", seed, cached, n_new=n_new, h_idx=h_idx, h=16, k=k, modes=(O.FULL,),
                        prefill=True, integer_indexer=True)
    _compare_group(spec, exact_topk=True, dense=True)


def test_prefill_dense_gaussian():
    spec = W.small_case("prefill_gauss", 44, [5000], n_new=200, h_idx=8, h=64, k=512, modes=(O.FULL, O.REINDEX),
                        prefill=True)
    _compare_group(spec, exact_topk=False, dense=True)


@pytest.mark.parametrize("seed,cached,n_new,h_idx,page_size,k", [
    (45, [6000], 300, 8, 64, 512),
    (46, [40000], 45, 8, 64, 512),   # several chunks per XCD (64-entry pages cap a chunk at 63 pages)
    (47, [3000], 77, 12, 128, 512),
    (48, [2500], 19, 3, 64, 512),
    (49, [20000], 64, 8, 256, 128),   # sampled threshold with k = 128
    (50, [30000], 40, 12, 1024, 512),
])
def test_prefill_dense_bit_identical_to_scan(seed, cached, n_new, h_idx, page_size, k):
    """The dense prefill indexer (sampled threshold, candidates, exact select)
    and the per-query scan select identically, so the whole layer output
    matches bit for bit."""
    spec = W.small_case("prefill_same", seed, cached, n_new=n_new, h_idx=h_idx, h=16, k=k,
                        modes=(O.FULL, O.REINDEX), prefill=True, page_size=page_size)
    say(f"[dense=scan] seed={seed} cached={cached} n_new={n_new} h_idx={h_idx} page={page_size} k={k}")
    _, a = _run_case(spec, dense=True)
    _, b = _run_case(spec, dense=False)
    for li, (x, y) in enumerate(zip(a, b)):
        for key in ("idx", "cnt", "out", "lse"):
            assert np.array_equal(x[key], y[key]), (li, key)


def _group_vs_layers(spec, n_aux, dense=None, shared_ws=False, reps=2):
    _, runner = _ops()
    say(f"[group step] {spec.name} seed={spec.seed} modes={spec.modes} n_aux={n_aux} shared_ws={shared_ws}")
    ref = runner.DeviceCase(spec, gen_device="cpu", dense=dense, poison_ws=True)
    ref.run_group()
    want = ref.results_host()
    dc = runner.DeviceCase(spec, gen_device="cpu", dense=dense, group=n_aux, shared_ws=shared_ws, poison_ws=True)
    for rep in range(reps):
        dc.run_group()
        got = dc.results_host()
        for li, (x, y) in enumerate(zip(got, want)):
            for key in ("idx", "cnt", "out", "lse"):
                assert np.array_equal(x[key], y[key]), (rep, li, key)


@pytest.mark.parametrize("n_aux", [1, 2, 3])
def test_group_step_matches_layer_calls(n_aux):
    """One csa2_group_step (selects and attentions on auxiliary streams)
    gives exactly the results of the layers called one by one."""
    spec = W.small_case("group_step", 61, [4096, 1500, 700, 3000], n_new=1, h_idx=8, h=64, k=512)
    _group_vs_layers(spec, n_aux)


def test_group_step_mixed_order_and_shared_workspace():
    """Reuse before Reindex, and every layer on one workspace (the group then
    orders the layers itself)."""
    spec = W.small_case("group_mixed", 62, [2048, 900], n_new=1, h_idx=4, h=32, k=256,
                        modes=(O.FULL, O.REUSE, O.REINDEX, O.REUSE), integer_indexer=True)
    _group_vs_layers(spec, 2)
    _group_vs_layers(spec, 2, shared_ws=True)


def test_group_step_prefill_dense():
    spec = W.small_case("group_prefill", 63, [3000], n_new=150, h_idx=8, h=16, k=256,
                        modes=(O.FULL, O.REINDEX, O.REUSE), prefill=True)
    _group_vs_layers(spec, 2, dense=True)


@pytest.mark.parametrize("factor", [0, 1, 64])
def test_prefill_dense_candidate_factor(factor):
    """Candidate factor 0 sends every query through the full rescore, 1 makes
    short candidate lists (some queries rescored), 64 keeps every entry; the
    selection is the same in all cases."""
    from fp4_kv_cache_layer_amd import _lib as L
    spec = W.small_case("prefill_factor", 52, [24000], n_new=48, h_idx=8, h=16, k=256,
                        modes=(O.FULL,), prefill=True, page_size=128)
    say(f"[dense factor] factor={factor}")
    _, ref = _run_case(spec, dense=False)
    _, got = _run_case(spec, dense=True, cand_factor=L.DENSE_RESCORE_ALL if factor == 0 else factor)
    for key in ("idx", "cnt", "out", "lse"):
        assert np.array_equal(got[0][key], ref[0][key]), key


def test_all_equal_scores_take_lowest_indices():
    """Zero indexer queries make every score 0: the first k entries win,
    including the long-tie path (more tied keys than the select kernel parks)."""
    ops, runner = _ops()
    for cached in ([20000], [300, 13000]):
        spec = W.small_case("ties", 51, cached, n_new=1, h_idx=4, h=16, k=512, modes=(O.FULL,), integer_indexer=True)
        say(f"[ties] cached={cached}")
        dc = runner.DeviceCase(spec, gen_device="cpu")
        dc.inputs[0][0].zero_()
        dc.run_group()
        got = dc.results_host()[0]
        for i, s in enumerate(spec.q_seq()):
            v = spec.seq_len_after(int(s))
            kp = min(512, v)
            assert got["cnt"][i] == kp
            assert list(got["idx"][i, :kp]) == list(range(kp))


@pytest.mark.parametrize("prefill", [False, True])
def test_repeat_calls_are_deterministic_and_workspace_self_cleans(prefill):
    """Repeated calls give the same bits and leave the workspace's state head
    zeroed; the prefill case takes the dense indexer with a candidate factor
    of 1, so some queries go through the full rescore (its counters, too,
    must be cleared)."""
    if prefill:
        spec = W.small_case("repeat_prefill", 62, [9000], n_new=40, h_idx=8, h=16, k=256, modes=(O.FULL,),
                            prefill=True, page_size=128)
    else:
        spec = W.small_case("repeat", 61, [3000, 900], n_new=1, h_idx=8, h=16, k=512)
    ops, runner = _ops()
    dc = runner.DeviceCase(spec, gen_device="cpu", dense=prefill, cand_factor=1 if prefill else 0)
    dc.run_group()
    a = dc.results_host()
    for _ in range(3):
        dc.run_group()
    b = dc.results_host()
    for x, y in zip(a, b):
        for key in ("idx", "cnt", "out", "lse"):
            assert np.array_equal(x[key], y[key]), key
    state = ops.workspace_state_bytes(spec.nq)           # counters and thresholds carry state
    assert int(dc.ws[:state].view(torch.int32).abs().sum().item()) == 0


# ---------------------------------------------------------------------------
# attention alone, on chosen selections
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("nq,h,k", [(523, 64, 512), (300, 128, 512), (520, 64, 2048)])
def test_sparse_attn_large_batch_shared_rows(nq, h, k):
    """Large batches take the form that gathers each selected row once for
    all 64 heads of a query: identical bits to the one-workgroup-per-16-heads
    form on every query, and the oracle's result on sampled queries (counts
    0, 1, 31..33, k and one above k, which counts as k)."""
    ops, _ = _ops()
    say(f"[attn-shared] nq={nq} h={h} k={k}")
    rng = np.random.default_rng(nq + h + k)
    n, ps = 5000, 64
    npg = (n + ps - 1) // ps
    perm = rng.permutation(npg).astype(np.int32)
    cache = ops.Cache(npg, ps, torch.from_numpy(perm[None]))
    ocache = O.Cache.empty(npg, ps, perm[None], [n])
    kv = (rng.standard_normal((n, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kv[5] = 0
    ik = np.zeros((n, 128), dtype=np.uint16)
    t = np.arange(n)
    slots = (perm[t // ps].astype(np.int64) * ps + t % ps).astype(np.int32)
    ops.csa2_append_quant_fp4(cache, torch.from_numpy(slots).cuda(), torch.from_numpy(kv.view(np.int16)).cuda(),
                              torch.from_numpy(ik.view(np.int16)).cuda())
    O.append_quant_fp4(ocache, slots, kv, ik)
    cnts = rng.integers(0, k + 1, nq).astype(np.int32)
    cnts[:7] = [0, 1, 31, 32, 33, k, k + 5]
    idx = np.full((nq, k), -1, dtype=np.int32)
    for i, c in enumerate(cnts):
        c = min(int(c), k)
        idx[i, :c] = np.sort(rng.choice(n, c, replace=False))
    q = (rng.standard_normal((nq, h, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q_seq = np.zeros(nq, dtype=np.int32)
    qd, sd = torch.from_numpy(q.view(np.int16)).cuda(), torch.from_numpy(q_seq).cuda()
    idd, cd = torch.from_numpy(idx).cuda(), torch.from_numpy(cnts).cuda()
    # the one-workgroup-per-16-heads form, through a Reuse layer step with the flag
    out0 = torch.empty((nq, h, 512), dtype=torch.float32, device="cuda")
    lse0 = torch.empty((nq, h), dtype=torch.float32, device="cuda")
    ops.LayerCall(ops.REUSE, cache, qd, sd, sd, k, 0, 1 / np.sqrt(512), idd, cd, out0, lse0,
                  attn_per_head_group=True)()
    out0, lse0 = out0.cpu().numpy(), lse0.cpu().numpy()
    out1, lse1 = (x.cpu().numpy() for x in ops.csa2_sparse_attn(cache, qd, sd, idd, cd, 1 / np.sqrt(512)))
    assert np.array_equal(out0.view(np.uint32), out1.view(np.uint32))
    assert np.array_equal(lse0.view(np.uint32), lse1.view(np.uint32))
    sample = [0, 1, 2, 3, 4, 5, 6, nq // 2, nq - 1]
    o_ref, lse_ref = O.sparse_attn(ocache, q[sample], q_seq[sample], idx[sample],
                                   np.minimum(cnts[sample], k), 1 / np.sqrt(512))
    err = np.abs(out1[sample] - o_ref).max()
    say(f"  max|dO| {err:.2e}")
    assert err <= OUT_ATOL
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse1[sample]), fin)
    assert (np.abs(lse1[sample][fin] - lse_ref[fin]) <= LSE_RTOL * np.maximum(1, np.abs(lse_ref[fin]))).all()
    assert (out1[0] == 0).all()


@pytest.mark.parametrize("with_ws", [False, True])
@pytest.mark.parametrize("h,cnts", [(16, [0, 1, 2, 3, 17, 512]), (64, [512, 300, 2]), (40, [33, 512]), (128, [511, 5])])
def test_sparse_attn_given_selection(h, cnts, with_ws):
    ops, _ = _ops()
    say(f"[attn] h={h} cnts={cnts} ws={with_ws}")
    rng = np.random.default_rng(h)
    n, ps = 3000, 64
    npg = (n + ps - 1) // ps
    perm = rng.permutation(npg).astype(np.int32)
    cache = ops.Cache(npg, ps, torch.from_numpy(perm[None]))
    ocache = O.Cache.empty(npg, ps, perm[None], [n])
    kv = (rng.standard_normal((n, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    kv[5] = 0                                              # an all-zero row
    kv[6, :32] = 0x0001                                    # a subnormal block
    ik = np.zeros((n, 128), dtype=np.uint16)
    t = np.arange(n)
    slots = (perm[t // ps].astype(np.int64) * ps + t % ps).astype(np.int32)
    ops.csa2_append_quant_fp4(cache, torch.from_numpy(slots).cuda(), torch.from_numpy(kv.view(np.int16)).cuda(),
                              torch.from_numpy(ik.view(np.int16)).cuda())
    O.append_quant_fp4(ocache, slots, kv, ik)
    k = 512
    nq = len(cnts)
    idx = np.full((nq, k), -1, dtype=np.int32)
    for i, c in enumerate(cnts):
        sel = np.sort(rng.choice(n, c, replace=False))
        if c >= 7:
            sel[:2] = [5, 6]
            sel = np.sort(sel)
        idx[i, :c] = sel
    q = (rng.standard_normal((nq, h, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    q_seq = np.zeros(nq, dtype=np.int32)
    ws = ops.workspace(ops.REUSE, nq, 0, 1, h, k) if with_ws else None      # small batch: rows split across workgroups
    for _ in range(2 if with_ws else 1):                                    # second call reuses the self-cleaned counters
        out, lse = ops.csa2_sparse_attn(cache, torch.from_numpy(q.view(np.int16)).cuda(), torch.from_numpy(q_seq).cuda(),
                                        torch.from_numpy(idx).cuda(), torch.tensor(cnts, dtype=torch.int32).cuda(),
                                        1 / np.sqrt(512), ws=ws)
    out, lse = out.cpu().numpy(), lse.cpu().numpy()
    o_ref, lse_ref = O.sparse_attn(ocache, q, q_seq, idx, np.array(cnts), 1 / np.sqrt(512))
    err = np.abs(out - o_ref).max()
    say(f"  max|dO| {err:.2e}")
    assert err <= OUT_ATOL
    fin = np.isfinite(lse_ref)
    assert np.array_equal(np.isfinite(lse), fin)
    assert (np.abs(lse[fin] - lse_ref[fin]) <= LSE_RTOL * np.maximum(1, np.abs(lse_ref[fin]))).all()
    for i, c in enumerate(cnts):
        if c == 0:
            assert (out[i] == 0).all()


def test_peaked_softmax_stays_within_tolerance():
    """Large logits make a near one-hot softmax, the worst case for rounding
    the probabilities before the P.V product."""
    ops, _ = _ops()
    rng = np.random.default_rng(77)
    n, ps, h = 600, 64, 16
    npg = (n + ps - 1) // ps
    cache = ops.Cache(npg, ps, torch.arange(npg, dtype=torch.int32)[None])
    ocache = O.Cache.empty(npg, ps, np.arange(npg, dtype=np.int32)[None], [n])
    kv = (rng.standard_normal((n, 512)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    ik = np.zeros((n, 128), dtype=np.uint16)
    slots = np.arange(n, dtype=np.int32)
    ops.csa2_append_quant_fp4(cache, torch.from_numpy(slots).cuda(), torch.from_numpy(kv.view(np.int16)).cuda(),
                              torch.from_numpy(ik.view(np.int16)).cuda())
    O.append_quant_fp4(ocache, slots, kv, ik)
    x = O.dequantize_kv_rows(ocache.kv.reshape(-1, 272)[:n])
    idx = np.sort(rng.choice(n, 512, replace=False)).astype(np.int32)[None]
    q32 = (x[idx[0, 10]] * 4.0)[None, None, :].repeat(h, 1).astype(np.float32)   # aligned with one row
    q32 *= np.linspace(0.2, 3.0, h, dtype=np.float32)[None, :, None]
    q = (q32.view(np.uint32) >> 16).astype(np.uint16)
    out, lse = ops.csa2_sparse_attn(cache, torch.from_numpy(q.view(np.int16)).cuda(), torch.zeros(1, dtype=torch.int32).cuda(),
                                    torch.from_numpy(idx).cuda(), torch.tensor([512], dtype=torch.int32).cuda(),
                                    1 / np.sqrt(512))
    o_ref, lse_ref = O.sparse_attn(ocache, q, [0], idx, [512], 1 / np.sqrt(512))
    err = np.abs(out.cpu().numpy() - o_ref).max()
    say(f"[attn peaked] max|dO| {err:.2e}")
    assert err <= OUT_ATOL


@pytest.mark.parametrize("k", [512, 2048])
def test_scan_chunk_repair_when_topk_concentrates(k):
    """Indexer-K rows 2,048..4,095 of sequence 0 point along the query's
    weighted heads, so that chunk holds far more of its Top-k than its local
    share: the
    per-query scan keeps only its local top entries there, and the final
    select must find the chunk's floor above the k-th key's bin and rescore
    it.  The selection stays bit-exact against the oracle."""
    ops, runner = _ops()
    spec = W.small_case("repair", 81 + k, [20000, 7000], n_new=1, h_idx=8, h=16, k=k,
                        modes=(O.FULL, O.REINDEX), integer_indexer=True)
    # rows along sign(sum_h w_h q_h) of the Full layer's query 0, magnitudes 4..8:
    # their scores dominate that query's Top-k
    qi, w, _ = W.layer_queries(spec, 0, "cpu")
    qv = qi[0].view(torch.float8_e4m3fn).float().numpy()                # [h_idx][128]
    u = (w[0].numpy()[:, None] * qv).sum(0)
    rng = np.random.default_rng(k)
    hot = (np.where(u >= 0, 1.0, -1.0)[None, :] * rng.integers(4, 9, (2048, 128))).astype(np.float32)
    hot_bits = (hot.view(np.uint32) >> 16).astype(np.uint16)           # small integers are exact in bf16
    say(f"[repair] k={k}")
    dc = runner.DeviceCase(spec, gen_device="cpu", poison_ws=True)
    pt = W.page_table(spec)
    slots = torch.from_numpy(W.slots_for(spec, pt, 0, 2048, 4096)).cuda()
    kv_bits = W.kv_rows(spec, 0, "cpu")[2048:4096].contiguous().cuda()
    ops.csa2_append_quant_fp4(dc.cache, slots, kv_bits, torch.from_numpy(hot_bits.view(np.int16)).cuda())
    dc.run_layers()
    got = dc.results_host()
    case = CB.build(spec)
    case.ik_src[0] = case.ik_src[0].copy()
    case.ik_src[0][2048:4096] = hot_bits
    ref = CB.run_group(case)
    # the case does exercise the repair: the chunk holds more of the Top-k than it keeps
    share = -(-k * 2048 // int(spec.q_vis()[0]))
    local = min(2048, max(16, 4 * share))
    in_chunk = int(((ref[0]["idx"][0] >= 2048) & (ref[0]["idx"][0] < 4096)).sum())
    say(f"  Top-{k} entries in the hot chunk: {in_chunk} (the chunk keeps about {local})")
    assert in_chunk > local
    for li in range(2):
        assert np.array_equal(got[li]["cnt"], ref[li]["cnt"]), li
        assert np.array_equal(got[li]["idx"], ref[li]["idx"]), li
