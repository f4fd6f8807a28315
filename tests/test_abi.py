"""The C ABI without a GPU: the library loads, exports every function the
header declares, and rejects bad arguments on the host before any launch."""
import ctypes
import os

import pytest

from fp4_kv_cache_layer_amd import _lib as L

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="libcsa2.so not built")

FAKE = 0x100000          # aligned, never dereferenced: every call below fails validation or is a no-op


def _view(**kw):
    v = dict(kv=FAKE, idx_k=FAKE, page_table=FAKE, seq_lens=FAKE, num_pages=4, page_size=64, num_seqs=1, max_pages=4)
    v.update(kw)
    return L.CacheView(**v)


def test_exports_every_header_function():
    lib = L.load()
    names = L.header_functions()
    assert set(names) >= {"csa2_append_quant_fp4", "csa2_index_topk", "csa2_prefill_index_topk", "csa2_sparse_attn",
                          "csa2_layer_step", "csa2_workspace_bytes", "csa2_workspace_init", "csa2_status_string"}
    # no process-wide setters: every knob is a per-call argument
    assert not any(n.startswith("csa2_set_") for n in names)
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings():
    lib = L.load()
    for st in range(5):
        assert lib.csa2_status_string(st)
    assert lib.csa2_status_string(99) == b"unknown status"


def test_workspace_bytes():
    lib = L.load()
    reuse = lib.csa2_workspace_bytes(L.CSA2_REUSE, 32, 65537, 8, 64, 512)
    assert reuse == 512                               # three per-query counters, padded to 256 bytes
    full = lib.csa2_workspace_bytes(L.CSA2_FULL, 32, 65537, 8, 64, 512)
    assert full == lib.csa2_workspace_bytes(L.CSA2_REINDEX, 32, 65537, 8, 64, 512)
    vstride = (65537 + 2 + 63) // 64 * 64
    # candidates, keys, chunk floors, prune masks, block maximum keys
    assert full == reuse + 2 * 32 * vstride * 4 + 2 * 32 * 33 * 4 + 32 * 33 * 32 * 4
    assert lib.csa2_workspace_bytes(L.CSA2_FULL, 4, 100, 8, 0, 512) == 0          # invalid h
    assert lib.csa2_workspace_bytes(L.CSA2_FULL, 4096, 70000, 8, 64, 512) >= 4096 * 70000 * 4
    assert lib.csa2_workspace_bytes(L.CSA2_FULL, 0, 100, 8, 64, 512) == 0


def test_prune_mask_view_ends_the_workspace():
    """ops.workspace_prune_masks reads the masks where the library puts them:
    just before the last nq * ceil(max_vis / 2048) * 32 words (the block
    maximum keys) of a Full workspace whose candidate region is larger than
    the pool region."""
    import numpy as np
    import torch

    from fp4_kv_cache_layer_amd import ops
    for nq, max_vis in ((32, 65537), (3, 70000), (17, 2049)):
        ws = torch.zeros(ops.csa2_workspace_bytes(ops.FULL, nq, max_vis, 8, 64, 512), dtype=torch.uint8)
        m = ops.workspace_prune_masks(ws, nq, max_vis)
        assert m.shape == (nq, (max_vis + 2047) // 2048)
        assert m.data_ptr() + m.numel() * 4 + m.numel() * 32 * 4 == ws.data_ptr() + ws.numel()
    # the block count of a mask view: bit i of word c is block 32c + i
    m = torch.zeros((2, 3), dtype=torch.int32)
    m[0, 0] = 0b101
    m[0, 2] = 1                               # block 64, past query 0's 40 blocks
    m[1, 1] = -1                              # blocks 32..63 of query 1
    assert ops.pruned_block_fraction(m, np.array([40 * 64, 96 * 64])) == (2 + 32) / (40 + 96)


def _topk(lib, view, fn="csa2_index_topk", **kw):
    a = dict(q_idx=FAKE, w=FAKE, q_seq=FAKE, q_vis=FAKE, nq=1, h_idx=8, k=512, max_vis=200,
             out_idx=FAKE, out_cnt=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    return getattr(lib, fn)(ctypes.byref(view), a["q_idx"], a["w"], a["q_seq"], a["q_vis"], a["nq"], a["h_idx"],
                            a["k"], a["max_vis"], a["out_idx"], a["out_cnt"], a["ws"], a["ws_bytes"], None)


TOPK_FNS = ["csa2_index_topk", "csa2_prefill_index_topk"]


@pytest.mark.parametrize("kw", [dict(h_idx=0), dict(h_idx=17), dict(k=0), dict(k=2049), dict(nq=-1),
                                dict(max_vis=-1), dict(max_vis=257), dict(q_idx=None), dict(w=None),
                                dict(out_idx=None), dict(ws=None), dict(q_idx=FAKE + 8)])
@pytest.mark.parametrize("fn", TOPK_FNS)
def test_index_topk_rejects(kw, fn):
    assert _topk(L.load(), _view(), fn, **kw) == L.CSA2_ERR_INVALID_ARG


@pytest.mark.parametrize("vkw", [dict(page_size=48), dict(page_size=32), dict(page_size=0), dict(kv=None),
                                 dict(page_table=None), dict(num_pages=0), dict(kv=FAKE + 4)])
@pytest.mark.parametrize("fn", TOPK_FNS)
def test_cache_view_rejects(vkw, fn):
    assert _topk(L.load(), _view(**vkw), fn) == L.CSA2_ERR_INVALID_ARG


@pytest.mark.parametrize("fn", TOPK_FNS)
def test_index_topk_workspace_too_small_and_empty(fn):
    lib = L.load()
    assert _topk(lib, _view(), fn, ws_bytes=100) == L.CSA2_ERR_WORKSPACE
    assert _topk(lib, _view(), fn, nq=0, q_idx=None, ws=None) == L.CSA2_OK          # nothing enqueued


def _attn(lib, view, **kw):
    a = dict(q=FAKE, q_seq=FAKE, idx=FAKE, cnt=FAKE, nq=1, h=64, k=512, sm_scale=0.044, out=FAKE, lse=None)
    a.update(kw)
    return lib.csa2_sparse_attn(ctypes.byref(view), a["q"], a["q_seq"], a["idx"], a["cnt"], a["nq"], a["h"], a["k"],
                                a["sm_scale"], a["out"], a["lse"], None, 0, None)


@pytest.mark.parametrize("kw", [dict(h=0), dict(h=129), dict(k=0), dict(sm_scale=0.0), dict(sm_scale=float("inf")),
                                dict(sm_scale=-1.0), dict(q=None), dict(out=None), dict(out=FAKE + 4)])
def test_sparse_attn_rejects(kw):
    assert _attn(L.load(), _view(), **kw) == L.CSA2_ERR_INVALID_ARG


def test_append_rejects_and_empty():
    lib = L.load()
    v = _view()
    assert lib.csa2_append_quant_fp4(ctypes.byref(v), FAKE, FAKE, FAKE, -1, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_append_quant_fp4(ctypes.byref(v), None, FAKE, FAKE, 3, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_append_quant_fp4(ctypes.byref(v), FAKE, FAKE + 2, FAKE, 3, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_append_quant_fp4(ctypes.byref(v), None, None, None, 0, None) == L.CSA2_OK


def test_layer_step_mode_field_rules():
    lib = L.load()
    v = _view()
    a = L.StepArgs()
    a.cache = ctypes.pointer(v)
    a.q, a.h, a.sm_scale, a.q_seq, a.q_vis, a.nq, a.k, a.max_vis = FAKE, 64, 0.04, FAKE, FAKE, 1, 512, 100
    a.idx, a.cnt, a.out = FAKE, FAKE, FAKE
    assert lib.csa2_layer_step(7, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.q_idx = FAKE                                       # Reuse must not carry indexer inputs
    assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.q_idx, a.n_new, a.new_slots = None, 1, FAKE        # Reindex must not append
    assert lib.csa2_layer_step(L.CSA2_REINDEX, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.n_new, a.new_slots = 0, None
    assert lib.csa2_layer_step(L.CSA2_FULL, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG   # Full needs q_idx/w/ws
    a.nq = 0
    assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_OK              # nothing to do
    a.flags = 16                                         # unknown flag bit
    assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.flags = L.STEP_DENSE_INDEX
    assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_OK
    assert lib.csa2_layer_step(L.CSA2_REUSE, None, None) == L.CSA2_ERR_INVALID_ARG


def _reuse_args(v):
    a = L.StepArgs()
    a.cache = ctypes.pointer(v)
    a.q, a.h, a.sm_scale, a.q_seq, a.q_vis, a.nq, a.k, a.max_vis = FAKE, 64, 0.04, FAKE, FAKE, 0, 512, 100
    a.idx, a.cnt, a.out = FAKE, FAKE, FAKE
    return a


def test_layer_step_per_call_knobs():
    """The dense indexer's candidate factor and the attention form are fields
    of the call: the factor is only allowed with the dense flag and within
    [-1, 64]; the attention-form flag is accepted in every mode."""
    lib = L.load()
    v = _view()
    a = _reuse_args(v)
    a.dense_cand_factor = 4                              # factor without the dense flag
    assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.flags = L.STEP_DENSE_INDEX
    for bad in (-2, 65, 1000):
        a.dense_cand_factor = bad
        assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    for ok in (L.DENSE_RESCORE_ALL, 0, 1, 64):
        a.dense_cand_factor = ok
        assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_OK
    a.flags, a.dense_cand_factor = L.STEP_ATTN_PER_HEAD_GROUP, 0
    assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_OK
    a.flags = 16                                         # unknown bit
    assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG


def test_layer_step_timing_is_per_call():
    """A timing struct rides on the call; rings without events or with no room
    are left alone (nothing is launched here: nq = 0)."""
    lib = L.load()
    v = _view()
    a = _reuse_args(v)
    r = L.TimingRing(None, None, 4, 0)
    t = L.Timing()
    t.ring[L.KCLASS_ATTN] = ctypes.pointer(r)
    a.timing = ctypes.pointer(t)
    assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_OK
    assert r.count == 0


def test_ops_checks_dtypes_and_lengths():
    """The binding rejects index and count tensors of the wrong dtype or
    length before touching the library (int64 tensors would be read as pairs
    of int32 words, short ones out of bounds)."""
    import torch

    from fp4_kv_cache_layer_amd import ops
    nq, h, k = 3, 16, 8
    q = torch.zeros((nq, h, 512), dtype=torch.int16)
    good = dict(q_seq=torch.zeros(nq, dtype=torch.int32), idx=torch.zeros((nq, k), dtype=torch.int32),
                cnt=torch.zeros(nq, dtype=torch.int32))
    bad_cases = [("q_seq", torch.zeros(nq, dtype=torch.int64), TypeError),
                 ("q_seq", torch.zeros(nq - 1, dtype=torch.int32), ValueError),
                 ("idx", torch.zeros((nq, k), dtype=torch.int64), TypeError),
                 ("idx", torch.zeros((nq - 1, k), dtype=torch.int32), ValueError),
                 ("cnt", torch.tensor([1, 2, 3]), TypeError),
                 ("cnt", torch.zeros(nq + 1, dtype=torch.int32), ValueError)]
    for name, t, exc in bad_cases:
        kw = dict(good)
        kw[name] = t
        with pytest.raises(exc):
            ops.csa2_sparse_attn(None, q, kw["q_seq"], kw["idx"], kw["cnt"], 0.04)
    qi = torch.zeros((nq, 8, 128), dtype=torch.uint8)
    w = torch.zeros((nq, 8), dtype=torch.float32)
    for name, t, exc in [("q_vis", torch.zeros(nq, dtype=torch.int64), TypeError),
                         ("q_vis", torch.zeros(2 * nq, dtype=torch.int32), ValueError),
                         ("q_seq", torch.zeros((nq, 1), dtype=torch.int32), ValueError),
                         ("out_idx", torch.zeros((nq, k + 1), dtype=torch.int32), ValueError),
                         ("out_cnt", torch.zeros(nq, dtype=torch.int64), TypeError)]:
        kw = dict(q_seq=torch.zeros(nq, dtype=torch.int32), q_vis=torch.zeros(nq, dtype=torch.int32),
                  out_idx=None, out_cnt=None)
        kw[name] = t
        with pytest.raises(exc):
            ops.csa2_index_topk(None, qi, w, kw["q_seq"], kw["q_vis"], k, 100, None,
                                out_idx=kw["out_idx"], out_cnt=kw["out_cnt"])
    with pytest.raises(ValueError):                      # w of the wrong width
        ops.csa2_index_topk(None, qi, torch.zeros((nq, 4)), good["q_seq"], good["q_seq"], k, 100, None)


def test_group_step_validation():
    lib = L.load()
    assert lib.csa2_group_events(4, 2) == 15
    assert lib.csa2_group_events(0, 0) == 1
    assert lib.csa2_group_events(-1, 0) == -1
    assert lib.csa2_group_events(L.GROUP_MAX_LAYERS + 1, 0) == -1
    assert lib.csa2_group_events(1, L.GROUP_MAX_AUX + 1) == -1
    modes = (ctypes.c_int32 * 1)(0)
    args = (L.StepArgs * 1)()
    assert lib.csa2_group_step(0, None, None, None, None) == L.CSA2_OK
    assert lib.csa2_group_step(-1, modes, args, None, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_group_step(L.GROUP_MAX_LAYERS + 1, modes, args, None, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_group_step(1, None, args, None, None) == L.CSA2_ERR_INVALID_ARG
    ex = L.GroupExec()
    ex.n_aux = L.GROUP_MAX_AUX + 1
    assert lib.csa2_group_step(1, modes, args, None, ctypes.byref(ex)) == L.CSA2_ERR_INVALID_ARG
    ex.n_aux = 1
    ex.aux[0] = 0x1234
    ev = (ctypes.c_void_p * 6)(1, 2, 3, 4, 5, 6)
    ex.events, ex.n_events = ctypes.cast(ev, ctypes.POINTER(ctypes.c_void_p)), 4   # needs 5
    assert lib.csa2_group_step(1, modes, args, None, ctypes.byref(ex)) == L.CSA2_ERR_INVALID_ARG
    ex.aux[0] = 0                                                                 # null stream
    ex.n_events = 5
    assert lib.csa2_group_step(1, modes, args, None, ctypes.byref(ex)) == L.CSA2_ERR_INVALID_ARG
    ex.n_aux, ex.aux[0], ex.aux[1], ex.n_events = 2, 0x1234, 0x1234, 6            # repeated stream
    assert lib.csa2_group_step(1, modes, args, None, ctypes.byref(ex)) == L.CSA2_ERR_INVALID_ARG
    # a layer that fails validation (no cache) is reported before anything is enqueued
    assert lib.csa2_group_step(1, modes, args, None, None) == L.CSA2_ERR_INVALID_ARG


def test_lse_merge_validation():
    lib = L.load()
    p, q, r = 4096, 8192, 12288           # fake, 16-byte aligned addresses: nothing is launched
    assert lib.csa2_lse_merge(None, None, None, None, 0, 512, None, None, None) == L.CSA2_OK
    assert lib.csa2_lse_merge(p, q, p, q, -1, 512, p, r, None) == L.CSA2_ERR_INVALID_ARG
    for dim in (0, 2, 6, -4):
        assert lib.csa2_lse_merge(p, q, p, q, 1, dim, p, r, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_lse_merge(None, q, p, q, 1, 512, p, r, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_lse_merge(p, q, p, q, 1, 512, None, r, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_lse_merge(p + 4, q, p, q, 1, 512, p, r, None) == L.CSA2_ERR_INVALID_ARG   # o_a misaligned
    assert lib.csa2_lse_merge(p, q + 2, p, q, 1, 512, p, r, None) == L.CSA2_ERR_INVALID_ARG   # lse_a misaligned
    assert lib.csa2_lse_merge(p, q, p, r, 1, 512, p, q, None) == L.CSA2_ERR_INVALID_ARG       # lse is lse_a
    assert lib.csa2_lse_merge(p, q, p, r, 1, 512, p, r, None) == L.CSA2_ERR_INVALID_ARG       # lse is lse_b


def test_fake_quant_validation():
    lib = L.load()
    p = 4096
    assert lib.csa2_fake_quant_fp4(None, None, 0, L.DTYPE_F32, None) == L.CSA2_OK
    for n in (-32, 16, 33):
        assert lib.csa2_fake_quant_fp4(p, p, n, L.DTYPE_F32, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_fake_quant_fp4(p, p, 32, 2, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_fake_quant_fp4(None, p, 32, L.DTYPE_BF16, None) == L.CSA2_ERR_INVALID_ARG
    assert lib.csa2_fake_quant_fp4(p + 8, p, 32, L.DTYPE_BF16, None) == L.CSA2_ERR_INVALID_ARG


def _pool(lib, view, **kw):
    a = dict(q_idx=FAKE, w=FAKE, q_seq=FAKE, pool=FAKE, pool_cnt=FAKE, nq=1, h_idx=8, p=2048, k=512,
             out_idx=FAKE, out_cnt=FAKE, ws=FAKE, ws_bytes=1 << 20)
    a.update(kw)
    return lib.csa2_pool_index_topk(ctypes.byref(view), a["q_idx"], a["w"], a["q_seq"], a["pool"], a["pool_cnt"],
                                    a["nq"], a["h_idx"], a["p"], a["k"], a["out_idx"], a["out_cnt"], a["ws"],
                                    a["ws_bytes"], None)


@pytest.mark.parametrize("kw", [dict(h_idx=0), dict(h_idx=17), dict(p=0), dict(p=2049), dict(k=0), dict(k=2049),
                                dict(nq=-1), dict(pool=None), dict(pool_cnt=None), dict(pool=FAKE + 4),
                                dict(q_idx=None), dict(w=None), dict(ws=None), dict(out_idx=None),
                                dict(q_idx=FAKE + 8), dict(ws=FAKE + 4)])
def test_pool_index_rejects(kw):
    assert _pool(L.load(), _view(), **kw) == L.CSA2_ERR_INVALID_ARG


def test_pool_index_workspace_and_empty():
    lib = L.load()
    assert lib.csa2_pool_workspace_bytes(32, 2048) == 32 * 2048 * 4
    assert lib.csa2_pool_workspace_bytes(3, 100) == 3 * 128 * 4          # rows padded to 64 scores
    assert lib.csa2_pool_workspace_bytes(0, 100) == 0
    assert lib.csa2_pool_workspace_bytes(4, 2049) == 0
    assert _pool(lib, _view(), ws_bytes=2048 * 4 - 4) == L.CSA2_ERR_WORKSPACE
    assert _pool(lib, _view(), nq=0, q_idx=None, ws=None) == L.CSA2_OK
    # Full / Reindex workspaces leave room to score a pool of any width
    assert lib.csa2_workspace_bytes(L.CSA2_FULL, 8, 10, 8, 64, 64) >= lib.csa2_pool_workspace_bytes(8, 2048)


def test_layer_step_pool_field_rules():
    lib = L.load()
    v = _view()
    a = L.StepArgs()
    a.cache = ctypes.pointer(v)
    a.q, a.h, a.sm_scale, a.q_seq, a.q_vis, a.nq, a.k, a.max_vis = FAKE, 64, 0.04, FAKE, FAKE, 0, 512, 100
    a.idx, a.cnt, a.out = FAKE, FAKE, FAKE
    a.q_idx, a.w, a.h_idx, a.ws, a.ws_bytes = FAKE, FAKE, 8, FAKE, 1 << 30
    assert lib.csa2_layer_step(L.CSA2_REINDEX, ctypes.byref(a), None) == L.CSA2_OK       # nq = 0: nothing to do
    a.pool = FAKE                                        # pool fields without the flag
    assert lib.csa2_layer_step(L.CSA2_REINDEX, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.pool, a.pool_k = None, 1024
    assert lib.csa2_layer_step(L.CSA2_REINDEX, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.flags, a.pool, a.pool_cnt = L.STEP_POOL, FAKE + 4096, FAKE + 8192
    assert lib.csa2_layer_step(L.CSA2_REINDEX, ctypes.byref(a), None) == L.CSA2_OK
    assert lib.csa2_layer_step(L.CSA2_FULL, ctypes.byref(a), None) == L.CSA2_OK
    a.pool_k = 256                                       # pool narrower than k
    assert lib.csa2_layer_step(L.CSA2_REINDEX, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.pool_k = 2049
    assert lib.csa2_layer_step(L.CSA2_REINDEX, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.pool_k, a.nq = 1024, 1
    a.pool = FAKE + 4                                    # misaligned pool
    assert lib.csa2_layer_step(L.CSA2_FULL, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.pool = FAKE                                        # the pool is the layer's own output
    assert lib.csa2_layer_step(L.CSA2_FULL, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.pool, a.pool_cnt = FAKE + 4096, None
    assert lib.csa2_layer_step(L.CSA2_REINDEX, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG
    a.q_idx, a.w, a.h_idx, a.pool_cnt = None, None, 0, FAKE + 8192          # Reuse: no pool
    assert lib.csa2_layer_step(L.CSA2_REUSE, ctypes.byref(a), None) == L.CSA2_ERR_INVALID_ARG


def test_probe_library_exports_and_rejects():
    """The peak-probe library exports what its header declares and rejects
    out-of-range arguments before launching anything."""
    import re

    from fp4_kv_cache_layer_amd import probe
    lib = probe.load()
    txt = re.sub(r"/\*.*?\*/", "", open(probe.HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(csa2_probe_[a-z0-9_]+)\s*\(", txt)))
    assert names == ["csa2_probe_mfma_fp8", "csa2_probe_stream_read"]
    for n in names:
        assert hasattr(lib, n), n
    invalid = 1                                   # hipErrorInvalidValue
    for blocks, iters, epi in ((0, 4, 0), (1 << 21, 4, 0), (1, 0, 0), (1, 6, 0), (1, 4, 2)):
        assert lib.csa2_probe_mfma_fp8(blocks, iters, epi, FAKE, None) == invalid
    assert lib.csa2_probe_mfma_fp8(1, 4, 0, None, None) == invalid
    for src, nbytes, blocks in ((FAKE, 0, 1), (FAKE, 24, 1), (FAKE + 8, 32, 1), (FAKE, 32, 0), (None, 32, 1)):
        assert lib.csa2_probe_stream_read(src, nbytes, blocks, FAKE, None) == invalid


def test_idxk_bounds_build_checks():
    """The block-level representation's build rejects a cache without bounds,
    misaligned bounds and block ranges outside the cache (4 pages x 64 rows =
    4 blocks); an empty range is a no-op."""
    lib = L.load()
    assert lib.csa2_idxk_bounds_build(ctypes.byref(_view()), 0, 1, None) == L.CSA2_ERR_INVALID_ARG   # no bounds
    assert lib.csa2_idxk_bounds_build(ctypes.byref(_view(idxk_bounds=FAKE + 4)), 0, 1, None) == L.CSA2_ERR_INVALID_ARG
    v = _view(idxk_bounds=FAKE)
    for first, n in ((-1, 1), (0, -1), (0, 5), (3, 2)):
        assert lib.csa2_idxk_bounds_build(ctypes.byref(v), first, n, None) == L.CSA2_ERR_INVALID_ARG, (first, n)
    assert lib.csa2_idxk_bounds_build(ctypes.byref(v), 4, 0, None) == L.CSA2_OK
    assert lib.csa2_idxk_bounds_build(None, 0, 0, None) == L.CSA2_ERR_INVALID_ARG


def test_layer_step_prune_field_rules():
    """Block-level pruning: Full/Reindex only, not with the dense indexer or
    the pool, needs the cache's bounds and a seed; seed fields without the
    flag are rejected."""
    lib = L.load()
    for mode in (L.CSA2_FULL, L.CSA2_REINDEX, L.CSA2_REUSE):
        for bounds, flags, seed, ok in ((FAKE, L.STEP_PRUNE, FAKE, True),
                                        (None, L.STEP_PRUNE, FAKE, False),
                                        (FAKE, L.STEP_PRUNE, None, False),
                                        (FAKE, L.STEP_PRUNE | L.STEP_DENSE_INDEX, FAKE, False),
                                        (FAKE, 0, FAKE, False)):
            v = _view(idxk_bounds=bounds)
            a = L.StepArgs()
            a.cache = ctypes.pointer(v)
            a.q, a.h, a.sm_scale, a.q_seq, a.q_vis, a.nq, a.k, a.max_vis = FAKE, 64, 0.04, FAKE, FAKE, 1, 64, 200
            a.idx, a.cnt, a.out = FAKE, FAKE, FAKE
            if mode != L.CSA2_REUSE:
                a.q_idx, a.w, a.h_idx, a.ws, a.ws_bytes = FAKE, FAKE, 8, FAKE, 16   # workspace too small
            a.flags, a.seed, a.seed_cnt = flags, seed, seed
            st = lib.csa2_layer_step(mode, ctypes.byref(a), None)
            want = L.CSA2_ERR_WORKSPACE if (ok and mode != L.CSA2_REUSE) else L.CSA2_ERR_INVALID_ARG
            assert st == want, (mode, bounds, flags, seed, st)
