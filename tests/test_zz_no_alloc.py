"""csa2_layer_step_static (the layer step whose workspace is the library's
own fixed device array, for callers that cannot allocate) against
csa2_layer_step with a caller workspace: identical bits, on two calls in a
row, the second with a smaller input; shapes beyond the array are refused."""
import ctypes

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    need_gpu()


def _static_call(call):
    from fp4_kv_cache_layer_amd import _lib as L
    a = L.StepArgs()
    ctypes.memmove(ctypes.byref(a), ctypes.byref(call.args), ctypes.sizeof(L.StepArgs))
    a.ws, a.ws_bytes = None, 0
    st = L.load().csa2_layer_step_static(call.mode, ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    L.check("csa2_layer_step_static", st)


def _run(spec):
    from fp4_kv_cache_layer_amd import runner
    say(f"[static] {spec.name}: {spec.num_seqs} seqs, cached {spec.cached[:4]}, modes {spec.modes}")
    dc = runner.DeviceCase(spec, gen_device="cpu")
    dc.run_layers()                                   # csa2_layer_step, caller workspace
    want = dc.results_host()
    for o in dc.outputs:                              # clobber, then the static entry point
        o["out"].fill_(float("nan"))
        o["lse"].fill_(float("nan"))
        o["idx"].fill_(-9)
        o["cnt"].fill_(-9)
    for c in dc.calls:
        _static_call(c)
    got = dc.results_host()
    for li, (x, y) in enumerate(zip(got, want)):
        for key in ("idx", "cnt", "out", "lse"):
            assert np.array_equal(x[key], y[key]), (spec.name, li, key)
    return dc


def test_static_matches_layer_step_twice_second_smaller():
    big = W.small_case("static_big", 71, [20000, 9000, 4096, 300], n_new=1, h_idx=8, h=64, k=512,
                       integer_indexer=False)
    small = W.small_case("static_small", 72, [1500, 77], n_new=1, h_idx=4, h=16, k=256, integer_indexer=True)
    _run(big)
    _run(small)


def test_static_refuses_shapes_beyond_the_array():
    from fp4_kv_cache_layer_amd import _lib as L
    from fp4_kv_cache_layer_amd import ops
    lib = L.load()
    nq, max_vis = 64, 1 << 20                          # needs far more than the array holds
    assert lib.csa2_workspace_bytes(L.CSA2_FULL, nq, max_vis, 8, 64, 512) > L.STATIC_SCRATCH_BYTES
    npg = max_vis // 4096
    cache = ops.Cache(npg, 4096, torch.arange(npg, dtype=torch.int32)[None].repeat(1, 1))
    a = L.StepArgs()
    a.cache = ctypes.pointer(cache.view)
    dev = torch.zeros(1 << 16, dtype=torch.uint8, device="cuda")
    p = dev.data_ptr()
    a.q_idx, a.w, a.h_idx = p, p, 8
    a.q, a.h, a.sm_scale, a.q_seq, a.q_vis, a.nq, a.k, a.max_vis = p, 64, 0.04, p, p, nq, 512, max_vis
    a.idx, a.cnt, a.out = p, p, p
    st = lib.csa2_layer_step_static(L.CSA2_REINDEX, ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    assert st == L.CSA2_ERR_WORKSPACE
    a.ws, a.ws_bytes = p, 1 << 16                      # a caller workspace is not taken
    st = lib.csa2_layer_step_static(L.CSA2_REINDEX, ctypes.byref(a), torch.cuda.current_stream().cuda_stream)
    assert st == L.CSA2_ERR_INVALID_ARG
