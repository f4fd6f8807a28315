"""The peak probes run on the GPU and report rates within the part's limits."""
import pytest
import torch

from tests.gpu_util import need_gpu, say

pytestmark = pytest.mark.gpu


def test_probe_rates_are_plausible():
    need_gpu()
    from fp4_kv_cache_layer_amd import probe
    say("[probe] mfma fp8 (bare, with epilogue), stream read 64 MiB")
    bare = probe.mfma_fp8_tflops(iters=1024, reps=3)
    epi = probe.mfma_fp8_tflops(epilogue=True, iters=1024, reps=3)
    assert 1000.0 < bare < 5000.0 * 1.05
    assert 500.0 < epi <= bare * 1.05
    buf = torch.ones(2 * 64 << 20, dtype=torch.uint8, device="cuda")
    gbps = probe.stream_read_gbps(buf, 64 << 20, rotate=2, reps=4)
    assert 500.0 < gbps < 8000.0 * 1.5           # a 64 MiB slice may partly hit the last-level cache
