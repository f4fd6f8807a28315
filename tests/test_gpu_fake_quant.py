"""GPU parity of csa2_fake_quant_fp4 (the FP4 quantization-aware-training
forward) against the oracle, bit for bit (sign of zero included), for fp32
and bf16 inputs; the straight-through backward."""
import numpy as np
import pytest
import torch

from oracle import csa2_oracle as O
from tests.gpu_util import say

pytestmark = pytest.mark.gpu


def _ops():
    from fp4_kv_cache_layer_amd import ops
    return ops


def _inputs(rng, n, kind):
    if kind == "normal":
        x = rng.standard_normal(n)
    elif kind == "spread":                                  # block scales over the whole E8M0 range
        x = rng.standard_normal(n) * np.exp2(np.repeat(rng.integers(-140, 126, n // 32), 32).astype(np.float64))
    else:                                                   # ties, zeros, signed zeros, grid values
        grid = np.array([0, 0.25, 0.5, 0.75, 1, 1.25, 1.5, 1.75, 2, 2.5, 3, 3.5, 4, 5, 6])
        x = grid[rng.integers(0, len(grid), n)] * np.where(rng.random(n) < 0.5, -1.0, 1.0)
        x[rng.random(n) < 0.05] = -0.0
        x = x * np.exp2(np.repeat(rng.integers(-20, 20, n // 32), 32).astype(np.float64))
    return x


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("n,kind", [(32, "ties"), (32 * 777, "normal"), (512 * 301, "spread"), (32 * 4099, "ties")])
def test_fake_quant_bit_exact(dtype, n, kind):
    ops = _ops()
    say(f"[fake_quant] dtype={dtype} n={n} kind={kind}")
    rng = np.random.default_rng(n + len(kind))
    x = _inputs(rng, n, kind).astype(np.float32)
    if dtype == "bf16":
        xt = torch.from_numpy(x).to(torch.bfloat16)
        x = xt.float().numpy()                             # the values the kernel sees
    else:
        xt = torch.from_numpy(x)
    y = ops.csa2_fake_quant_fp4(xt.cuda()).cpu().float().numpy()
    want = O.fake_quant_e2m1(x.astype(np.float64).reshape(-1, 32)).reshape(-1).astype(np.float32)
    assert np.array_equal(y.view(np.uint32), want.view(np.uint32)), np.nonzero(y != want)[0][:5]


def test_fake_quant_in_place_and_straight_through():
    ops = _ops()
    rng = np.random.default_rng(9)
    x = torch.from_numpy(rng.standard_normal(32 * 64).astype(np.float32)).cuda()
    want = ops.csa2_fake_quant_fp4(x)
    y = x.clone()
    ops.csa2_fake_quant_fp4(y, out=y)
    assert torch.equal(y, want)
    xr = x.clone().requires_grad_(True)
    out = ops.FakeQuantFP4.apply(xr)
    g = torch.from_numpy(rng.standard_normal(32 * 64).astype(np.float32)).cuda()
    out.backward(g)
    assert torch.equal(out.detach(), want) and torch.equal(xr.grad, g)
