"""Pins of the oracle's FP4 fake quantisation (the forward of
quantization-aware training with the main-KV E2M1 + E8M0 rules): a
hand-worked example, fixed points on the E2M1 grid, the error bound,
idempotence, and agreement with the cache's row encoder and decoder."""
import os

import numpy as np

from oracle import csa2_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fake_quant_example.txt")


def test_worked_example():
    rows = np.loadtxt(GOLDEN)
    x, want = rows[0::2], rows[1::2]
    got = O.fake_quant_e2m1(x)
    assert np.array_equal(got, want)
    assert np.array_equal(np.signbit(got), np.signbit(want))          # -0.25 -> -0


def test_grid_values_are_fixed_points():
    rng = np.random.default_rng(1)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6])
    for _ in range(50):
        e = int(rng.integers(-30, 30))
        v = grid[rng.integers(0, 8, 32)] * np.where(rng.random(32) < 0.5, -1, 1)
        v[rng.integers(0, 32)] = 6.0 * (1 if rng.random() < 0.5 else -1)   # amax = 6 * 2^e
        x = v * 2.0 ** e
        assert np.array_equal(O.fake_quant_e2m1(x), x)


def test_error_bound_sign_and_idempotence():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((64, 512)) * np.exp2(rng.integers(-40, 40, (64, 1)))
    y = O.fake_quant_e2m1(x)
    b, yb = x.reshape(-1, 32), y.reshape(-1, 32)
    scale = np.exp2(O.block_exponent(np.abs(b).max(axis=1)).astype(np.float64))[:, None]
    assert (np.abs(yb - b) <= scale + 0).all()                         # half the widest gap (2) of the grid
    assert (np.abs(yb) <= 6 * scale).all()
    assert np.array_equal(np.signbit(y), np.signbit(x))
    assert np.array_equal(O.fake_quant_e2m1(y), y)


def test_matches_cache_encoder_and_decoder():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((20, 512)) * np.exp2(rng.integers(-10, 10, (20, 1)))
    x[3, 64:96] = 0.0                                                 # an all-zero block
    via_cache = O.dequantize_kv_rows(O.quantize_kv_rows(x))
    assert np.array_equal(O.fake_quant_e2m1(x), via_cache)
