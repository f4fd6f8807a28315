"""Pins for the oracle's number formats and row encoding (CPU only).

Each pin comes from outside the oracle: the OCP MX and OFP8 value tables
(golden files), torch's own float8_e4m3fn / float8_e8m0fnu conversions (a
library routine independent of the oracle), brute-force nearest search, and a
hand-worked row.
"""
import os

import numpy as np
import pytest
import torch
from hypothesis import given, settings, strategies as st

from oracle import csa2_oracle as O

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _pairs(name):
    out = []
    with open(os.path.join(GOLD, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                a, b = line.split()
                out.append((a, b))
    return out


def test_e2m1_table_matches_ocp():
    for code, val in _pairs("e2m1_values.txt"):
        c = int(code, 16)
        got = float(O.e2m1_decode(c))
        assert got == float(val), (code, got, val)
        assert np.signbit(got) == val.startswith("-"), code


def test_e2m1_roundtrip_all_16_codes():
    codes = np.arange(16)
    assert (O.e2m1_encode(O.e2m1_decode(codes)) == codes).all()


def test_e2m1_rounding_golden():
    for r, code in _pairs("e2m1_rounding.txt"):
        assert int(O.e2m1_encode(float(r))) == int(code, 16), (r, code)


def test_e2m1_encode_bruteforce():
    """Nearest of all 16 codes (same sign as input), ties to the even code."""
    rng = np.random.default_rng(5)
    r = np.concatenate([rng.uniform(-6, 6, 4000), np.arange(-24, 25) / 4.0])
    vals = np.array([O.e2m1_decode(c) for c in range(16)], dtype=np.float64)
    got = O.e2m1_encode(r)
    for x, g in zip(r, got):
        best = None
        for c in range(16):
            if bool(c & 8) != bool(np.signbit(x)):
                continue
            d = abs(x - vals[c])
            if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
                best = (d, c)
        assert g == best[1], (x, g, best)


def test_e8m0_decode_matches_torch():
    codes = np.arange(256)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e8m0fnu).double().numpy()
    got = O.e8m0_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])


def test_e4m3_decode_matches_torch_all_256():
    codes = np.arange(256)
    ref = torch.from_numpy(codes.astype(np.uint8)).view(torch.float8_e4m3fn).double().numpy()
    got = O.e4m3fn_decode(codes)
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    m = ~np.isnan(ref)
    assert np.array_equal(ref[m], got[m])
    assert np.array_equal(np.signbit(ref[m]), np.signbit(got[m]))


def test_e4m3_golden_points():
    for code, val in _pairs("e4m3fn_points.txt"):
        got = float(O.e4m3fn_decode(int(code, 16)))
        if val == "nan":
            assert np.isnan(got), code
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), (code, got)


def test_e4m3_encode_matches_torch_on_every_bf16():
    """All 65,536 bf16 patterns: finite values with |x| <= 448 encode exactly
    as torch's round-to-nearest-even cast; larger finite values saturate."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = O.bf16_to_f64(bits)
    fin = np.isfinite(x)
    inr = fin & (np.abs(x) <= 448)
    ref = torch.from_numpy(x[inr]).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = O.e4m3fn_encode(x[inr])
    bad = np.nonzero(ref != got)[0]
    assert bad.size == 0, [(x[inr][i], ref[i], got[i]) for i in bad[:5]]
    big = fin & (np.abs(x) > 448)
    sat = O.e4m3fn_encode(x[big])
    assert ((sat & 0x7F) == 0x7E).all()
    assert np.array_equal(sat >> 7, np.signbit(x[big]).astype(np.uint8))


def test_e4m3_integers_exact():
    v = np.arange(-16, 17, dtype=np.float64)
    assert np.array_equal(O.e4m3fn_decode(O.e4m3fn_encode(v)), v)


def test_block_exponent_closed_forms():
    for k in range(-120, 120, 7):
        a = 6.0 * 2.0 ** k
        assert O.block_exponent(a) == k
        # next bf16 value above 6 * 2^k needs the next power of two
        assert O.block_exponent(a * (1 + 2.0 ** -7)) == k + 1
        # 3 * 2^k + ulp still fits under 6 * 2^k
        assert O.block_exponent(3.0 * 2.0 ** k * (1 + 2.0 ** -7)) == k
        assert O.block_exponent(3.0 * 2.0 ** k) == k - 1
    assert O.block_exponent(0.0) == -127
    assert O.block_exponent(2.0 ** -133) == -127           # smallest bf16 subnormal: clamped
    big = float(O.bf16_to_f64(np.uint16(0x7F7F)))           # largest finite bf16
    assert O.block_exponent(big) == 126
    assert O.block_exponent(1.0) == -2                      # 6 * 2^-3 = 0.75 < 1 <= 1.5


def test_kv_row_hand_worked_example():
    spec = dict(l.split(None, 1) for l in open(os.path.join(GOLD, "kv_row_example.txt"))
                if l.strip() and not l.startswith("#"))
    pat = []
    for tok in spec["pattern"].split():
        if "*" in tok:
            v, n = tok.split("*")
            pat += [float(v)] * int(n)
        else:
            pat.append(float(tok))
    assert len(pat) == 32
    shift = int(spec["block_shift"])
    row = np.concatenate([np.array(pat) * 2.0 ** (j + shift) for j in range(16)])
    blk = []
    for tok in spec["bytes_per_block"].split():
        if "*" in tok:
            v, n = tok.split("*")
            blk += [int(v, 16)] * int(n)
        else:
            blk.append(int(tok, 16))
    want = np.array(blk * 16 + [int(spec["scale_base"]) + j for j in range(16)], dtype=np.uint8)
    got = O.quantize_kv_rows(row[None])[0]
    assert got.shape == (272,)
    assert np.array_equal(got, want)


def test_kv_roundtrip_exact_on_grid():
    rng = np.random.default_rng(1)
    grid = np.array([O.e2m1_decode(c) for c in range(16)])
    for _ in range(50):
        e = rng.integers(-30, 30, size=16)
        codes = rng.integers(0, 16, size=(16, 32))
        codes[:, 0] = 7                                     # block max 6 * 2^e fixes the scale at e
        x = (grid[codes] * 2.0 ** e[:, None]).reshape(-1)
        y = O.dequantize_kv_rows(O.quantize_kv_rows(x[None]))[0]
        assert np.array_equal(x, y)


@settings(max_examples=60, deadline=None)
@given(st.integers(0, 2 ** 32 - 1), st.floats(-40, 40))
def test_kv_quant_error_bound(seed, log2scale):
    """|x - deq(q(x))| <= half the local grid gap times 2^e, and 2^e < amax/3."""
    rng = np.random.default_rng(seed)
    x32 = (rng.standard_normal(512) * 2.0 ** log2scale).astype(np.float32)
    bits = (x32.view(np.uint32) >> 16).astype(np.uint16)    # truncate to a bf16 value
    x = O.bf16_to_f64(bits)
    b = O.quantize_kv_rows(x[None])[0]
    y = O.dequantize_kv_rows(b[None])[0]
    e = b[256:].astype(np.int64) - 127
    xb = x.reshape(16, 32)
    yb = y.reshape(16, 32)
    for j in range(16):
        s = 2.0 ** e[j]
        r = np.abs(xb[j]) / s
        half_gap = np.where(r <= 2, 0.25, np.where(r <= 4, 0.5, 1.0)) * s
        assert (np.abs(xb[j] - yb[j]) <= half_gap).all()
        amax = np.abs(xb[j]).max()
        if amax > 0 and e[j] > -127:
            assert s < amax / 3 * (1 + 1e-12) and amax <= 6 * s


def test_idxk_row_is_elementwise_e4m3():
    rng = np.random.default_rng(2)
    x = rng.integers(-8, 9, size=(5, 128)).astype(np.float64)
    b = O.quantize_idxk_rows(x)
    assert b.shape == (5, 128)
    assert np.array_equal(O.e4m3fn_decode(b), x)


def test_bf16_decode_matches_torch_every_pattern():
    """bf16_to_f64 against torch's own bfloat16 -> float64 conversion on all
    65,536 bit patterns: values equal, NaN at the same positions, sign bits
    equal (so -0 stays -0)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    got = O.bf16_to_f64(bits)
    want = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).double().numpy()
    nan = np.isnan(want)
    assert (np.isnan(got) == nan).all()
    assert (got[~nan] == want[~nan]).all()
    assert (np.signbit(got[~nan]) == np.signbit(want[~nan])).all()
    assert nan.sum() == 2 * 127                     # exponent 0xFF with a nonzero mantissa, both signs


def test_bf16_decode_closed_forms():
    """bf16 is fp32's top half: sign, 8 exponent bits (bias 127), 7 mantissa
    bits; exponent 0 is subnormal (m * 2^-133), exponent 0xFF with m = 0 is
    infinity.  Spot values written from that definition, not from the oracle."""
    cases = {0x0000: 0.0, 0x8000: -0.0, 0x3F80: 1.0, 0xBF80: -1.0, 0x4000: 2.0, 0xC040: -3.0,
             0x3F00: 0.5, 0x3FC0: 1.5, 0x4120: 10.0, 0x0001: 2.0 ** -133, 0x807F: -127 * 2.0 ** -133,
             0x0080: 2.0 ** -126, 0x7F7F: (2 - 2.0 ** -7) * 2.0 ** 127, 0x7F80: np.inf, 0xFF80: -np.inf,
             0x3E00: 0.125, 0x42F6: 123.0}
    for b, v in cases.items():
        got = float(O.bf16_to_f64(np.array([b], dtype=np.uint16))[0])
        assert got == v and np.signbit(got) == np.signbit(v), (hex(b), got, v)
    # every normal pattern against the bit-field formula, in exact Python integers
    for b in range(0, 1 << 16, 97):
        s, e, m = b >> 15, (b >> 7) & 0xFF, b & 0x7F
        if e == 0xFF:
            continue
        mag = m * 2.0 ** -133 if e == 0 else (128 + m) * 2.0 ** (e - 134)
        assert float(O.bf16_to_f64(np.array([b], dtype=np.uint16))[0]) == (-mag if s else mag), hex(b)
