"""Pins of the oracle's number formats: published tables, a library decoder,
brute force in exact rationals, and hand-worked FP4 blocks."""

import os
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle.formats import E2M1_GRID, E4M3_GRID

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return [l.split("#")[0].strip() for l in f if l.split("#")[0].strip()]


def test_e2m1_table_matches_spec():
    for row in _rows("e2m1_table.txt"):
        code, val = row.split()
        got = float(oracle.e2m1_value(int(code, 16)))
        assert got == float(val) and np.signbit(got) == val.startswith("-"), row


def test_e4m3_points_match_spec():
    for row in _rows("e4m3_points.txt"):
        code, val = row.split()
        got = float(oracle.e4m3_value(int(code, 16)))
        if val == "nan":
            assert np.isnan(got)
        else:
            assert got == float(val) and np.signbit(got) == val.startswith("-"), row


def test_e4m3_all_codes_match_torch_decoder():
    codes = torch.arange(256, dtype=torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = oracle.e4m3_value(np.arange(256))
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(1)
    v = np.concatenate([
        rng.standard_normal(20000) * 30,
        rng.standard_normal(5000) * 2.0 ** -8,                       # subnormal range
        (E4M3_GRID[:-1] + E4M3_GRID[1:]) / 2,                        # every tie
        -(E4M3_GRID[:-1] + E4M3_GRID[1:]) / 2,
        E4M3_GRID, -E4M3_GRID, [448.0, -448.0]])
    v = np.clip(v, -448, 448).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = oracle.e4m3_encode(v.astype(np.float64))
    assert np.array_equal(ref, got)


def test_e4m3_encode_saturates():
    assert list(oracle.e4m3_encode([448.0, 460.0, 1e6, -1e6])) == [0x7E, 0x7E, 0x7E, 0xFE]


def _nearest_exact(r, grid):
    """Brute force: nearest grid magnitude to the exact rational r, ties to the
    even index, saturating."""
    r = abs(r)
    if r >= grid[-1]:
        return len(grid) - 1
    best = None
    for i, g in enumerate(grid):
        d = abs(r - g)
        if best is None or d < best[0] or (d == best[0] and i % 2 == 0):
            best = (d, i)
    return best[1]


def test_fp4_encode_brute_force_exact_rationals():
    rng = np.random.default_rng(7)
    e2m1 = [Fraction(float(g)) for g in E2M1_GRID]
    e4m3 = [Fraction(float(g)) for g in E4M3_GRID]
    blocks = (rng.standard_normal((600, 16)) * np.exp(rng.uniform(-9, 8, (600, 1)))).astype(np.float32)
    x = np.zeros((600 // 32 + 1, 512), np.float32).reshape(-1)
    x[: blocks.size] = blocks.reshape(-1)
    x = x.reshape(-1, 512)
    nib, scale = oracle.fp4_encode_rows(x)
    for bi in range(600):
        row, blk = divmod(bi, 32)
        xs = [Fraction(float(v)) for v in x[row, 16 * blk: 16 * blk + 16]]
        amax = max(abs(v) for v in xs)
        sc = _nearest_exact(amax / 6, e4m3)
        assert scale[row, blk] == sc, bi
        s = e4m3[sc]
        for c in range(16):
            ch = 16 * blk + c
            byte = int(nib[row, ch // 2])
            code = (byte >> 4) if ch % 2 else (byte & 15)
            if s == 0:
                assert code == 0
                continue
            want = _nearest_exact(xs[c] / s, e2m1) | (8 if np.signbit(x[row, ch]) else 0)
            assert code == want, (bi, c)


def test_fp4_golden_blocks():
    for row in _rows("fp4_blocks.txt"):
        name, xs, sc, by = [t.strip() for t in row.split("|")]
        x = np.zeros((1, 512), np.float32)
        x[0, :16] = [float(t) for t in xs.split()]
        nib, scale = oracle.fp4_encode_rows(x)
        assert scale[0, 0] == int(sc, 16), name
        assert [int(b, 16) for b in by.split()] == list(nib[0, :8]), name


def test_fp4_roundtrip_error_bound_and_symmetries():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((64, 512)).astype(np.float32)
    nib, scale = oracle.fp4_encode_rows(x)
    y = oracle.fp4_decode_rows(nib, scale)
    s = np.repeat(oracle.e4m3_value(scale), 16, axis=1)
    # nearest-value rounding: error at most half the widest E2M1 gap (1.0 between 4 and 6)
    # in scale units, plus the clip of an amax element when S rounded down
    amax = np.repeat(np.abs(x.reshape(64, 32, 16)).max(axis=2), 16, axis=1)
    assert np.all(np.abs(y - x) <= np.maximum(1.0 * s, amax - 6 * s) + 1e-12)
    # sign symmetry: negating the input flips only the sign bits
    nib2, scale2 = oracle.fp4_encode_rows(-x)
    assert np.array_equal(scale, scale2) and np.array_equal(nib ^ 0x88, nib2)
    # power-of-two scaling shifts only the scale exponent
    nib3, scale3 = oracle.fp4_encode_rows(x * np.float32(4.0))
    assert np.array_equal(nib, nib3)
    assert np.array_equal(oracle.e4m3_value(scale3), 4 * oracle.e4m3_value(scale))


def test_bf16_value_matches_torch_on_every_pattern():
    # every one of the 65,536 bfloat16 bit patterns against torch's own
    # bfloat16 -> float64 conversion: the value, its sign (signed zeros) and
    # NaN-ness
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.bf16_value(bits)
    assert got.dtype == np.float64
    assert np.array_equal(np.isnan(ref), np.isnan(got))
    ok = ~np.isnan(ref)
    assert np.array_equal(ref[ok], got[ok])
    assert np.array_equal(np.signbit(ref[ok]), np.signbit(got[ok]))
    # closed forms: 0x3F80 = 1, 0xC000 = -2, 0x7F80 = +inf, 0x0001 = 2^-133
    assert got[0x3F80] == 1.0 and got[0xC000] == -2.0 and np.isposinf(got[0x7F80])
    assert got[0x0001] == 2.0 ** -133
