"""Number formats of the CSA2 KV cache, written out from their definitions.

TEST INFRASTRUCTURE: see oracle/__init__.py for who may use this package.

Sources. The pages (ai-wave.ru, "DeepSeek V4.1-Flash: 1M context, FP4 KV cache
and an attention-reuse architecture", fourth paragraph; agentnet.co.il,
"DeepSeek launches V4.1-Flash ...", section "Quantization and deployment")
name the main-KV format only as E2M1 values with one E4M3 scale per 16
channels, following NVFP4 with the global scale left out.  The bit layouts of
E2M1 and E4M3 themselves come from the public OCP Microscaling (MX) format
specification: E2M1 has 1 sign, 2 exponent (bias 1) and 1 mantissa bit; E4M3
("E4M3FN") has 1 sign, 4 exponent (bias 7) and 3 mantissa bits, subnormals
m * 2**-9, a largest finite magnitude of 448, no infinities, and NaN at
0x7F / 0xFF.

Rounding (a reading, the pages are silent): round to nearest, ties to the
code whose lowest bit is 0 ("ties to even"), saturating at the largest
finite magnitude, sign kept even when the magnitude rounds to zero.

Everything here is float64 numpy: every E2M1 and E4M3 value, and every
midpoint between neighbours, is a short dyadic rational and exact in float64.
"""

import numpy as np

# --- E2M1 -------------------------------------------------------------------


def e2m1_value(code):
    """Value of 4-bit E2M1 codes (int array) as float64."""
    code = np.asarray(code, dtype=np.int64)
    sign = (code >> 3) & 1
    exp = (code >> 1) & 3
    man = code & 1
    # exponent field 0 is subnormal: 0.m * 2**(1 - bias) with bias 1
    mag = np.where(exp == 0, man * 0.5, (1.0 + 0.5 * man) * np.exp2(exp - 1.0))
    return np.where(sign == 1, -mag, mag)


# magnitudes of codes 0..7 in code order (ascending)
E2M1_GRID = e2m1_value(np.arange(8))


def _nearest_ties_even(mag, grid):
    """Index into the ascending grid nearest to mag; ties go to the even index;
    magnitudes beyond the last grid point saturate to it."""
    mag = np.asarray(mag, dtype=np.float64)
    hi = np.clip(np.searchsorted(grid, mag, side="left"), 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = mag - grid[lo]
    d_hi = grid[hi] - mag
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(mag >= grid[-1], len(grid) - 1, idx)
    return idx.astype(np.int64)


def e2m1_encode(r):
    """E2M1 code of the real value r (float64): nearest magnitude, ties to the
    even code, saturating at 6; the sign bit is the sign of r, so a negative r
    that rounds to zero gives code 0x8."""
    r = np.asarray(r, dtype=np.float64)
    code = _nearest_ties_even(np.abs(r), E2M1_GRID)
    return (code | (np.signbit(r).astype(np.int64) << 3)).astype(np.uint8)


# --- E4M3 (E4M3FN) ----------------------------------------------------------


def e4m3_value(code):
    """Value of 8-bit E4M3FN codes (int array) as float64; 0x7F/0xFF are NaN."""
    code = np.asarray(code, dtype=np.int64)
    sign = (code >> 7) & 1
    exp = (code >> 3) & 15
    man = code & 7
    mag = np.where(exp == 0, man * 2.0 ** -9, (1.0 + man / 8.0) * np.exp2(exp - 7.0))
    mag = np.where((exp == 15) & (man == 7), np.nan, mag)
    return np.where(sign == 1, -mag, mag)


# magnitudes of the finite non-negative codes 0x00..0x7E in code order (ascending)
E4M3_GRID = e4m3_value(np.arange(0x7F))
E4M3_MAX = 448.0


def e4m3_encode(v):
    """E4M3FN code of the real value v (float64): nearest finite value, ties to
    the even code, saturating at +-448, sign kept for values rounding to 0."""
    v = np.asarray(v, dtype=np.float64)
    if not np.all(np.isfinite(v)):
        raise ValueError("non-finite input is outside the contract")
    code = _nearest_ties_even(np.abs(v), E4M3_GRID)
    return (code | (np.signbit(v).astype(np.int64) << 7)).astype(np.uint8)


# --- bfloat16 ----------------------------------------------------------------


def bf16_value(bits):
    """float64 value of bfloat16 bit patterns (uint16 array): the upper half of
    an IEEE binary32."""
    bits = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)
