"""Number formats of the NVFP4 block-scaled path, written from their definitions.

Test infrastructure (see the package header): plain NumPy, float64 wherever a
value is formed, exhaustive tables instead of bit tricks, so that every line can
be checked by eye.

Source of the format: "From Empirical Limits to Research-Driven Optimization:
The SM120 FP4 Kernel Research Campaign", section "Section 1: CUTLASS Kernels -
The Foundation", which gives the block-scaled MMA the method runs on: both
operands are ``e2m1`` (4-bit float), the block scales are ``ue4m3`` (an 8-bit
E4M3 float used without sign), ``scale_vec::4X`` on a K=64 instruction means four
scales per 64 K-elements, i.e. one scale per 16 consecutive K-elements, and the
accumulator is ``f32``.  E2M1 and E4M3 themselves are the OCP 8-bit/4-bit
floating-point formats (OCP Microscaling Formats v1.0 / OCP 8-bit FP spec).
"""
from __future__ import annotations

import numpy as np

# ---------------------------------------------------------------------------
# E2M1: 1 sign bit, 2 exponent bits (bias 1), 1 mantissa bit, no inf/nan.
# ---------------------------------------------------------------------------


def e2m1_value(code: int) -> float:
    """Value of one 4-bit E2M1 code from the bit fields (s e1 e0 m)."""
    s = (code >> 3) & 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        mag = 0.5 * m                       # subnormal: m * 2^(1-bias) * 2^-1
    else:
        mag = 2.0 ** (e - 1) * (1.0 + m / 2.0)
    return -mag if s else mag


E2M1_TABLE = np.array([e2m1_value(c) for c in range(16)], dtype=np.float64)
E2M1_MAGNITUDES = E2M1_TABLE[:8].copy()      # 0, .5, 1, 1.5, 2, 3, 4, 6


def e2m1_decode(codes: np.ndarray) -> np.ndarray:
    return E2M1_TABLE[np.asarray(codes, dtype=np.int64) & 0xF]


# ---------------------------------------------------------------------------
# E4M3 (OCP "E4M3FN"): 1 sign, 4 exponent bits (bias 7), 3 mantissa bits,
# subnormals, no infinities, S.1111.111 is NaN, max finite 448.
# ---------------------------------------------------------------------------


def e4m3_value(code: int) -> float:
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 7
    if e == 0xF and m == 7:
        return float("nan")
    if e == 0:
        mag = m * 2.0 ** -9                  # m/8 * 2^(1-7)
    else:
        mag = 2.0 ** (e - 7) * (1.0 + m / 8.0)
    return -mag if s else mag


E4M3_TABLE = np.array([e4m3_value(c) for c in range(256)], dtype=np.float64)
# finite non-negative values, ascending with the code: codes 0..126
E4M3_POS = E4M3_TABLE[:127].copy()
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_TABLE[np.asarray(codes, dtype=np.int64) & 0xFF]


def _nearest_code_ties_even(x: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the grid value nearest to each x (grid ascending, x >= 0,
    x <= grid[-1]); an exact tie goes to the even index.  For E2M1 and E4M3 the
    index is the code, and an even code has a zero mantissa LSB, so this is
    IEEE round-to-nearest-even restricted to the format."""
    x = np.asarray(x, dtype=np.float64)
    hi = np.searchsorted(grid, x, side="left")          # grid[hi] >= x
    hi = np.clip(hi, 0, len(grid) - 1)
    lo = np.clip(hi - 1, 0, len(grid) - 1)
    d_lo = x - grid[lo]
    d_hi = grid[hi] - x
    pick_hi = d_hi < d_lo
    tie = d_hi == d_lo
    pick_hi = np.where(tie, (hi % 2) == 0, pick_hi)
    out = np.where(pick_hi, hi, lo)
    out = np.where(x == grid[hi], hi, out)               # exact hit
    return out.astype(np.int64)


def e4m3_encode_satfinite(t: np.ndarray) -> np.ndarray:
    """Non-negative float -> E4M3 code, nearest with ties to even, values at or
    above 448 clamp to 448 (code 0x7E)."""
    t = np.asarray(t, dtype=np.float64)
    assert np.all(t >= 0) and np.all(np.isfinite(t)), "scales are finite and >= 0"
    tc = np.minimum(t, E4M3_MAX)
    return _nearest_code_ties_even(tc, E4M3_POS).astype(np.uint8)


def e2m1_encode_magnitude(v: np.ndarray) -> np.ndarray:
    """|v| -> 3-bit E2M1 magnitude code, nearest with ties to even, saturating at 6."""
    v = np.asarray(v, dtype=np.float64)
    assert np.all(v >= 0) and np.all(np.isfinite(v))
    vc = np.minimum(v, 6.0)
    return _nearest_code_ties_even(vc, E2M1_MAGNITUDES).astype(np.uint8)


# ---------------------------------------------------------------------------
# bfloat16 rounding (8 significant bits, ties to even) of float64 values.
# ---------------------------------------------------------------------------


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float64 -> nearest bfloat16 value (ties to even), returned as float32.

    Rounds the float64 value directly to 8 significant bits (no intermediate
    float32 rounding).  Valid for the normal bfloat16 range, which is all this
    path produces."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                  # x = m * 2^e, 0.5 <= |m| < 1
    r = np.rint(m * 256.0) / 256.0      # np.rint rounds half to even
    return np.ldexp(r, e).astype(np.float32)


def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """bfloat16 bit pattern of float32 values that are already bfloat16 values."""
    b = np.asarray(x32, dtype=np.float32).view(np.uint32)
    assert np.all((b & 0xFFFF) == 0), "value is not a bfloat16 value"
    return (b >> 16).astype(np.uint16)
