"""MXFP4: E2M1 values with one E8M0 power-of-two scale per 32 consecutive
values along the reduction axis (CPU oracle; test infrastructure).

The pages name MXFP4 as the format of the other grouped-GEMM line of work they
survey ("From Empirical Limits to Research-Driven Optimization: The SM120 FP4
Kernel Research Campaign", section "Sections 2-4: Framework and Community
Landscape": an MXFP4 grouped GEMM with 128x128x128 tiles) but do not define
it.  The format is the OCP Microscaling (MX) v1.0 one, read here as:

* element   E2M1 (the same 4-bit code as NVFP4: +-{0, .5, 1, 1.5, 2, 3, 4, 6})
* scale     E8M0: an 8-bit biased exponent, code c means 2^(c - 127); code 255
            (NaN) is never produced
* block     32 consecutive values along the reduction axis share one scale;
            no per-tensor scale
* encode    X = floor(log2(absmax_block)) - 2 (2 = the exponent of E2M1's
            largest power of two, so absmax / 2^X lies in [4, 8)), clamped to
            [-127, 127]; code = E2M1 nearest-even of x / 2^X, saturating at 6,
            sign copied from x; an all-zero block gets scale code 0 and codes 0
* value     E2M1(q) * 2^X

Dividing by a power of two is exact, so the E2M1 decision here needs no
rounding rule beyond nearest-even on the exact quotient.

The GEMM is the block-scaled product of the two operands, per expert, with an
optional float32 multiplier per operand (1 for plain MX tensors):
    y[p, n] = g_a g_b[e] sum_kb 2^(Xa[r,kb] + Xb[e,n,kb]) sum_{i<32} q_a q_b
Every product of two MX values is exact in float64; the sum runs in float64
(numpy matmul as the summation primitive) and is rounded to float32 once.
"""
from __future__ import annotations

import numpy as np

from .formats import e2m1_decode, e2m1_encode_magnitude
from .quant import pack_codes, unpack_codes

MX_BLOCK = 32
E8M0_BIAS = 127


def e8m0_value(code: int) -> float:
    """Value of one E8M0 scale code from its definition (NaN for 255)."""
    code = int(code)
    if code == 255:
        return float("nan")
    return 2.0 ** (code - E8M0_BIAS)


E8M0_TABLE = np.array([e8m0_value(c) for c in range(256)], dtype=np.float64)


def e8m0_decode(codes: np.ndarray) -> np.ndarray:
    return E8M0_TABLE[np.asarray(codes, dtype=np.int64) & 0xFF]


def mx_shared_exponent(absmax: np.ndarray) -> np.ndarray:
    """X = floor(log2(absmax)) - 2, clamped to [-127, 127]; -127 for a zero block.
    floor(log2(a)) comes from frexp (a = m 2^E with 0.5 <= m < 1, so it is E - 1),
    exact for every float."""
    a = np.asarray(absmax, dtype=np.float64)
    _, E = np.frexp(a)
    X = np.where(a > 0, E.astype(np.int64) - 1 - 2, -127)
    return np.clip(X, -127, 127)


def mx_quantize(x: np.ndarray):
    """x [rows, cols] (float32 values, finite) -> (codes u8 [rows, cols/2],
    scales u8 [rows, cols/32]).  Element 2i in the low nibble of byte i."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x32.shape
    assert cols % MX_BLOCK == 0
    blk = x32.astype(np.float64).reshape(rows, cols // MX_BLOCK, MX_BLOCK)
    absmax = np.abs(blk).max(axis=2)
    X = mx_shared_exponent(absmax)                              # [rows, cols/32]
    v = np.abs(blk) / np.ldexp(1.0, X)[..., None]               # exact: a power of two
    mag = e2m1_encode_magnitude(np.minimum(v, 6.0))
    sign = np.signbit(blk).astype(np.uint8) << 3
    code = (mag | sign).astype(np.uint8)
    code = np.where((absmax > 0)[..., None], code, np.uint8(0)).reshape(rows, cols)
    scales = (X + E8M0_BIAS).astype(np.uint8)
    return pack_codes(code), scales


def mx_dequantize(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """E2M1(q) * 2^(scale - 127), float64 (exact)."""
    q = e2m1_decode(unpack_codes(codes))
    s = np.repeat(e8m0_decode(scales), MX_BLOCK, axis=-1)
    return q * s


def mx_grouped_gemm(a_codes, a_scales, b_codes, b_scales, offsets, a_rows=None, a_g=1.0, b_g=None,
                    want_absdot=True):
    """Grouped MXFP4 GEMM: for expert e and permuted row p in
    [offsets[e], offsets[e+1]) with A row r = a_rows[p] (or p),
        y[p, n] = g_a g_b[e] sum_k a^[r, k] b^[e, n, k]
    with a^, b^ the dequantised MX values.  Returns (y float32, absdot) where
    absdot = sum_k |a^ b^| g_a g_b[e], the scale of the error bound.
    a_*: codes [rows_a, K/2], scales [rows_a, K/32]; b_*: codes [E, N, K/2],
    scales [E, N, K/32]; b_g [E] (None: ones)."""
    E, N, K2 = b_codes.shape
    offsets = np.asarray(offsets, dtype=np.int64)
    M = int(offsets[-1])
    y = np.zeros((M, N), dtype=np.float32)
    absdot = np.zeros((M, N), dtype=np.float64) if want_absdot else None
    ga = np.float64(np.float32(a_g))
    gb = np.ones(E, np.float32) if b_g is None else np.asarray(b_g, np.float32)
    for e in range(E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        rows = np.arange(p0, p1) if a_rows is None else np.asarray(a_rows)[p0:p1]
        a_hat = mx_dequantize(a_codes[rows], a_scales[rows])
        b_hat = mx_dequantize(b_codes[e], b_scales[e])
        gab = ga * np.float64(gb[e])
        y[p0:p1] = ((a_hat @ b_hat.T) * gab).astype(np.float32)
        if want_absdot:
            absdot[p0:p1] = (np.abs(a_hat) @ np.abs(b_hat).T) * gab
    return y, absdot


def mx_swiglu_quantize(y1: np.ndarray):
    """h = silu(gate) * up (float64, gate = y1[:, :I], up = y1[:, I:]), rounded to
    float32, then MXFP4.  Returns (codes, scales, h64)."""
    y = np.asarray(y1, dtype=np.float64)
    I = y.shape[1] // 2
    g = y[:, :I]
    with np.errstate(over="ignore"):
        h64 = g / (1.0 + np.exp(-g)) * y[:, I:]
    codes, scales = mx_quantize(h64.astype(np.float32))
    return codes, scales, h64
