"""FP8 block-scaled operands and their grouped GEMM (CPU oracle; test
infrastructure).

The pages name an FP8 grouped GEMM next to the FP4 ones ("From Empirical
Limits to Research-Driven Optimization: The SM120 FP4 Kernel Research
Campaign", section "Sections 2-4: Framework and Community Landscape") and an
FP8 collective with blockwise scaling among the CUTLASS sources they search
("The Critical Search: Uncovering SM120 CUTLASS Collective Implementations",
section "Output Knowledge Created").  They give no block shape or quantiser;
this module takes the plainest blockwise reading:

* element     FP8 E4M3 (OCP E4M3FN: bias 7, max 448, no infinities), the byte
              holds the sign in bit 7
* blocks      128 consecutive values along the reduction axis; activations
              have one scale per row and block (1 x 128), weights one per
              128 x 128 tile (128 output rows x 128 values of K)
* scale       float32 s = absmax_block / 448 (float32 division); s = 1 for an
              all-zero block
* encode      q = E4M3 nearest-even of |x| / s (float32 division, correctly
              rounded), saturating at 448, sign copied from x
* value       E4M3(q) * s

GEMM, per expert:
    y[p, n] = sum_kb sa[r, kb] * sb[e, n // 128, kb] * sum_{k in kb} qa[r, k] qb[e, n, k]
computed as written: each block's sum of code products is exact in float64
(a product of two E4M3 values has at most 8 significant bits and lies in
[2^-18, 2^17], so 128 of them sum exactly), the product of the two float32
scales is exact (48 bits), each scaled block term is rounded once, the terms
sum in float64 (numpy matmul as the summation primitive for the block sums)
and the result is rounded to float32 once.  (A product of two dequantised
values, E4M3 * float32 scale on each side, can need 56 bits and would not be
exact in float64.)
"""
from __future__ import annotations

import numpy as np

from .formats import E4M3_MAX, e4m3_decode, e4m3_encode_satfinite

FP8_BLOCK = 128
F32_448 = np.float32(448.0)


def fp8_block_scales(x32: np.ndarray, block_rows: int) -> np.ndarray:
    """float32 scale of each (block_rows x 128) block: absmax / 448, 1 for a zero block.
    A last row block may be shorter than block_rows."""
    rows, cols = x32.shape
    assert cols % FP8_BLOCK == 0
    rb = (rows + block_rows - 1) // block_rows
    a = np.abs(x32.astype(np.float32))
    pad = rb * block_rows - rows
    if pad:
        a = np.concatenate([a, np.zeros((pad, cols), np.float32)])
    amax = a.reshape(rb, block_rows, cols // FP8_BLOCK, FP8_BLOCK).max(axis=(1, 3)).astype(np.float32)
    s = (amax / F32_448).astype(np.float32)
    return np.where(amax > 0, s, np.float32(1.0)).astype(np.float32)


def fp8_quantize(x: np.ndarray, block_rows: int = 1):
    """x [rows, cols] (float32 values, finite) -> (codes u8 [rows, cols] (E4M3
    bytes), scales f32 [ceil(rows/block_rows), cols/128])."""
    x32 = np.ascontiguousarray(x, dtype=np.float32)
    rows, cols = x32.shape
    s = fp8_block_scales(x32, block_rows)
    s_el = np.repeat(np.repeat(s, block_rows, axis=0)[:rows], FP8_BLOCK, axis=1)
    v = (np.abs(x32) / s_el).astype(np.float32)                    # float32 division
    mag = e4m3_encode_satfinite(np.minimum(v.astype(np.float64), E4M3_MAX))
    sign = (np.signbit(x32).astype(np.uint8) << 7)
    return (mag | sign).astype(np.uint8), s


def fp8_row_scales(scales: np.ndarray, block_rows: int, rows: int) -> np.ndarray:
    """The scale of each row and 128-value block: [..., rows, cols/128] (row i
    takes its row block i // block_rows), float64."""
    return np.repeat(np.asarray(scales, np.float64), block_rows, axis=-2)[..., :rows, :]


def fp8_dequantize(codes: np.ndarray, scales: np.ndarray, block_rows: int = 1) -> np.ndarray:
    """E4M3(q) * s, float64 (exact)."""
    codes = np.asarray(codes)
    s = np.repeat(fp8_row_scales(scales, block_rows, codes.shape[-2]), FP8_BLOCK, axis=-1)
    return e4m3_decode(codes) * s


def fp8_grouped_gemm(a_codes, a_scales, b_codes, b_scales, offsets, a_rows=None, want_absdot=True):
    """Grouped FP8 GEMM.  a_codes [rows_a, K], a_scales [rows_a, K/128] (1 x 128
    blocks); b_codes [E, N, K], b_scales [E, ceil(N/128), K/128] (128 x 128
    blocks).  Rows p in [offsets[e], offsets[e+1]) use expert e and A row
    a_rows[p] (or p).  Returns (y float32 [M, N], absdot = sum_k |a^ b^|)."""
    E, N, K = b_codes.shape
    nkb = K // FP8_BLOCK
    offsets = np.asarray(offsets, dtype=np.int64)
    M = int(offsets[-1])
    y = np.zeros((M, N), dtype=np.float32)
    absdot = np.zeros((M, N), dtype=np.float64) if want_absdot else None
    for e in range(E):
        p0, p1 = int(offsets[e]), int(offsets[e + 1])
        if p1 == p0:
            continue
        rows = np.arange(p0, p1) if a_rows is None else np.asarray(a_rows)[p0:p1]
        qa = e4m3_decode(a_codes[rows])                                   # float64, exact
        qb = e4m3_decode(b_codes[e])
        sa = fp8_row_scales(np.asarray(a_scales)[rows], 1, len(rows))     # [m, nkb]
        sb = fp8_row_scales(b_scales[e], FP8_BLOCK, N)                     # [N, nkb]
        acc = np.zeros((p1 - p0, N))
        accm = np.zeros((p1 - p0, N)) if want_absdot else None
        for kb in range(nkb):
            blk = slice(kb * FP8_BLOCK, (kb + 1) * FP8_BLOCK)
            s = sa[:, kb:kb + 1] * sb[None, :, kb]                         # exact: 24 x 24 bits
            acc += (qa[:, blk] @ qb[:, blk].T) * s                         # exact block sum, one rounding
            if want_absdot:
                accm += (np.abs(qa[:, blk]) @ np.abs(qb[:, blk]).T) * s
        y[p0:p1] = acc.astype(np.float32)
        if want_absdot:
            absdot[p0:p1] = accm
    return y, absdot


def fp8_swiglu_quantize(y1: np.ndarray):
    """h = silu(gate) * up (float64; gate = y1[:, :I], up = y1[:, I:]), rounded
    to float32, then FP8 with 1 x 128 blocks.  Returns (codes, scales, h64)."""
    y = np.asarray(y1, dtype=np.float64)
    I = y.shape[1] // 2
    g = y[:, :I]
    with np.errstate(over="ignore"):
        h64 = g / (1.0 + np.exp(-g)) * y[:, I:]
    codes, scales = fp8_quantize(h64.astype(np.float32), 1)
    return codes, scales, h64
