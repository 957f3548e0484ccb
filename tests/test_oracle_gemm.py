"""Pins of the oracle's grouped GEMM: exact rational brute force, the blockwise
definition, special cases with an order-independent float32 result, and the
dense single-expert case against numpy matmul."""
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F
from oracle.moe import grouped_gemm, grouped_gemm_blockwise
from oracle.quant import dequantize_unscaled, quantize, unpack_codes


def _rand_operands(rng, E, N, K, rows_a, scale_lo=0x20, scale_hi=0x50):
    a_codes = rng.integers(0, 256, (rows_a, K // 2), dtype=np.uint8)
    a_scales = rng.integers(scale_lo, scale_hi, (rows_a, K // 16), dtype=np.uint8)
    b_codes = rng.integers(0, 256, (E, N, K // 2), dtype=np.uint8)
    b_scales = rng.integers(scale_lo, scale_hi, (E, N, K // 16), dtype=np.uint8)
    return a_codes, a_scales, b_codes, b_scales


def _frac_e2m1(c):
    return Fraction(F.e2m1_value(int(c)))


def _frac_e4m3(c):
    return Fraction(F.e4m3_value(int(c)))


def _exact(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets, a_rows, want_abs=False):
    """Exact rational value of every output, from the definition (nested loops).
    With want_abs, also the exact sum_k |a^_k b^_k| g_a g_b[e] of every output
    (the scale of the error bound), from the same loops with each product's
    magnitude."""
    E, N, K2 = b_codes.shape
    K = 2 * K2
    M = int(offsets[-1])
    out = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    ua = unpack_codes(a_codes)
    ub = unpack_codes(b_codes)
    for e in range(E):
        for p in range(int(offsets[e]), int(offsets[e + 1])):
            r = int(a_rows[p]) if a_rows is not None else p
            for n in range(N):
                acc = Fraction(0)
                acc_abs = Fraction(0)
                for kb in range(K // 16):
                    part = Fraction(0)
                    part_abs = Fraction(0)
                    for i in range(16):
                        kk = 16 * kb + i
                        prod = _frac_e2m1(ua[r, kk]) * _frac_e2m1(ub[e, n, kk])
                        part += prod
                        part_abs += abs(prod)
                    s = _frac_e4m3(a_scales[r, kb]) * _frac_e4m3(b_scales[e, n, kb])
                    acc += s * part
                    acc_abs += s * part_abs
                g = Fraction(float(np.float32(a_g))) * Fraction(float(np.float32(b_g[e])))
                out[p][n] = acc * g
                mag[p][n] = acc_abs * g
    return (out, mag) if want_abs else out


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_grouped_gemm_equals_exact_rational(seed):
    rng = np.random.default_rng(seed)
    E, N, K = 3, 5, 64                      # N != M != K so a transposed operand fails
    counts = [2, 0, 4]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    rows_a = 7
    a_codes, a_scales, b_codes, b_scales = _rand_operands(rng, E, N, K, rows_a)
    a_rows = rng.permutation(rows_a)[: offsets[-1]].astype(np.int32)
    a_g = np.float32(0.37)
    b_g = np.array([1.5, 0.25, 0.0078125 * 3], np.float32)
    y, absdot = grouped_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets, a_rows=a_rows)
    ex, ex_abs = _exact(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets, a_rows, want_abs=True)
    for p in range(offsets[-1]):
        for n in range(N):
            want = np.float32(float(ex[p][n]))          # correctly rounded
            got = y[p, n]
            assert abs(float(got) - float(ex[p][n])) <= abs(float(want)) * 2 ** -23 + 1e-30, (p, n)
            # the tolerance scale sum|a^ b^| is pinned from both sides: exact
            # up to float64 rounding of the per-tensor scale product
            assert abs(Fraction(float(absdot[p, n])) - ex_abs[p][n]) <= ex_abs[p][n] * Fraction(1, 2 ** 50), (p, n)
    assert np.all(absdot >= np.abs(y) * (1 - 1e-6))


def test_blockwise_definition_matches_matmul_form():
    rng = np.random.default_rng(5)
    E, N, K = 2, 6, 96
    offsets = np.array([0, 3, 8])
    a_codes, a_scales, b_codes, b_scales = _rand_operands(rng, E, N, K, 8, 0x01, 0x7E)
    a_g, b_g = np.float32(0.01), np.array([2.0, 0.3], np.float32)
    y, _ = grouped_gemm(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets)
    yb = grouped_gemm_blockwise(a_codes, a_scales, a_g, b_codes, b_scales, b_g, offsets)
    np.testing.assert_allclose(y.astype(np.float64), yb, rtol=2 ** -23, atol=1e-30)


def test_constant_block_scales_are_order_independent_in_float32():
    # With one scale for all blocks and g = 1 every partial sum is an integer
    # multiple m of 0.25*s_a*s_b = 5/32 with |m| <= 4096*144 < 2^24/5, so float32
    # accumulation in ANY order is exact: a reversed float32 loop must equal the
    # oracle bit for bit.
    rng = np.random.default_rng(11)
    M, N, K = 4, 3, 4096
    a_codes = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    b_codes = rng.integers(0, 256, (1, N, K // 2), dtype=np.uint8)
    a_scales = np.full((M, K // 16), 0x3A, np.uint8)       # 1.25
    b_scales = np.full((1, N, K // 16), 0x30, np.uint8)    # 0.5
    y, _ = grouped_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(1, np.float32),
                        np.array([0, M]))
    qa = F.e2m1_decode(unpack_codes(a_codes)).astype(np.float32)
    qb = F.e2m1_decode(unpack_codes(b_codes[0])).astype(np.float32)
    for m in range(M):
        for n in range(N):
            acc = np.float32(0)
            for kk in range(K - 1, -1, -1):
                acc = np.float32(acc + np.float32(qa[m, kk] * np.float32(1.25)) * np.float32(qb[n, kk] * np.float32(0.5)))
            assert acc == y[m, n]


def test_single_block_k16_exact():
    rng = np.random.default_rng(12)
    a_codes, a_scales, b_codes, b_scales = _rand_operands(rng, 1, 4, 16, 3, 0x01, 0x7E)
    y, _ = grouped_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(1, np.float32),
                        np.array([0, 3]))
    for m in range(3):
        for n in range(4):
            s = sum(F.e2m1_value(int(unpack_codes(a_codes)[m, i])) *
                    F.e2m1_value(int(unpack_codes(b_codes)[0, n, i])) for i in range(16))
            want = s * F.e4m3_value(int(a_scales[m, 0])) * F.e4m3_value(int(b_scales[0, n, 0]))
            assert float(y[m, n]) == want         # exact in float32 (<= 20 significant bits)


def test_dense_single_expert_is_matmul_of_dequantised_operands():
    # E = 1, identity rows: the grouped GEMM is a plain GEMM of the dequantised
    # matrices (torch.matmul in float64 as the independent library routine).
    import torch
    rng = np.random.default_rng(13)
    A = rng.standard_normal((24, 160)).astype(np.float32)
    B = rng.standard_normal((40, 160)).astype(np.float32) * 0.02
    ac, as_, ag = quantize(A)
    bc, bs, bg = quantize(B)
    y, _ = grouped_gemm(ac, as_, ag, bc[None], bs[None], np.array([bg]), np.array([0, 24]))
    Ah = torch.from_numpy(dequantize_unscaled(ac, as_) * float(ag))
    Bh = torch.from_numpy(dequantize_unscaled(bc, bs) * float(bg))
    ref = (Ah @ Bh.T).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-9)
    # and it approximates the unquantised product within NVFP4's resolution
    full = A.astype(np.float64) @ B.astype(np.float64).T
    rel = np.linalg.norm(y - full) / np.linalg.norm(full)
    assert rel < 0.2


def test_empty_experts_and_row_gather():
    rng = np.random.default_rng(14)
    a_codes, a_scales, b_codes, b_scales = _rand_operands(rng, 4, 2, 32, 5)
    offsets = np.array([0, 0, 2, 2, 5])
    a_rows = np.array([4, 0, 1, 3, 2], np.int32)
    y, _ = grouped_gemm(a_codes, a_scales, 1.0, b_codes, b_scales, np.ones(4, np.float32), offsets, a_rows=a_rows)
    y_id, _ = grouped_gemm(a_codes[a_rows], a_scales[a_rows], 1.0, b_codes, b_scales,
                           np.ones(4, np.float32), offsets)
    assert np.array_equal(y, y_id)
    # rows of expert 1 use expert 1's weights only
    y1 = dequantize_unscaled(a_codes[[4, 0]], a_scales[[4, 0]]) @ dequantize_unscaled(b_codes[1], b_scales[1]).T
    np.testing.assert_allclose(y[:2], y1, rtol=1e-7)
