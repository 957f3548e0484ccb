"""Pins of the FP8 block-scaled oracle (oracle/fp8.py): the encoder against
torch's float8_e4m3fn cast (nearest-even), a block worked by hand, the block
shapes (1 x 128 for activations, 128 x 128 for weights, a short last row
block), the quantisation error bound and sign symmetry, and the grouped GEMM
against exact rational brute force and numpy's matmul of the dequantised
operands."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import fp8 as P


def test_worked_block_by_hand():
    # absmax 896 -> s = 896 / 448 = 2; then x / 2 rounds to E4M3 (bias 7):
    #   3.0 -> 1.5 = 2^0 * 1.100b: exponent field 7, mantissa 4 -> 0x3C
    #   -100 -> 50 = 2^5 * 1.5625, halfway between mantissas 4 (48) and 5 (52):
    #          ties to even -> 48: sign | exponent 12 | mantissa 4 -> 0xE4
    #   896 -> 448 (the largest finite value, 0x7E); -0.0 -> 0x80
    #   0.001 -> 0.0005, below half the smallest subnormal (2^-10) -> 0x00
    #   0.0039 -> 0.00195, rounds to 1 * 2^-9 (subnormal) -> 0x01
    x = np.zeros((1, 128), np.float32)
    x[0, :6] = [3.0, -100.0, 896.0, -0.0, 0.001, 0.0039]
    codes, scales = P.fp8_quantize(x)
    assert scales.tolist() == [[2.0]]
    assert codes[0, :6].tolist() == [0x3C, 0xE4, 0x7E, 0x80, 0x00, 0x01]
    assert F.e4m3_value(0x3C) == 1.5 and F.e4m3_value(0xE4) == -48.0 and F.e4m3_value(0x7E) == 448.0


def test_encoder_matches_torch_float8_cast():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((64, 512)) * np.exp2(rng.integers(-20, 20, (64, 1)))).astype(np.float32)
    codes, scales = P.fp8_quantize(x)
    s_el = np.repeat(scales, 128, axis=1)
    v = (x / s_el).astype(np.float32)                       # same float32 quotient, with its sign
    lib = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(lib, codes)


@pytest.mark.parametrize("block_rows,rows", [(1, 7), (128, 128), (128, 300)])
def test_block_shapes_and_error_bound(block_rows, rows):
    rng = np.random.default_rng(block_rows + rows)
    x = (rng.standard_normal((rows, 384)) * np.exp2(rng.integers(-8, 8, (rows, 1)))).astype(np.float32)
    x[0, 128:256] = 0.0                                      # a zero block (in a 1 x 128 layout)
    codes, scales = P.fp8_quantize(x, block_rows)
    assert scales.shape == ((rows + block_rows - 1) // block_rows, 3)
    # each scale is its block's absmax / 448 (float32), 1 for a zero block
    for rb in range(scales.shape[0]):
        for cb in range(3):
            blk = np.abs(x[rb * block_rows:(rb + 1) * block_rows, 128 * cb:128 * (cb + 1)])
            want = np.float32(np.float32(blk.max()) / np.float32(448.0)) if blk.max() > 0 else np.float32(1.0)
            assert scales[rb, cb] == want
    deq = P.fp8_dequantize(codes, scales, block_rows)
    s_el = np.repeat(np.repeat(scales.astype(np.float64), block_rows, axis=0)[:rows], 128, axis=1)
    v = np.abs(x.astype(np.float64)) / s_el
    hi = np.clip(np.searchsorted(F.E4M3_POS, v), 1, len(F.E4M3_POS) - 1)
    gap = F.E4M3_POS[hi] - F.E4M3_POS[hi - 1]
    # half a gap of the float32 quotient's neighbourhood, plus the quotient's own rounding
    assert np.all(np.abs(deq - x) <= (0.5 * gap + v * 2.0 ** -23) * s_el * (1 + 1e-9) + 1e-300)
    # sign symmetry
    cn, sn = P.fp8_quantize(-x, block_rows)
    assert np.array_equal(sn, scales) and np.array_equal(cn, codes ^ 0x80)


def _rand_fp8(rng, shape):
    c = rng.integers(0, 256, shape, dtype=np.uint8)
    c[(c & 0x7F) == 0x7F] = 0x7E                              # no NaN codes
    return c


def test_fp8_gemm_equals_exact_rational():
    rng = np.random.default_rng(3)
    E, N, K = 2, 130, 256                                      # two 128-row weight blocks, the second short
    counts = [2, 3]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    ac = _rand_fp8(rng, (6, K))
    as_ = rng.uniform(0.01, 2, (6, K // 128)).astype(np.float32)
    bc = _rand_fp8(rng, (E, N, K))
    bs = rng.uniform(0.01, 2, (E, 2, K // 128)).astype(np.float32)
    a_rows = rng.permutation(6)[:5].astype(np.int32)
    y, absdot = P.fp8_grouped_gemm(ac, as_, bc, bs, offsets, a_rows=a_rows)
    # brute force from the definition on a column subset that spans both
    # weight row blocks (128 x 128 scales): exact rationals, nested loops
    cols = [0, 1, 127, 128, 129]
    for p in range(5):
        e = 0 if p < counts[0] else 1
        r = int(a_rows[p])
        for n in cols:
            acc, accm = Fraction(0), Fraction(0)
            for kb in range(K // 128):
                part, partm = Fraction(0), Fraction(0)
                for i in range(128):
                    k = 128 * kb + i
                    prod = Fraction(F.e4m3_value(int(ac[r, k]))) * Fraction(F.e4m3_value(int(bc[e, n, k])))
                    part += prod
                    partm += abs(prod)
                sc = Fraction(float(as_[r, kb])) * Fraction(float(bs[e, n // 128, kb]))
                acc += sc * part
                accm += sc * partm
            assert abs(float(y[p, n]) - float(acc)) <= abs(float(acc)) * 2 ** -23 + 1e-300, (p, n)
            assert abs(Fraction(float(absdot[p, n])) - accm) <= accm * Fraction(1, 2 ** 50)


def test_fp8_gemm_single_block_terms_correctly_rounded():
    # one nonzero 128-block, arbitrary float32 scales: each output is one exact
    # block term, so the oracle must return its float32 rounding (up to a
    # double rounding through float64) and exactly 0 where the code products
    # cancel.  Rows 0-1 against weight rows 0-1 cancel exactly with terms of
    # different size: 1.875 * 1.875 - 1.75 * 2 - 0.125 * 0.125 = 0, where the
    # first term times the scales needs more than float64's 53 bits
    rng = np.random.default_rng(6)
    M, N, K = 6, 20, 384
    ac = np.zeros((M, K), np.uint8)
    bc = np.zeros((1, N, K), np.uint8)
    ac[:, 128:256] = _rand_fp8(rng, (M, 128))
    bc[0, :, 128:256] = _rand_fp8(rng, (N, 128))
    ac[0:2, 128:256] = 0
    bc[0, 0:2, 128:256] = 0
    ac[0:2, 128:131] = [0x3F, 0x3E, 0x20]                       # 1.875, 1.75, 0.125
    bc[0, 0:2, 128:131] = [0x3F, 0xC0, 0xA0]                    # 1.875, -2, -0.125
    as_ = rng.uniform(0.1, 10, (M, K // 128)).astype(np.float32)
    bs = rng.uniform(0.1, 10, (1, 1, K // 128)).astype(np.float32)
    y, _ = P.fp8_grouped_gemm(ac, as_, bc, bs, np.array([0, M]))
    for p in range(M):
        for n in range(N):
            part = sum(Fraction(F.e4m3_value(int(ac[p, k]))) * Fraction(F.e4m3_value(int(bc[0, n, k])))
                       for k in range(128, 256))
            exact = part * Fraction(float(as_[p, 1])) * Fraction(float(bs[0, 0, 1]))
            if p < 2 and n < 2:
                assert exact == 0 and y[p, n] == 0
            assert abs(Fraction(float(y[p, n])) - exact) <= abs(exact) * Fraction(1, 2 ** 24) * (1 + Fraction(1, 2 ** 27))


def test_fp8_gemm_dense_is_matmul_and_approximates_full_precision():
    rng = np.random.default_rng(4)
    A = rng.standard_normal((20, 256)).astype(np.float32)
    B = (rng.standard_normal((140, 256)) * 0.05).astype(np.float32)
    ac, as_ = P.fp8_quantize(A, 1)
    bc, bs = P.fp8_quantize(B, 128)
    y, _ = P.fp8_grouped_gemm(ac, as_, bc[None], bs[None], np.array([0, 20]))
    ref = (torch.from_numpy(P.fp8_dequantize(ac, as_, 1)) @ torch.from_numpy(P.fp8_dequantize(bc, bs, 128)).T).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-12)
    full = A.astype(np.float64) @ B.astype(np.float64).T
    assert np.linalg.norm(y - full) / np.linalg.norm(full) < 0.05


def test_fp8_swiglu_quantize_matches_parts():
    # silu against scipy's logistic function, the product, then the 1 x 128
    # quantiser on the float32 rounding of h
    from scipy.special import expit
    rng = np.random.default_rng(12)
    y1 = (rng.standard_normal((5, 512)) * 4).astype(np.float32)
    codes, scales, h64 = P.fp8_swiglu_quantize(y1)
    g, u = y1[:, :256].astype(np.float64), y1[:, 256:].astype(np.float64)
    np.testing.assert_allclose(h64, g * expit(g) * u, rtol=1e-14, atol=1e-300)
    c2, s2 = P.fp8_quantize(h64.astype(np.float32), 1)
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    assert codes.shape == (5, 256) and scales.shape == (5, 2)
