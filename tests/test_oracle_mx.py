"""Pins of the MXFP4 oracle (oracle/mx.py): the E8M0 scale against its closed
form and torch's float8_e8m0fnu, the shared exponent at powers of two and
around them, a block worked by hand, quantiser invariants (scale choice, error
bound, idempotence, sign symmetry, zero blocks), and the grouped GEMM against
exact rational brute force, an order-independent special case and numpy's
matmul of the dequantised operands."""
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import mx as MX
from oracle.quant import unpack_codes


# ------------------------------------------------------------------ E8M0
def test_e8m0_closed_form_and_library():
    for c in range(255):
        assert MX.e8m0_value(c) == 2.0 ** (c - 127)
    assert np.isnan(MX.e8m0_value(255))
    lib = torch.arange(256, dtype=torch.int32).to(torch.uint8).view(torch.float8_e8m0fnu).to(torch.float64).numpy()
    ours = MX.E8M0_TABLE
    assert np.array_equal(np.isnan(lib), np.isnan(ours))
    ok = ~np.isnan(ours)
    assert np.array_equal(lib[ok], ours[ok])


def test_shared_exponent_at_and_around_powers_of_two():
    for k in range(-120, 120, 7):
        p = 2.0 ** k
        assert MX.mx_shared_exponent(np.array([p]))[0] == k - 2                 # floor(log2(2^k)) = k
        assert MX.mx_shared_exponent(np.array([np.nextafter(p, 0)]))[0] == k - 3
        assert MX.mx_shared_exponent(np.array([p * 1.999]))[0] == k - 2
    assert MX.mx_shared_exponent(np.array([0.0]))[0] == -127
    assert MX.mx_shared_exponent(np.array([2.0 ** -140]))[0] == -127           # clamped below
    assert MX.mx_shared_exponent(np.array([3.0e38]))[0] == 125


# ------------------------------------------------------------------ quantiser
def test_worked_block_by_hand():
    # absmax 7.9: floor(log2 7.9) = 2, X = 0, scale code 127; then each value
    # / 2^0 rounds to the E2M1 grid: 1.0 -> 1 (code 2), -0.3 -> 0.5 with sign
    # (code 9), 5.0 is a tie between 4 (code 6, even) and 6 (code 7) -> 4,
    # 7.9 saturates to 6 (code 7), 0.25 is a tie between 0 and 0.5 -> 0 (code 0),
    # -0.0 keeps its sign (code 8), 2.6 -> 3 (code 5), 1.25 ties to 1 (code 2)
    x = np.zeros((1, 32), np.float32)
    x[0, :8] = [1.0, -0.3, 5.0, 7.9, 0.25, -0.0, 2.6, 1.25]
    codes, scales = MX.mx_quantize(x)
    assert scales.tolist() == [[127]]
    assert unpack_codes(codes)[0, :8].tolist() == [2, 9, 6, 7, 0, 8, 5, 2]
    # the same block scaled by 2^-10 only moves the scale
    codes2, scales2 = MX.mx_quantize(x * np.float32(2.0 ** -10))
    assert scales2.tolist() == [[117]] and np.array_equal(codes2, codes)


def _random_blocks(rng, rows, cols):
    x = rng.standard_normal((rows, cols)).astype(np.float32)
    x *= np.exp2(rng.integers(-30, 30, (rows, cols // 32))).repeat(32, axis=1).astype(np.float32)
    x[0, :32] = -0.0                                    # a zero block (negative zeros)
    x[1, 5] = -0.0
    return x


def test_quantiser_invariants():
    rng = np.random.default_rng(3)
    x = _random_blocks(rng, 40, 256)
    codes, scales = MX.mx_quantize(x)
    q = unpack_codes(codes)
    blk = np.abs(x.astype(np.float64)).reshape(40, 8, 32)
    amax = blk.max(axis=2)
    X = scales.astype(np.int64) - 127
    nz = amax > 0
    # the block's largest value lands in [4, 8) after the scale: code 4 or 6
    qmax = (q & 7).reshape(40, 8, 32)[np.arange(40)[:, None], np.arange(8)[None], blk.argmax(axis=2)]
    assert np.all(qmax[nz] >= 6)                                     # E2M1 codes 6, 7 = 4, 6
    assert np.all((amax[nz] / np.exp2(X[nz]) >= 4) & (amax[nz] / np.exp2(X[nz]) < 8))
    # zero block: scale code 0, codes 0
    assert scales[0, 0] == 0 and not q[0, :32].any()
    # error bound: half the E2M1 gap at the value, or the saturation excess
    deq = MX.mx_dequantize(codes, scales)
    s = np.exp2(X).repeat(32, axis=1)
    v = np.abs(x.astype(np.float64)) / s
    hi = np.clip(np.searchsorted(F.E2M1_MAGNITUDES, v), 1, 7)
    gap = F.E2M1_MAGNITUDES[hi] - F.E2M1_MAGNITUDES[hi - 1]
    bound = np.where(v > 6, np.abs(x) - 6 * s, 0.5 * gap * s)
    assert np.all(np.abs(deq - x) <= bound * (1 + 1e-12) + 1e-300)
    # idempotence: the dequantised tensor quantises to itself
    c2, s2 = MX.mx_quantize(deq.astype(np.float32))
    assert np.array_equal(c2, codes) and np.array_equal(s2, scales)
    # sign symmetry (outside zero blocks): q(-x) = q(x) ^ 8
    cn, sn = MX.mx_quantize(-x)
    qn = unpack_codes(cn)
    assert np.array_equal(sn, scales)
    assert np.array_equal(qn[1:], q[1:] ^ 8)


def test_quantiser_brute_force_every_bf16_in_a_block():
    # every positive bf16 value below the block's absmax, one per block, with
    # the block's absmax fixed at 4.0 (X = 0): the code must be the nearest
    # E2M1 value, ties to the even code (checked against the grid directly)
    vals = torch.arange(0, 0x4080, dtype=torch.int32).to(torch.int16).view(torch.bfloat16).float().numpy()
    vals = vals[np.isfinite(vals) & (vals >= 0) & (vals < 4.0)]
    x = np.zeros((len(vals), 32), np.float32)
    x[:, 0] = 4.0
    x[:, 1] = vals
    codes, scales = MX.mx_quantize(x)
    assert np.all(scales == 127)
    got = (unpack_codes(codes)[:, 1] & 7).astype(np.int64)
    grid = F.E2M1_MAGNITUDES
    for v, g in zip(vals.astype(np.float64), got):
        d = np.abs(grid - v)
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert g == want, (v, g, want)


# ------------------------------------------------------------------ GEMM
def _rand_mx(rng, shape_rows, K, lo=120, hi=134):
    codes = rng.integers(0, 256, shape_rows + (K // 2,), dtype=np.uint8)
    scales = rng.integers(lo, hi, shape_rows + (K // 32,), dtype=np.uint8)
    return codes, scales


def _exact(ac, as_, bc, bs, offsets, a_rows, ga, gb):
    E, N, K2 = bc.shape
    K = 2 * K2
    M = int(offsets[-1])
    ua, ub = unpack_codes(ac), unpack_codes(bc)
    out = [[None] * N for _ in range(M)]
    mag = [[None] * N for _ in range(M)]
    for e in range(E):
        for p in range(int(offsets[e]), int(offsets[e + 1])):
            r = int(a_rows[p]) if a_rows is not None else p
            for n in range(N):
                acc = Fraction(0)
                acc_abs = Fraction(0)
                for kb in range(K // 32):
                    part = Fraction(0)
                    part_abs = Fraction(0)
                    for i in range(32):
                        kk = 32 * kb + i
                        prod = Fraction(F.e2m1_value(int(ua[r, kk]))) * Fraction(F.e2m1_value(int(ub[e, n, kk])))
                        part += prod
                        part_abs += abs(prod)
                    s = Fraction(2) ** (int(as_[r, kb]) - 127) * Fraction(2) ** (int(bs[e, n, kb]) - 127)
                    acc += s * part
                    acc_abs += s * part_abs
                g = Fraction(float(np.float32(ga))) * Fraction(float(np.float32(gb[e])))
                out[p][n] = acc * g
                mag[p][n] = acc_abs * g
    return out, mag


@pytest.mark.parametrize("seed", [0, 1])
def test_mx_gemm_equals_exact_rational(seed):
    rng = np.random.default_rng(40 + seed)
    E, N, K = 3, 5, 96
    counts = [2, 0, 3]
    offsets = np.concatenate([[0], np.cumsum(counts)])
    ac, as_ = _rand_mx(rng, (7,), K)
    bc, bs = _rand_mx(rng, (E, N), K)
    a_rows = rng.permutation(7)[: offsets[-1]].astype(np.int32)
    ga, gb = np.float32(0.75), np.array([1.5, 0.25, 3.0], np.float32)
    y, absdot = MX.mx_grouped_gemm(ac, as_, bc, bs, offsets, a_rows=a_rows, a_g=ga, b_g=gb)
    ex, ex_abs = _exact(ac, as_, bc, bs, offsets, a_rows, ga, gb)
    for p in range(offsets[-1]):
        for n in range(N):
            want = float(ex[p][n])
            assert abs(float(y[p, n]) - want) <= abs(want) * 2 ** -23 + 1e-300, (p, n)
            assert abs(Fraction(float(absdot[p, n])) - ex_abs[p][n]) <= ex_abs[p][n] * Fraction(1, 2 ** 50)


def test_mx_gemm_constant_scales_order_independent():
    # one scale for every block: every partial sum is a multiple of
    # 0.25 * 2^(Xa+Xb) far below 2^24 of them, so float32 in any order is exact
    rng = np.random.default_rng(9)
    M, N, K = 3, 4, 2048
    ac = rng.integers(0, 256, (M, K // 2), dtype=np.uint8)
    bc = rng.integers(0, 256, (1, N, K // 2), dtype=np.uint8)
    as_ = np.full((M, K // 32), 125, np.uint8)
    bs = np.full((1, N, K // 32), 130, np.uint8)
    y, _ = MX.mx_grouped_gemm(ac, as_, bc, bs, np.array([0, M]))
    qa = F.e2m1_decode(unpack_codes(ac)).astype(np.float32) * np.float32(0.25)
    qb = F.e2m1_decode(unpack_codes(bc[0])).astype(np.float32) * np.float32(8.0)
    for m in range(M):
        for n in range(N):
            acc = np.float32(0)
            for kk in range(K - 1, -1, -1):
                acc = np.float32(acc + qa[m, kk] * qb[n, kk])
            assert acc == y[m, n]


def test_mx_gemm_dense_single_expert_is_matmul():
    rng = np.random.default_rng(10)
    A = rng.standard_normal((12, 128)).astype(np.float32)
    B = (rng.standard_normal((20, 128)) * 0.05).astype(np.float32)
    ac, as_ = MX.mx_quantize(A)
    bc, bs = MX.mx_quantize(B)
    y, _ = MX.mx_grouped_gemm(ac, as_, bc[None], bs[None], np.array([0, 12]))
    ref = (torch.from_numpy(MX.mx_dequantize(ac, as_)) @ torch.from_numpy(MX.mx_dequantize(bc, bs)).T).numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-12)
    full = A.astype(np.float64) @ B.astype(np.float64).T
    assert np.linalg.norm(y - full) / np.linalg.norm(full) < 0.25


def test_mx_swiglu_quantize_matches_parts():
    rng = np.random.default_rng(11)
    y1 = (rng.standard_normal((6, 128)) * 3).astype(np.float32)
    codes, scales, h64 = MX.mx_swiglu_quantize(y1)
    g, u = y1[:, :64].astype(np.float64), y1[:, 64:].astype(np.float64)
    np.testing.assert_allclose(h64, g / (1 + np.exp(-g)) * u, rtol=1e-15)
    c2, s2 = MX.mx_quantize(h64.astype(np.float32))
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
