"""Pins of the oracle's NVFP4 quantiser: a worked example written by hand,
invariants that hold for any correct nearest-even quantiser, and brute force."""
import numpy as np
import pytest

from oracle import formats as F
from oracle.quant import (dequantize, dequantize_unscaled, global_scale, pack_codes,
                          quantize, unpack_codes)


def test_worked_example_by_hand():
    # One row of 32 values with amax 2688, so g = 2688/2688 = 1 exactly.
    # Block 0 has absmax 6 -> t = (6/6)/1 = 1 -> scale code 0x38 (1.0), so its
    # codes are the E2M1 codes of the values themselves.
    # Block 1 has absmax 2688 -> t = 448 -> scale 0x7E (448); 2688/448 = 6 -> code 7,
    # -896/448 = -2 -> code 0xC, 100/448 = 0.223 -> code 0 (below .25).
    b0 = [1, -2, 0.5, 6, 0, -0.5, 3, -4, 1.5, 2, -6, 4, -1, 0.25, 0.75, -1.25]
    b1 = [2688, -896, 100] + [0] * 13
    x = np.array([b0 + b1], dtype=np.float32)
    codes, scales, g = quantize(x)
    assert g == np.float32(1.0)
    assert scales.tolist() == [[0x38, 0x7E]]
    # element codes of block 0: 1->2, -2->0xC, .5->1, 6->7, 0->0, -.5->9, 3->5,
    # -4->0xE, 1.5->3, 2->4, -6->0xF, 4->6, -1->0xA, .25->0 (tie->even), .75->2
    # (tie->even), -1.25->0xA (tie->even, 1.0)
    want0 = [2, 0xC, 1, 7, 0, 9, 5, 0xE, 3, 4, 0xF, 6, 0xA, 0, 2, 0xA]
    want1 = [7, 0xC, 0] + [0] * 13
    want = want0 + want1
    packed = [want[2 * i] | (want[2 * i + 1] << 4) for i in range(16)]
    assert codes.tolist() == [packed]
    assert codes[0, 0] == 0xC2                      # low nibble = element 0


def test_zero_tensor():
    codes, scales, g = quantize(np.zeros((3, 64), np.float32))
    assert g == 1.0 and not scales.any() and not codes.any()


def test_zero_block_gives_zero_codes_including_negative_zero():
    x = np.zeros((1, 32), np.float32)
    x[0, 16:] = np.linspace(-3, 3, 16)
    x[0, 3] = -0.0
    codes, scales, g = quantize(x)
    assert scales[0, 0] == 0 and not unpack_codes(codes)[0, :16].any()


def test_global_scale_is_float32_amax_over_2688():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 48)).astype(np.float32)
    amax = np.float32(np.abs(x).max())
    assert global_scale(x) == np.float32(amax / np.float32(2688))


def _rand(shape, seed, kind):
    rng = np.random.default_rng(seed)
    if kind == "normal":
        return rng.standard_normal(shape).astype(np.float32)
    if kind == "heavy":
        return (rng.standard_normal(shape) * np.exp(rng.uniform(-6, 6, shape))).astype(np.float32)
    if kind == "small":
        return (rng.standard_normal(shape) * 0.02).astype(np.float32)
    raise ValueError(kind)


@pytest.mark.parametrize("kind", ["normal", "heavy", "small"])
def test_sign_symmetry(kind):
    x = _rand((16, 128), 1, kind)
    c1, s1, g1 = quantize(x)
    c2, s2, g2 = quantize(-x)
    assert g1 == g2 and np.array_equal(s1, s2)
    u1, u2 = unpack_codes(c1), unpack_codes(c2)
    nz = np.repeat(s1 != 0, 16, axis=1)
    assert np.array_equal(u2[nz], u1[nz] ^ 0x8)


@pytest.mark.parametrize("kind", ["normal", "heavy", "small"])
def test_dequantize_quantize_is_idempotent(kind):
    x = _rand((16, 256), 2, kind)
    c, s, g = quantize(x)
    xh = dequantize(c, s, g).astype(np.float32)
    c2, s2, g2 = quantize(xh, g=g)
    xh2 = dequantize(c2, s2, g2).astype(np.float32)
    assert np.array_equal(xh, xh2)


@pytest.mark.parametrize("kind", ["normal", "heavy"])
def test_requantise_exact_on_blocks_holding_a_six(kind):
    # A block whose largest code is +-6 re-derives the same scale from its own
    # dequantised values (absmax^ = 6 s g -> t = s exactly), hence the same codes.
    x = _rand((32, 256), 3, kind)
    c, s, g = quantize(x)
    u = unpack_codes(c)
    has6 = ((u & 7) == 7).reshape(32, 16, 16).any(axis=2)
    xh = dequantize(c, s, g).astype(np.float32)
    c2, s2, _ = quantize(xh, g=g)
    u2 = unpack_codes(c2)
    assert has6.sum() > 100
    assert np.array_equal(s2[has6], s[has6])
    blk = np.repeat(has6, 16, axis=1)
    assert np.array_equal(u2[blk], u[blk])


@pytest.mark.parametrize("kind", ["normal", "heavy", "small"])
def test_error_bound(kind):
    # |x - x^| <= half the gap between the two grid points around x/(s g), times
    # s g (a tiny allowance for the float32 rounding of x/(s g)); beyond 6 it
    # saturates to 6 s g.
    x = _rand((16, 512), 4, kind)
    c, s, g = quantize(x)
    sv = np.repeat(F.e4m3_decode(s), 16, axis=1) * np.float64(g)
    xh = dequantize(c, s, g)
    v = np.abs(x.astype(np.float64)) / np.where(sv > 0, sv, 1)
    grid = F.E2M1_MAGNITUDES
    hi = np.clip(np.searchsorted(grid, v), 1, 7)
    gap = grid[hi] - grid[hi - 1]
    ok_inside = np.abs(x - xh) <= (0.5 * gap * (1 + 1e-6)) * sv
    sat = v > 6
    assert np.all(ok_inside[(~sat) & (sv > 0)])
    assert np.all(np.abs(xh[sat]) == 6 * sv[sat])
    # a block scale never exceeds what its absmax asks for by more than one E4M3 step
    absmax = np.abs(x).reshape(16, -1, 16).max(axis=2).astype(np.float64)
    t = absmax / 6 / np.float64(g)
    sd = F.e4m3_decode(s)
    assert np.all(np.abs(sd - np.minimum(t, 448)) <= np.maximum(t, 2 ** -6) * 2 ** -3 + 2 ** -10)


def test_brute_force_every_bf16_value_with_fixed_scale():
    # Every positive finite bf16 value between 2^-12 and 2^7, quantised with a
    # fixed g = 1 and a block whose scale is forced to 1.0 by planting a 6:
    # each code must be the grid point nearest to the value (exhaustive check
    # over all 8 grid points, ties to the even code).
    bits = np.arange(0x3980, 0x4300, dtype=np.uint32)            # 2^-12 .. 2^7
    vals = (bits << 16).view(np.float32)
    n = len(vals)
    x = np.zeros((n, 16), np.float32)
    x[:, 0] = 6.0
    x[:, 1] = np.minimum(vals, 6.0)
    c, s, g = quantize(x, g=1.0)
    assert np.all(s == 0x38)
    code = unpack_codes(c)[:, 1]
    v = np.minimum(vals, 6.0).astype(np.float64)
    d = np.abs(v[:, None] - F.E2M1_MAGNITUDES[None, :])
    best = d.min(axis=1)
    cand = d == best[:, None]
    for i in np.nonzero(cand.sum(axis=1) > 1)[0]:               # ties -> even code
        cand[i] = False
        cand[i, [j for j in range(8) if d[i, j] == best[i] and j % 2 == 0][0]] = True
    assert np.array_equal(code, np.argmax(cand, axis=1))


def test_pack_unpack_layout():
    u = np.arange(32, dtype=np.uint8).reshape(1, 32) % 16
    p = pack_codes(u)
    assert p[0, 0] == (0 | (1 << 4)) and p[0, 1] == (2 | (3 << 4))
    assert np.array_equal(unpack_codes(p), u)


def test_dequantize_unscaled_exact_products():
    # every E2M1 x E4M3 product is exactly representable: compare with Python floats
    for q in range(16):
        for s in range(0, 127, 5):
            c = np.array([[q | (q << 4)] * 8], np.uint8)
            sc = np.array([[s]], np.uint8)
            v = dequantize_unscaled(c, sc)[0, 0]
            assert v == F.e2m1_value(q) * F.e4m3_value(s)
