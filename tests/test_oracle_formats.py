"""Pins of the oracle's number formats against closed forms, golden tables and
torch's float8 conversion (a library routine independent of the oracle)."""
import os

import numpy as np
import pytest
import torch

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as fh:
        for line in fh:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            a, b = line.split()
            rows.append((int(a, 0), float(b)))
    return rows


def test_e2m1_table_matches_golden():
    rows = _read_golden("e2m1_values.txt")
    assert len(rows) == 16
    for code, val in rows:
        got = F.E2M1_TABLE[code]
        assert got == val, (code, got, val)
        assert np.signbit(got) == np.signbit(val), code   # 8 is -0


def test_e2m1_magnitude_set_is_the_fp4_grid():
    assert sorted(set(np.abs(F.E2M1_TABLE).tolist())) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e4m3_points_match_golden():
    for code, val in _read_golden("e4m3_points.txt"):
        got = F.E4M3_TABLE[code]
        if np.isnan(val):
            assert np.isnan(got), code
        else:
            assert got == val and np.signbit(got) == np.signbit(val), (hex(code), got, val)


def test_e4m3_decode_all_codes_matches_torch():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    got = F.e4m3_decode(np.arange(256))
    nan = np.isnan(ref)
    assert np.array_equal(nan, np.isnan(got))
    assert np.array_equal(ref[~nan], got[~nan])
    assert np.array_equal(np.signbit(ref[~nan]), np.signbit(got[~nan]))
    assert F.E4M3_POS.max() == 448.0 and len(F.E4M3_POS) == 127


def _torch_e4m3(t32):
    return torch.from_numpy(t32).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_encode_matches_torch_rne():
    rng = np.random.default_rng(7)
    vals = F.E4M3_POS
    mids = (vals[:-1] + vals[1:]) / 2                       # exact ties
    near = np.concatenate([mids, np.nextafter(mids.astype(np.float32), 0),
                           np.nextafter(mids.astype(np.float32), 1000)])
    t = np.concatenate([
        vals, mids, near,
        rng.uniform(0, 448, 20000),
        np.exp(rng.uniform(np.log(2.0 ** -12), np.log(448), 20000)),
        [0.0, 2.0 ** -10, 2.0 ** -10 * 1.0000001, 2.0 ** -11, 447.9, 448.0],
    ]).astype(np.float32)
    t = t[(t >= 0) & (t <= 448)]
    assert np.array_equal(F.e4m3_encode_satfinite(t), _torch_e4m3(t))


def test_e4m3_encode_saturates_above_448():
    t = np.array([448.0, 449.0, 463.9, 464.0, 470.0, 1e6, 3.0e38], dtype=np.float32)
    assert np.all(F.e4m3_encode_satfinite(t) == 0x7E)


def test_e4m3_encode_roundtrip_all_finite_codes():
    assert np.array_equal(F.e4m3_encode_satfinite(F.E4M3_POS.astype(np.float32)),
                          np.arange(127, dtype=np.uint8))


# E2M1 nearest-even decisions written out by hand: the decision points are the
# midpoints of the grid 0, .5, 1, 1.5, 2, 3, 4, 6; an exact midpoint goes to the
# code with an even mantissa (0:0, 2:1.0, 4:2.0, 6:4.0).
E2M1_CASES = [
    (0.0, 0), (0.1, 0), (0.25, 0), (0.2500001, 1), (0.5, 1), (0.7499999, 1),
    (0.75, 2), (1.0, 2), (1.25, 2), (1.2500001, 3), (1.5, 3), (1.7499999, 3),
    (1.75, 4), (2.0, 4), (2.5, 4), (2.5000002, 5), (3.0, 5), (3.4999998, 5),
    (3.5, 6), (4.0, 6), (5.0, 6), (5.0000005, 7), (6.0, 7), (7.0, 7), (1e9, 7),
]


@pytest.mark.parametrize("v,code", E2M1_CASES)
def test_e2m1_encode_decisions(v, code):
    assert int(F.e2m1_encode_magnitude(np.array([v], dtype=np.float32))[0]) == code


def test_e2m1_encode_roundtrip_and_monotone():
    assert np.array_equal(F.e2m1_encode_magnitude(F.E2M1_MAGNITUDES), np.arange(8))
    v = np.linspace(0, 8, 100001, dtype=np.float32)
    c = F.e2m1_encode_magnitude(v)
    assert np.all(np.diff(c.astype(int)) >= 0)
    # the chosen grid point is never farther than any other grid point
    d = np.abs(v.astype(np.float64) - F.E2M1_MAGNITUDES[c])
    dmin = np.min(np.abs(np.minimum(v, 6).astype(np.float64)[:, None] - F.E2M1_MAGNITUDES[None, :]), axis=1)
    assert np.all(d[v <= 6] == dmin[v <= 6])


def test_round_to_bf16_matches_torch_on_float32_inputs():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(50000) * 10.0 ** rng.uniform(-8, 8, 50000)]).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    assert np.array_equal(F.round_to_bf16(x.astype(np.float64)), ref)


def test_round_to_bf16_rounds_float64_once():
    # 1 + 2^-8 is the exact midpoint between bf16 1.0 and 1 + 2^-7: tie -> even (1.0).
    # Adding 2^-40 makes it round up; a detour through float32 would lose the 2^-40
    # and produce 1.0.
    assert F.round_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert F.round_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -40]))[0] == np.float32(1 + 2.0 ** -7)
    assert F.round_to_bf16(np.array([-(1 + 3 * 2.0 ** -8)]))[0] == np.float32(-(1 + 2.0 ** -6))
