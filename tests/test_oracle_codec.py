"""Pins of the oracle's E4M3 codec against things other than itself:
hand-worked values of the format (tests/golden), an exact brute-force
nearest-value search in rational arithmetic, and torch's independent
float8_e4m3fn CPU cast."""

import bisect
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_table(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                rows.append(line.split()[:2])
    return rows


# ---------------------------------------------------------------- brute force
def _grid():
    """All non-negative finite E4M3FN magnitudes, by construction from the
    bit fields (no shared code with the oracle): (Fraction value, code)."""
    out = []
    for code in range(0x7F):               # 0x7F is NaN
        ex, man = code >> 3, code & 7
        if ex == 0:
            v = Fraction(man, 512)
        else:
            v = Fraction(8 + man) * Fraction(2) ** (ex - 10)
        out.append((v, code))
    return out


GRID = _grid()


GRID_VALUES = [v for v, _ in GRID]          # increasing with the code


def brute_encode(y):
    """Nearest grid magnitude by an exact search in rationals (the two
    neighbours of |y| on the sorted grid), ties to the even code (adjacent
    magnitudes have adjacent codes, so exactly one is even), saturation above
    the largest value, sign bit of y kept."""
    a = abs(Fraction(float(y)))
    if a >= GRID[-1][0]:
        code = GRID[-1][1]
    else:
        hi = bisect.bisect_left(GRID_VALUES, a)
        if GRID_VALUES[hi] == a:
            code = GRID[hi][1]
        else:
            lo = hi - 1
            dlo, dhi = a - GRID_VALUES[lo], GRID_VALUES[hi] - a
            if dlo < dhi or (dlo == dhi and GRID[lo][1] % 2 == 0):
                code = GRID[lo][1]
            else:
                code = GRID[hi][1]
    if math.copysign(1.0, float(y)) < 0:
        code |= 0x80
    return code


def _probe_points():
    mags = np.array([float(v) for v, _ in GRID])
    mids = (mags[:-1] + mags[1:]) / 2
    pts = np.concatenate([mags, mids]).astype(np.float32)
    up = np.nextafter(pts, np.float32(np.inf))
    dn = np.nextafter(pts, np.float32(-np.inf))
    rng = np.random.Generator(np.random.PCG64(7))
    rnd = rng.uniform(-448, 448, 4000).astype(np.float32)
    tiny = (rng.uniform(-2.0 ** -5, 2.0 ** -5, 2000)).astype(np.float32)
    allp = np.concatenate([pts, up, dn, -pts, -up, -dn, rnd, tiny,
                           np.array([0.0, -0.0, 1e-30, -1e-30, 1e-45], np.float32)])
    return allp[np.abs(allp) <= 500].astype(np.float32)


# ---------------------------------------------------------------------- tests
def test_golden_decode_values():
    for code_s, val_s in _read_table("e4m3fn_values.txt"):
        code = int(code_s, 16)
        got = float(e4m3.decode(np.array([code], np.uint8))[0])
        if val_s == "nan":
            assert math.isnan(got), code_s
        else:
            want = float(val_s)
            assert got == want and math.copysign(1, got) == math.copysign(1, want), (code_s, got)


def test_golden_encode_values():
    for val_s, code_s in _read_table("e4m3fn_encode.txt"):
        y = np.float32(float(val_s))
        got = int(e4m3.encode(np.array([y], np.float32))[0])
        assert got == int(code_s, 16), (val_s, hex(got), code_s)


def test_all_256_codes_closed_form():
    codes = np.arange(256, dtype=np.uint8)
    vals = e4m3.decode(codes)
    nan = np.isnan(vals)
    assert sorted(np.nonzero(nan)[0].tolist()) == [0x7F, 0xFF]
    pos = vals[:0x7F]
    assert np.all(np.diff(pos) > 0), "codes 0x00..0x7E must increase strictly"
    assert pos[-1] == 448.0 and pos[1] == 2.0 ** -9 and pos[8] == 2.0 ** -6
    neg = vals[0x80:0xFF]
    assert np.array_equal(neg, -pos) and np.signbit(vals[0x80])
    # agreement with the brute-force grid, value by value
    for v, c in GRID:
        assert Fraction(float(vals[c])) == v


def test_round_trip_254_codes():
    fin = e4m3.finite_codes()
    assert fin.size == 254
    back = e4m3.encode(e4m3.decode(fin).astype(np.float32))
    assert np.array_equal(back, fin)


def test_encode_matches_brute_force():
    pts = _probe_points()
    got = e4m3.encode(pts)
    want = np.array([brute_encode(p) for p in pts], dtype=np.uint8)
    bad = np.nonzero(got != want)[0]
    assert bad.size == 0, [(float(pts[i]), hex(got[i]), hex(want[i])) for i in bad[:10]]


def test_encode_matches_torch_cast_in_range():
    pts = _probe_points()
    pts = pts[np.abs(pts) <= 448]
    ref = torch.from_numpy(pts).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode(pts)
    assert np.array_equal(got, ref)
    rng = np.random.Generator(np.random.PCG64(11))
    big = rng.uniform(-448, 448, 200000).astype(np.float32)
    ref = torch.from_numpy(big).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(e4m3.encode(big), ref)


def test_saturation_and_signed_zero():
    y = np.array([448.0, 449.0, 463.9, 464.0, 465.0, 1e6, 3.0e38,
                  -449.0, -1e6, 0.0, -0.0, -1e-40, 1e-40], np.float32)
    got = e4m3.encode(y).tolist()
    assert got == [0x7E] * 7 + [0xFE] * 2 + [0x00, 0x80, 0x80, 0x00]


def test_encode_rejects_nan():
    with pytest.raises(ValueError):
        e4m3.encode(np.array([np.nan], np.float32))
