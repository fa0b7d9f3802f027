"""Pins of the oracle's E4M3 codec against things other than itself:
torch's float8_e4m3fn decoder and cast, a brute-force nearest-code search in
exact rationals, and the landmark values the format definition fixes.

E4M3 with 4 exponent / 3 mantissa bits and a +-448 range: page "FP8
Trainingsinfrastructuur: Numerieke Precisie van de Volgende Generatie",
section "Het landschap van numerieke precisie".
"""
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests._exact import brute_force_e4m3, f32_from_bits, torch_e4m3_values

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _read_landmarks():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_landmarks.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if not line:
                continue
            code, val = line.split()[:2]
            rows.append((int(code, 16), val))
    return rows


def test_decode_table_matches_torch(oracle_lib):
    t = oracle_lib.e4m3_decode_table()
    ref = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(np.isnan(t), np.isnan(ref))
    ok = ~np.isnan(t)
    assert np.array_equal(t[ok], ref[ok])
    # sign of zero
    assert math.copysign(1.0, t[0x80]) == -1.0 and math.copysign(1.0, t[0x00]) == 1.0


def test_decode_landmarks(oracle_lib):
    t = oracle_lib.e4m3_decode_table()
    for code, val in _read_landmarks():
        if val == "nan":
            assert math.isnan(t[code]), hex(code)
        elif val == "-0":
            assert t[code] == 0.0 and math.copysign(1.0, t[code]) < 0
        else:
            assert Fraction(t[code]) == Fraction(val), hex(code)


def test_code_table_structure(oracle_lib):
    t = oracle_lib.e4m3_decode_table()
    pos = t[:0x80]
    finite = pos[~np.isnan(pos)]
    assert np.count_nonzero(np.isnan(t)) == 2            # 0x7F and 0xFF only
    assert np.count_nonzero(finite > 0) == 126            # positive finite values
    assert finite.max() == 448.0
    assert np.all(np.diff(finite) > 0)                    # monotone in the code
    assert np.array_equal(t[0x80:0xFF], -t[0x00:0x7F])    # sign symmetry


def _codes_midpoints_and_neighbours():
    vals = [v for v in torch_e4m3_values()[:0x7F] if v is not None]
    pts = set()
    for v in vals:
        pts.add(v)
    for a, b in zip(vals[:-1], vals[1:]):
        pts.add((a + b) / 2)
    out = []
    for p in sorted(pts):
        f = float(p)  # every code and midpoint here is an exact fp32 value
        assert Fraction(f) == p
        b = np.float32(f).view(np.uint32).item()
        for d in (-1, 0, 1):
            if b + d >= 0:
                out.append(f32_from_bits(b + d))
    # around the saturation threshold and above
    for v in (447.99997, 448.0, 448.00003, 455.0, 463.99997, 464.0, 464.00003, 1e6, 3.0e38):
        out.append(float(np.float32(v)))
    return out


def test_encode_vs_brute_force_codes_midpoints(oracle_lib):
    xs = _codes_midpoints_and_neighbours()
    xs = xs + [-x for x in xs]
    got = oracle_lib.e4m3_encode(np.array(xs, dtype=np.float32))
    for x, g in zip(xs, got):
        want = brute_force_e4m3(Fraction(x), negative_zero=math.copysign(1.0, x) < 0)
        assert g == want, (x, hex(g), hex(want))


def test_encode_vs_brute_force_random(oracle_lib):
    rng = np.random.default_rng(7)
    # log-uniform magnitudes over the whole E4M3 range and below, both signs
    mag = np.exp2(rng.uniform(-14, 9.2, size=3000)).astype(np.float32)
    xs = mag * rng.choice([-1.0, 1.0], size=mag.size).astype(np.float32)
    got = oracle_lib.e4m3_encode(xs)
    for x, g in zip(xs.tolist(), got):
        want = brute_force_e4m3(Fraction(x), negative_zero=math.copysign(1.0, x) < 0)
        assert g == want, (x, hex(g), hex(want))


def test_encode_signed_zero_and_tiny(oracle_lib):
    xs = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, -(2.0 ** -10), 2.0 ** -10 * 1.0000001],
                  dtype=np.float32)
    got = oracle_lib.e4m3_encode(xs).tolist()
    # 2^-10 is the midpoint between 0 and 2^-9: ties to even -> zero
    assert got == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80, 0x01]


def test_encode_saturates(oracle_lib):
    xs = np.array([448.0, 449.0, 480.0, 1e4, 3.4e38, -448.0, -1e10], dtype=np.float32)
    assert oracle_lib.e4m3_encode(xs).tolist() == [0x7E] * 5 + [0xFE] * 2


def _torch_cast(x):
    return torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


@pytest.mark.parametrize("stride", [1])
def test_encode_exhaustive_vs_torch(oracle_lib, stride):
    """Every non-negative fp32 value up to 464 (torch's cast rounds to nearest
    even and agrees with saturation up to there), plus every 97th negative one."""
    hi = np.float32(464.0).view(np.uint32).item()
    chunk = 1 << 26
    for start in range(0, hi + 1, chunk):
        bits = np.arange(start, min(start + chunk, hi + 1), stride, dtype=np.uint32)
        x = bits.view(np.float32)
        a = oracle_lib.e4m3_encode(x)
        b = _torch_cast(x)
        bad = np.nonzero(a != b)[0]
        assert bad.size == 0, (x[bad[:5]], a[bad[:5]], b[bad[:5]])
        neg = (bits[::97] | np.uint32(0x80000000)).view(np.float32)
        assert np.array_equal(oracle_lib.e4m3_encode(neg), _torch_cast(neg))
