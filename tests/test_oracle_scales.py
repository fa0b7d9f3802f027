"""Pins of the oracle's block scale (amax and power-of-two modes).

amax mode is pinned to exact rational rounding; pow2 mode to its closed form
(448 = 1.75 * 2^8, so with amax = m * 2^E, m in [1,2): e = E-8 if m <= 1.75
else E-7, kept at -127 or above, the range of an E8M0 scale) and to its
defining inequality.  Power-of-two scales: page "NVIDIA
NeMo RL erreicht 48% Geschwindigkeitssteigerung ...", section "Warum dies fuer
die KI-Oekonomie wichtig ist"; 448: page "FP8 Trainingsinfrastructuur",
section "Het landschap van numerieke precisie".
"""
import math
import os
from fractions import Fraction

import numpy as np

from tests._exact import f32_bits, round_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    rows = []
    with open(os.path.join(GOLDEN, "closed_form_scales.txt")) as f:
        for line in f:
            line = line.split("#")[0].strip()
            if line:
                a, bits, p2 = line.split()[:3]
                rows.append((float(a), int(bits, 16), Fraction(p2)))
    return rows


def test_closed_form_table(oracle_lib):
    rows = _golden()
    assert len(rows) >= 6
    for amax, bits, p2 in rows:
        s_amax = oracle_lib.block_scale(np.float32(amax), oracle_lib.MODE_AMAX).item()
        s_pow2 = oracle_lib.block_scale(np.float32(amax), oracle_lib.MODE_POW2).item()
        assert f32_bits(s_amax) == bits, (amax, hex(f32_bits(s_amax)))
        assert Fraction(s_pow2) == p2, (amax, s_pow2)


def _bf16_values(rng, n):
    """Random positive finite bf16 values over the whole range, incl. subnormals."""
    bits = rng.integers(1, 0x7F80, size=n).astype(np.uint32) << 16
    return bits.view(np.float32)


def _edge_amax():
    vals = [2.0 ** -133, 2.0 ** -126, 2.0 ** -127, 1.75, 1.7578125, 448.0, 449.0, 3.3895314e38,
            1.0, 2.0 ** -141, 7.0, 0.5, 1.75 * 2.0 ** -100, 1.7578125 * 2.0 ** 100]
    return np.array(vals, dtype=np.float32)


def test_amax_mode_is_correctly_rounded_quotient(oracle_lib):
    rng = np.random.default_rng(3)
    amax = np.concatenate([_bf16_values(rng, 4000), _edge_amax()])
    got = oracle_lib.block_scale(amax, oracle_lib.MODE_AMAX)
    for a, s in zip(amax.tolist(), got.tolist()):
        want = round_to_f32(Fraction(a) / 448)
        assert s == want and want > 0, (a, s, want)


def test_pow2_mode_closed_form(oracle_lib):
    rng = np.random.default_rng(4)
    amax = np.concatenate([_bf16_values(rng, 4000), _edge_amax()])
    got = oracle_lib.block_scale(amax, oracle_lib.MODE_POW2)
    for a, s in zip(amax.tolist(), got.tolist()):
        m, E = math.frexp(a)       # a = m * 2^E, m in [0.5,1)
        m, E = 2 * m, E - 1         # m in [1,2)
        e = E - 8 if m <= 1.75 else E - 7
        e = max(e, -127)
        assert s == math.ldexp(1.0, e), (a, s, e)
        # defining property: smallest power of two, not below 2^-127, with
        # 448*s >= amax
        assert Fraction(448) * Fraction(s) >= Fraction(a)
        assert s == 2.0 ** -127 or Fraction(448) * Fraction(s) / 2 < Fraction(a)


def test_pow2_mode_lower_bound(oracle_lib):
    """Blocks with amax <= 448 * 2^-127 all get the E8M0 floor 2^-127; the next
    power of two up is the first above it."""
    a = np.array([2.0 ** -149, 2.0 ** -140, 448 * 2.0 ** -127, 448 * 2.0 ** -127 * (1 + 2.0 ** -23),
                  1.75 * 2.0 ** -119], dtype=np.float32)
    got = oracle_lib.block_scale(a, oracle_lib.MODE_POW2).tolist()
    assert got == [2.0 ** -127, 2.0 ** -127, 2.0 ** -127, 2.0 ** -126, 2.0 ** -127]


def test_zero_block_scale_is_one(oracle_lib):
    z = np.zeros(2, dtype=np.float32)
    assert oracle_lib.block_scale(z, oracle_lib.MODE_AMAX).tolist() == [1.0, 1.0]
    assert oracle_lib.block_scale(z, oracle_lib.MODE_POW2).tolist() == [1.0, 1.0]
