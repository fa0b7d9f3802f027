"""Pins of the oracle's activation (1x128) and weight (128x128) quantizers.

Blocks of 1x128 for activations and 128x128 for weights, E4M3 codes: page
"NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung ...", section "Der
technische Durchbruch".  Pins: brute force in exact rationals on one block and
one tile, exact round trips of representable values, and invariants that any
correct quantizer satisfies (sign symmetry, power-of-two equivariance, block
independence, permutation and row-gather equivariance).
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests._exact import brute_force_e4m3, round_to_f32

MODES = (0, 1)


def _bf16(x):
    """fp32 numpy -> bf16 bits (uint16), torch's round-to-nearest-even."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f32(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32)


def _exact_block(vals, mode):
    """Exact quantization of one block of fp32 values: amax, scale and codes."""
    amax = max(abs(Fraction(v)) for v in vals)
    if amax == 0:
        s = 1.0
    elif mode == 0:
        s = round_to_f32(amax / 448)
    else:
        e = 0
        while Fraction(448) * Fraction(2) ** e < amax:
            e += 1
        while Fraction(448) * Fraction(2) ** (e - 1) >= amax:
            e -= 1
        e = max(e, -127)  # a power-of-two scale is an E8M0 value: 2^-127 at least
        s = float(Fraction(2) ** e)
    codes = []
    for v in vals:
        r = round_to_f32(Fraction(v) / Fraction(s))
        neg0 = math.copysign(1.0, v) < 0
        codes.append(brute_force_e4m3(Fraction(r), negative_zero=neg0))
    return s, codes


@pytest.mark.parametrize("mode", MODES)
def test_act_block_brute_force(oracle_lib, mode):
    rng = np.random.default_rng(11 + mode)
    x = rng.standard_normal((3, 256)).astype(np.float32)
    x[1, 130] = 37.0                      # an outlier in one block only
    x[2, :128] *= 1e-3
    xb = _bf16(x)
    q, s = oracle_lib.quant_act_1x128(xb, mode)
    vals = _f32(xb)
    for m in range(3):
        for kb in range(2):
            blk = vals[m, kb * 128:(kb + 1) * 128].tolist()
            s_ref, c_ref = _exact_block(blk, mode)
            assert s[m, kb] == s_ref
            assert q[m, kb * 128:(kb + 1) * 128].tolist() == c_ref


@pytest.mark.parametrize("mode", MODES)
def test_weight_tile_brute_force(oracle_lib, mode):
    rng = np.random.default_rng(21 + mode)
    w = (rng.standard_normal((128, 256)) * 0.02).astype(np.float32)
    w[5, 200] = -0.5                      # tile (0,1) gets a larger amax
    wb = _bf16(w)
    q, s = oracle_lib.quant_weight_128x128(wb, mode)
    vals = _f32(wb)
    for kb in range(2):
        tile = vals[:, kb * 128:(kb + 1) * 128].reshape(-1).tolist()
        s_ref, c_ref = _exact_block(tile, mode)
        assert s[0, kb] == s_ref
        assert q[:, kb * 128:(kb + 1) * 128].reshape(-1).tolist() == c_ref


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("j", [-20, -3, 0, 5, 30])
def test_exact_round_trip(oracle_lib, mode, j):
    """A block of E4M3 values times 2^j that contains +-448*2^j comes back as
    exactly those codes with s = 2^j, in both modes."""
    vals = torch.arange(256, dtype=torch.uint8).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    rng = np.random.default_rng(5)
    codes = rng.choice([c for c in range(256) if c not in (0x7F, 0xFF)], size=128).astype(np.uint8)
    codes[17] = 0x7E
    codes[90] = 0xFE
    x = (vals[codes] * 2.0 ** j).astype(np.float32)
    xb = _bf16(x)
    assert np.array_equal(_f32(xb), x)    # E4M3 values times 2^j are exact in bf16
    q, s = oracle_lib.quant_act_1x128(xb[None, :], mode)
    assert s[0, 0] == 2.0 ** j
    assert np.array_equal(q[0], codes)


@pytest.mark.parametrize("mode", MODES)
def test_sign_symmetry(oracle_lib, mode):
    rng = np.random.default_rng(31)
    xb = _bf16(rng.standard_normal((4, 512)).astype(np.float32) * 3)
    q, s = oracle_lib.quant_act_1x128(xb, mode)
    qn, sn = oracle_lib.quant_act_1x128(xb ^ np.uint16(0x8000), mode)
    assert np.array_equal(s, sn)
    assert np.array_equal(qn, q ^ np.uint8(0x80))


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("j", [-7, 4])
def test_power_of_two_equivariance(oracle_lib, mode, j):
    rng = np.random.default_rng(41)
    x = _f32(_bf16(rng.standard_normal((4, 256)).astype(np.float32)))
    q, s = oracle_lib.quant_act_1x128(_bf16(x), mode)
    q2, s2 = oracle_lib.quant_act_1x128(_bf16(x * 2.0 ** j), mode)
    assert np.array_equal(q, q2)
    assert np.array_equal(s * np.float32(2.0 ** j), s2)


@pytest.mark.parametrize("mode", MODES)
def test_block_independence_and_permutation(oracle_lib, mode):
    rng = np.random.default_rng(51)
    xb = _bf16(rng.standard_normal((2, 384)).astype(np.float32))
    q, s = oracle_lib.quant_act_1x128(xb, mode)
    x2 = xb.copy()
    x2[0, 128:256] = _bf16(rng.standard_normal(128).astype(np.float32) * 50)
    q2, s2 = oracle_lib.quant_act_1x128(x2, mode)
    keep = np.ones_like(q, dtype=bool)
    keep[0, 128:256] = False
    assert np.array_equal(q[keep], q2[keep])
    assert s2[0, 0] == s[0, 0] and s2[0, 2] == s[0, 2] and np.array_equal(s[1], s2[1])
    perm = rng.permutation(128)
    x3 = xb.copy()
    x3[1, 256:384] = xb[1, 256:384][perm]
    q3, s3 = oracle_lib.quant_act_1x128(x3, mode)
    assert np.array_equal(q3[1, 256:384], q[1, 256:384][perm]) and s3[1, 2] == s[1, 2]


def test_row_gather_commutes(oracle_lib):
    rng = np.random.default_rng(61)
    xb = _bf16(rng.standard_normal((40, 256)).astype(np.float32))
    idx = rng.integers(0, 40, size=100)
    q, s = oracle_lib.quant_act_1x128(xb, 0)
    qg, sg = oracle_lib.quant_act_1x128(xb[idx], 0)
    assert np.array_equal(qg, q[idx]) and np.array_equal(sg, s[idx])


@pytest.mark.parametrize("mode", MODES)
def test_zero_blocks(oracle_lib, mode):
    xb = np.zeros((2, 256), dtype=np.uint16)
    xb[1, :] = 0x8000                     # -0.0
    xb[0, 128:] = _bf16(np.linspace(-1, 1, 128, dtype=np.float32))
    q, s = oracle_lib.quant_act_1x128(xb, mode)
    assert s[0, 0] == 1.0 and s[1, 0] == 1.0 and s[1, 1] == 1.0
    assert np.all(q[0, :128] == 0) and np.all(q[1] == 0x80)


@pytest.mark.parametrize("mode", MODES)
def test_subnormal_block(oracle_lib, mode):
    """A block of bf16 subnormals: scale may itself be an fp32 subnormal and
    saturation can occur; checked against exact arithmetic."""
    rng = np.random.default_rng(71)
    bits = rng.integers(1, 0x80, size=128).astype(np.uint16)      # positive subnormals
    bits[::3] |= np.uint16(0x8000)
    q, s = oracle_lib.quant_act_1x128(bits[None, :], mode)
    s_ref, c_ref = _exact_block(_f32(bits).tolist(), mode)
    assert s[0, 0] == s_ref
    assert q[0].tolist() == c_ref


def test_weight_tiles_match_row_blocks_with_shared_scale(oracle_lib):
    """Each 128x128 weight tile uses one scale: its codes equal those of the
    per-element rule with that tile's scale (cross-check of the tile indexing
    on a 256x384 matrix, with a distinct amax planted in every tile)."""
    rng = np.random.default_rng(81)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    for i in range(2):
        for j in range(3):
            w[i * 128 + 3 * j, j * 128 + 7 * i] = 0.1 * (1 + i + 2 * j)
    wb = _bf16(w)
    q, s = oracle_lib.quant_weight_128x128(wb, 0)
    vals = _f32(wb)
    for i in range(2):
        for j in range(3):
            tile = vals[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128]
            assert s[i, j] == round_to_f32(Fraction(float(np.abs(tile).max())) / 448)
            r = (tile / s[i, j]).astype(np.float32)   # numpy fp32 division: IEEE
            want = torch.from_numpy(np.clip(r, -448, 448)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
            assert np.array_equal(q[i * 128:(i + 1) * 128, j * 128:(j + 1) * 128], want)
