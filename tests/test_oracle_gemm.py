"""Pins of the oracle's block-scaled GEMM and grouped GEMM.

The GEMM is Y = X * W^T with each operand dequantised by its block scales
(1x128 for X, 128x128 for W) and the products summed in fp64; linear layers
run in FP8 per page "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung
...", section "Der technische Durchbruch".  Pins: numpy's float64 matmul on
operands dequantised through torch's E4M3 decoder, exact rational arithmetic on
a small tile, exact integers, and the grouped form against per-group numpy.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch


def _torch_dec(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _rand_operands(rng, M, N, K, groups=None):
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    aq = rng.choice(codes, size=(M, K)).astype(np.uint8)
    as_ = np.exp2(rng.uniform(-12, 4, size=(M, K // 128))).astype(np.float32)
    shape_b = (N, K) if groups is None else (groups, N, K)
    bq = rng.choice(codes, size=shape_b).astype(np.uint8)
    shape_s = (N // 128, K // 128) if groups is None else (groups, N // 128, K // 128)
    bs = rng.uniform(1e-5, 1e-2, size=shape_s).astype(np.float32)
    return aq, as_, bq, bs


def _numpy_ref(aq, as_, bq, bs):
    a = _torch_dec(aq) * np.repeat(as_.astype(np.float64), 128, axis=1)
    sb = np.repeat(np.repeat(bs.astype(np.float64), 128, axis=0), 128, axis=1)
    b = _torch_dec(bq) * sb
    return a @ b.T


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (37, 256, 384), (130, 384, 256)])
def test_gemm_vs_numpy(oracle_lib, M, N, K):
    rng = np.random.default_rng(M * 7 + N + K)
    aq, as_, bq, bs = _rand_operands(rng, M, N, K)
    y = oracle_lib.gemm_f64(aq, as_, bq, bs)
    ref = _numpy_ref(aq, as_, bq, bs)
    scale = np.abs(_torch_dec(aq) * np.repeat(as_, 128, 1)) @ np.abs(
        _torch_dec(bq) * np.repeat(np.repeat(bs, 128, 0), 128, 1)).T
    assert np.all(np.abs(y - ref) <= 1e-12 * scale + 1e-300)


def test_gemm_exact_rational_tile(oracle_lib):
    """16x16 outputs over K = 256 (two scale blocks along K, two along N)."""
    rng = np.random.default_rng(99)
    M, N, K = 16, 256, 256
    aq, as_, bq, bs = _rand_operands(rng, M, N, K)
    ns = np.array(list(range(8)) + list(range(128, 136)))
    y = oracle_lib.gemm_f64(aq, as_, bq, bs)
    da = _torch_dec(aq).tolist()
    db = _torch_dec(bq).tolist()
    for m in range(M):
        for n in ns:
            exact = Fraction(0)
            for k in range(K):
                exact += (Fraction(da[m][k]) * Fraction(float(as_[m, k // 128]))) * (
                    Fraction(db[n][k]) * Fraction(float(bs[n // 128, k // 128])))
            err = abs(Fraction(y[m, n]) - exact)
            bound = sum(abs(Fraction(da[m][k]) * Fraction(db[n][k])) for k in range(K)) * Fraction(1, 10 ** 15) * Fraction(float(as_[m].max() * bs.max()))
            assert err <= bound + Fraction(1, 10 ** 300)


def test_gemm_exact_integers(oracle_lib):
    """Codes for -1, 0, 1 with unit scales: every output is an exact integer
    equal to the integer matrix product."""
    rng = np.random.default_rng(5)
    M, N, K = 50, 256, 256
    lut = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)     # -1, 0, +1
    ia = rng.integers(-1, 2, size=(M, K))
    ib = rng.integers(-1, 2, size=(N, K))
    y = oracle_lib.gemm_f64(lut[ia + 1], np.ones((M, 2), np.float32), lut[ib + 1], np.ones((2, 2), np.float32))
    assert np.array_equal(y, (ia @ ib.T).astype(np.float64))


def test_gemm_sampled_equals_full(oracle_lib):
    rng = np.random.default_rng(6)
    aq, as_, bq, bs = _rand_operands(rng, 70, 256, 256)
    y = oracle_lib.gemm_f64(aq, as_, bq, bs)
    ms = rng.integers(0, 70, size=200)
    ns = rng.integers(0, 256, size=200)
    assert np.array_equal(oracle_lib.gemm_sampled_f64(aq, as_, bq, bs, ms, ns), y[ms, ns])


def test_grouped_vs_numpy_with_empty_groups(oracle_lib):
    rng = np.random.default_rng(8)
    G, N, K = 5, 256, 256
    sizes = [3, 0, 70, 1, 0]
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    aq, as_, bq, bs = _rand_operands(rng, int(off[-1]), N, K, groups=G)
    y = oracle_lib.grouped_gemm_f64(aq, as_, bq, bs, off)
    for g in range(G):
        r0, r1 = off[g], off[g + 1]
        if r1 > r0:
            ref = _numpy_ref(aq[r0:r1], as_[r0:r1], bq[g], bs[g])
            assert np.allclose(y[r0:r1], ref, rtol=1e-12, atol=0)
    ms = rng.integers(0, off[-1], size=50)
    grp = np.searchsorted(off, ms, side="right") - 1
    ns = rng.integers(0, N, size=50)
    assert np.array_equal(oracle_lib.grouped_gemm_sampled_f64(aq, as_, bq, bs, grp, ms, ns), y[ms, ns])
