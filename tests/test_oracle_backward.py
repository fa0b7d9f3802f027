"""Pins of the oracle's backward-pass functions of the FP8 linear layer.

Training runs end to end in FP8 (page "NVIDIA NeMo RL erreicht 48%
Geschwindigkeitssteigerung ...", section "Der technische Durchbruch"), so the
data gradient dX = dY W and the weight gradient dW = dY^T X are block-scaled
FP8 GEMMs too, each with its scale blocks along its contraction dimension.
Pins, none of which uses the oracle function under test:
  - the 128-token column blocks against brute force in exact rationals,
    including a ragged last block whose padding must not change the scale;
  - the transposed weight tiles against quantizing W^T directly;
  - dgrad and wgrad against numpy float64 on operands decoded by torch,
    exact rational sums, exact integers, and (wgrad) the special case of
    scales constant over 128 rows, where it is the forward GEMM.
"""
from fractions import Fraction

import numpy as np
import pytest
import torch

from tests.test_oracle_quant import _bf16, _exact_block, _f32

MODES = (0, 1)


def _torch_dec(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _codes(rng, shape):
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    return rng.choice(finite, size=shape).astype(np.uint8)


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M", [128, 200, 1])
def test_colwise_blocks_brute_force(oracle_lib, mode, M):
    """Every 128x1 block of a [M, 256] input (M = 200: one full block and a
    72-row block) against exact rational quantization of its valid values;
    padding codes are +0 and padding does not enter the scale."""
    rng = np.random.default_rng(40 + M + mode)
    x = rng.standard_normal((M, 256)).astype(np.float32)
    x[M // 2, 7] = 91.0                     # outlier in one column block
    x[:, 130] *= 1e-4                       # a column of small values
    xb = _bf16(x)
    qt, st = oracle_lib.quant_act_colwise_t(xb, mode)
    Mp = -(-M // 128) * 128
    assert qt.shape == (256, Mp) and st.shape == (256, Mp // 128)
    vals = _f32(xb)
    for k in (0, 7, 130, 255):
        for mb in range(Mp // 128):
            r0, r1 = 128 * mb, min(M, 128 * mb + 128)
            s_ref, c_ref = _exact_block(vals[r0:r1, k].tolist(), mode)
            assert st[k, mb] == s_ref, (k, mb)
            assert qt[k, r0:r1].tolist() == c_ref, (k, mb)
            assert not qt[k, r1:128 * mb + 128].any()


def test_colwise_blocks_are_independent_and_permute(oracle_lib):
    """Changing one column block changes nothing else; permuting the rows
    inside a block permutes that block's codes and keeps its scale."""
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((256, 384)).astype(np.float32))
    qt, st = oracle_lib.quant_act_colwise_t(x)
    y = x.copy()
    y[128:, 5] = _bf16(rng.standard_normal(128).astype(np.float32) * 100)
    qt2, st2 = oracle_lib.quant_act_colwise_t(y)
    diff = np.argwhere(st2 != st)
    assert diff.tolist() in ([], [[5, 1]])
    keep = np.ones_like(qt, dtype=bool)
    keep[5, 128:] = False
    assert np.array_equal(qt[keep], qt2[keep])
    perm = rng.permutation(128)
    z = x.copy()
    z[:128] = x[perm]
    qt3, st3 = oracle_lib.quant_act_colwise_t(z)
    assert np.array_equal(st3, st)
    assert np.array_equal(qt3[:, :128], qt[:, :128][:, perm])
    assert np.array_equal(qt3[:, 128:], qt[:, 128:])


@pytest.mark.parametrize("mode", MODES)
def test_weight_transposed_equals_quantizing_the_transpose(oracle_lib, mode):
    rng = np.random.default_rng(8 + mode)
    w = (rng.standard_normal((256, 384)) * 0.02).astype(np.float32)
    w[3, 300] = 0.9
    wb = _bf16(w)
    qt, st = oracle_lib.quant_weight_128x128_t(wb, mode)
    q2, s2 = oracle_lib.quant_weight_128x128(np.ascontiguousarray(wb.T), mode)
    assert np.array_equal(qt, q2)
    assert np.array_equal(st.view(np.uint32), s2.view(np.uint32))


def _deq_rows(q, s):
    return _torch_dec(q) * np.repeat(s.astype(np.float64), 128, axis=1)


def _deq_tiles(q, s):
    return _torch_dec(q) * np.repeat(np.repeat(s.astype(np.float64), 128, axis=0), 128, axis=1)


@pytest.mark.parametrize("M,N,K", [(1, 128, 128), (70, 256, 384), (130, 384, 256)])
def test_dgrad_vs_numpy(oracle_lib, M, N, K):
    rng = np.random.default_rng(M + N + K)
    gq = _codes(rng, (M, N))
    gs = np.exp2(rng.uniform(-20, -4, size=(M, N // 128))).astype(np.float32)
    wq = _codes(rng, (N, K))
    ws = rng.uniform(1e-5, 1e-2, size=(N // 128, K // 128)).astype(np.float32)
    y = oracle_lib.gemm_dgrad_f64(gq, gs, wq, ws)
    a, b = _deq_rows(gq, gs), _deq_tiles(wq, ws)
    ref = a @ b
    bound = 1e-12 * (np.abs(a) @ np.abs(b))
    assert y.shape == (M, K)
    assert np.all(np.abs(y - ref) <= bound + 1e-300)
    ms = rng.integers(0, M, 50)
    ks = rng.integers(0, K, 50)
    assert np.array_equal(oracle_lib.gemm_dgrad_sampled_f64(gq, gs, wq, ws, ms, ks), y[ms, ks])


def test_dgrad_exact_rational(oracle_lib):
    """A few outputs summed in exact rationals over N = 256 (two row blocks of
    W, two scale blocks of dY)."""
    rng = np.random.default_rng(17)
    M, N, K = 4, 256, 256
    gq, wq = _codes(rng, (M, N)), _codes(rng, (N, K))
    gs = rng.uniform(1e-6, 1e-3, size=(M, 2)).astype(np.float32)
    ws = rng.uniform(1e-4, 1e-2, size=(2, 2)).astype(np.float32)
    y = oracle_lib.gemm_dgrad_f64(gq, gs, wq, ws)
    dg, dw = _torch_dec(gq).tolist(), _torch_dec(wq).tolist()
    for m in range(M):
        for k in (0, 1, 127, 128, 255):
            terms = [Fraction(dg[m][n]) * Fraction(float(gs[m, n // 128])) * Fraction(dw[n][k])
                     * Fraction(float(ws[n // 128, k // 128])) for n in range(N)]
            exact = sum(terms)
            bound = sum(abs(t) for t in terms) * Fraction(1, 10 ** 14)
            assert abs(Fraction(y[m, k]) - exact) <= bound + Fraction(1, 10 ** 300)


def test_dgrad_exact_integers(oracle_lib):
    rng = np.random.default_rng(19)
    M, N, K = 33, 256, 384
    lut = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)     # -1, 0, +1
    ig = rng.integers(-1, 2, size=(M, N))
    iw = rng.integers(-1, 2, size=(N, K))
    y = oracle_lib.gemm_dgrad_f64(lut[ig + 1], np.ones((M, 2), np.float32), lut[iw + 1],
                                  np.ones((2, 3), np.float32))
    assert np.array_equal(y, (ig @ iw).astype(np.float64))


@pytest.mark.parametrize("N,K,Mp", [(128, 128, 128), (256, 384, 256), (384, 128, 512)])
def test_wgrad_vs_numpy(oracle_lib, N, K, Mp):
    rng = np.random.default_rng(N + K + Mp + 1)
    gq, xq = _codes(rng, (N, Mp)), _codes(rng, (K, Mp))
    gs = np.exp2(rng.uniform(-20, -4, size=(N, Mp // 128))).astype(np.float32)
    xs = rng.uniform(1e-3, 1.0, size=(K, Mp // 128)).astype(np.float32)
    y = oracle_lib.gemm_wgrad_f64(gq, gs, xq, xs)
    a, b = _deq_rows(gq, gs), _deq_rows(xq, xs)
    bound = 1e-12 * (np.abs(a) @ np.abs(b).T)
    assert y.shape == (N, K)
    assert np.all(np.abs(y - a @ b.T) <= bound + 1e-300)
    ns = rng.integers(0, N, 60)
    ks = rng.integers(0, K, 60)
    got = oracle_lib.gemm_wgrad_sampled_f64(gq, gs, xq, xs, ns, ks)
    assert np.all(np.abs(got - y[ns, ks]) <= bound[ns, ks] + 1e-300)


def test_wgrad_exact_rational(oracle_lib):
    rng = np.random.default_rng(23)
    N, K, Mp = 3, 4, 256
    gq, xq = _codes(rng, (N, Mp)), _codes(rng, (K, Mp))
    gs = rng.uniform(1e-6, 1e-3, size=(N, 2)).astype(np.float32)
    xs = rng.uniform(1e-2, 10.0, size=(K, 2)).astype(np.float32)
    y = oracle_lib.gemm_wgrad_f64(gq, gs, xq, xs)
    dg, dx = _torch_dec(gq).tolist(), _torch_dec(xq).tolist()
    for n in range(N):
        for k in range(K):
            terms = [Fraction(dg[n][m]) * Fraction(float(gs[n, m // 128])) * Fraction(dx[k][m])
                     * Fraction(float(xs[k, m // 128])) for m in range(Mp)]
            exact = sum(terms)
            bound = sum(abs(t) for t in terms) * Fraction(1, 10 ** 14)
            assert abs(Fraction(y[n, k]) - exact) <= bound + Fraction(1, 10 ** 300)


def test_wgrad_exact_integers(oracle_lib):
    rng = np.random.default_rng(29)
    N, K, Mp = 128, 256, 384
    lut = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)
    ig = rng.integers(-1, 2, size=(N, Mp))
    ix = rng.integers(-1, 2, size=(K, Mp))
    y = oracle_lib.gemm_wgrad_f64(lut[ig + 1], np.ones((N, 3), np.float32), lut[ix + 1],
                                  np.ones((K, 3), np.float32))
    assert np.array_equal(y, (ig @ ix.T).astype(np.float64))


def test_wgrad_with_tile_constant_scales_is_the_forward_gemm(oracle_lib):
    """When the x-side scales are constant over each 128-row block they are
    128x128 tile scales, and wgrad is the forward GEMM's definition (the C
    oracle's loops, pinned on their own)."""
    rng = np.random.default_rng(31)
    N, K, Mp = 200, 256, 256
    gq, xq = _codes(rng, (N, Mp)), _codes(rng, (K, Mp))
    gs = rng.uniform(1e-5, 1e-3, size=(N, 2)).astype(np.float32)
    tiles = rng.uniform(1e-3, 1.0, size=(2, 2)).astype(np.float32)
    xs = np.repeat(tiles, 128, axis=0)
    y = oracle_lib.gemm_wgrad_f64(gq, gs, xq, xs)
    ref = oracle_lib.gemm_f64(gq, gs, xq, tiles)
    scale = np.abs(_deq_rows(gq, gs)) @ np.abs(_deq_rows(xq, xs)).T
    assert np.all(np.abs(y - ref) <= 1e-12 * scale + 1e-300)


def test_backward_of_quantized_layer_approximates_exact_gradients(oracle_lib):
    """Closing the loop: quantizing dY and W (dgrad) or dY and X along tokens
    (wgrad) and multiplying gives the bf16-exact gradients to within the E4M3
    rounding (relative Frobenius error well below 2^-4)."""
    rng = np.random.default_rng(37)
    M, N, K = 300, 256, 384
    x = _bf16(rng.standard_normal((M, K)).astype(np.float32))
    w = _bf16((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    g = _bf16((rng.standard_normal((M, N)) * 1e-3).astype(np.float32))
    xf, wf, gf = (_f32(a).astype(np.float64) for a in (x, w, g))
    gq, gs = oracle_lib.quant_act_1x128(g)
    wq, ws = oracle_lib.quant_weight_128x128(w)
    dx = oracle_lib.gemm_dgrad_f64(gq, gs, wq, ws)
    ref = gf @ wf
    assert np.linalg.norm(dx - ref) / np.linalg.norm(ref) < 0.04
    gtq, gts = oracle_lib.quant_act_colwise_t(g)
    xtq, xts = oracle_lib.quant_act_colwise_t(x)
    dw = oracle_lib.gemm_wgrad_f64(gtq, gts, xtq, xts)
    ref = gf.T @ xf
    assert np.linalg.norm(dw - ref) / np.linalg.norm(ref) < 0.04
