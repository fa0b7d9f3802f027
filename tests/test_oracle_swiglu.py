"""Pins of the oracle's fused gate+up GEMM with SwiGLU and output quantization.

The activation's quantization is part of the quantization-kernel overhead the
page blames for the gap to 2x (page "NVIDIA NeMo RL erreicht 48%
Geschwindigkeitssteigerung ...", section "Leistungsgewinne in der
Praxis").  Pins, independent of the functions under test:
  - the 128-block interleave against explicit index arithmetic;
  - h against torch's silu in float64 on the bf16-rounded gate and up taken
    from the plain GEMM by that index arithmetic;
  - closed forms: g = 0 gives 0, exact-integer products give h from math.exp;
  - the quantized output against the pinned row quantizer of bf16(h).
"""
import math

import numpy as np
import torch


def _codes(rng, shape):
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    return rng.choice(finite, size=shape).astype(np.uint8)


def test_interleave_index_arithmetic(oracle_lib):
    y = np.arange(3 * 768, dtype=np.float64).reshape(3, 768)
    g, u = oracle_lib.swiglu_split(y)
    for j in range(384):
        p, c = divmod(j, 128)
        assert (g[:, j] == y[:, 256 * p + c]).all()
        assert (u[:, j] == y[:, 256 * p + 128 + c]).all()


def test_h_against_torch_silu(oracle_lib):
    rng = np.random.default_rng(3)
    M, F, K = 40, 256, 256
    aq, bq = _codes(rng, (M, K)), _codes(rng, (2 * F, K))
    as_ = rng.uniform(1e-3, 1e-2, size=(M, 2)).astype(np.float32)
    bs = rng.uniform(1e-3, 1e-2, size=(2 * F // 128, 2)).astype(np.float32)
    h = oracle_lib.swiglu_h_f64(aq, as_, bq, bs)
    y = oracle_lib.bf16_to_f64(oracle_lib.round_bf16(oracle_lib.gemm_f64(aq, as_, bq, bs)))
    gi = [256 * (j // 128) + j % 128 for j in range(F)]
    ui = [256 * (j // 128) + 128 + j % 128 for j in range(F)]
    g = torch.from_numpy(y[:, gi])
    u = torch.from_numpy(y[:, ui])
    ref = (torch.nn.functional.silu(g) * u).numpy()
    assert np.allclose(h, ref, rtol=1e-14, atol=1e-300)


def test_closed_forms(oracle_lib):
    """Codes for -1/0/+1 and unit scales: gate and up are exact integers; h is
    then g / (1 + e^-g) * u from math.exp, and g = 0 gives exactly 0."""
    rng = np.random.default_rng(5)
    M, F, K = 8, 128, 128
    lut = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)
    ia = rng.integers(-1, 2, size=(M, K))
    ib = rng.integers(-1, 2, size=(2 * F, K))
    ib[0, :] = 0                                         # gate column 0 is 0 in every row
    h = oracle_lib.swiglu_h_f64(lut[ia + 1], np.ones((M, 1), np.float32), lut[ib + 1],
                                np.ones((2, 1), np.float32))
    y = ia @ ib.T
    for m in range(M):
        for j in range(F):
            g, u = float(y[m, j]), float(y[m, 128 + j])
            assert math.isclose(h[m, j], g / (1.0 + math.exp(-g)) * u, rel_tol=1e-15, abs_tol=0.0)
    assert (h[:, 0] == 0).all()


def test_quantized_output_is_the_row_quantizer_of_bf16_h(oracle_lib):
    rng = np.random.default_rng(7)
    M, F, K = 16, 256, 128
    aq, bq = _codes(rng, (M, K)), _codes(rng, (2 * F, K))
    as_ = rng.uniform(1e-3, 1e-2, size=(M, 1)).astype(np.float32)
    bs = rng.uniform(1e-3, 1e-2, size=(4, 1)).astype(np.float32)
    for mode in (0, 1):
        q, s = oracle_lib.gemm_swiglu_quant(aq, as_, bq, bs, mode)
        q2, s2 = oracle_lib.quant_act_1x128(oracle_lib.round_bf16(oracle_lib.swiglu_h_f64(aq, as_, bq, bs)), mode)
        assert q.shape == (M, F) and s.shape == (M, F // 128)
        assert np.array_equal(q, q2) and np.array_equal(s.view(np.uint32), s2.view(np.uint32))
