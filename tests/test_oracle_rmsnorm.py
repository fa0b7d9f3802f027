"""Pins of the oracle's RMS normalization with fused 1x128 quantization.

The norms of a Llama/Qwen3 block produce the activations of the QKV and gate+up
projections; quantizing them in the norm's own pass removes one of the
quantization kernels the page counts as overhead (page "NVIDIA NeMo RL erreicht
48% Geschwindigkeitssteigerung ...", section "Leistungsgewinne in der Praxis").
Pins, none of which uses the function under test:
  - torch's rms_norm in float64 on the decoded bf16 values, with eps large
    enough to matter for half of the rows;
  - closed forms: a constant row gives +-gamma; a row of +-1 on half of its
    entries gives +-sqrt(2) gamma; an all-zero row gives zeros;
  - invariants: with eps = 0 the result is unchanged, bit for bit, when x is
    scaled by a power of two; eps shrinks a row by sqrt(ms / (ms + eps));
  - the quantized output against the pinned bf16 rounding and row quantizer
    of torch's result.
"""
import math

import numpy as np
import torch

from tests.test_oracle_quant import _bf16


def _dec(bits):
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _rows(rng, M, K):
    """Rows at two magnitudes: std 1 and std 1e-3 (where eps = 1e-5 matters)."""
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[M // 2:] *= 1e-3
    return _bf16(x)


def test_against_torch_rms_norm(oracle_lib):
    rng = np.random.default_rng(1)
    M, K = 24, 640
    xb = _rows(rng, M, K)
    gb = _bf16((1.0 + 0.1 * rng.standard_normal(K)).astype(np.float32))
    for eps in (1e-5, 1e-6, 0.0):
        y = oracle_lib.rmsnorm_f64(xb, gb, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(_dec(xb)), (K,), weight=torch.from_numpy(_dec(gb)),
                                           eps=float(np.float32(eps))).numpy()
        assert np.allclose(y, ref, rtol=1e-13, atol=0), eps


def test_closed_forms(oracle_lib):
    K = 256
    g = _bf16(np.linspace(0.5, 2.0, K).astype(np.float32))
    gd = _dec(g)
    x = np.zeros((3, K), np.float32)
    x[0] = -3.0                                       # constant row
    x[1, :128] = np.where(np.arange(128) % 2, 1.0, -1.0)  # +-1 on half of the row
    y = oracle_lib.rmsnorm_f64(_bf16(x[:2]), g, 0.0)
    assert np.array_equal(y[0], -gd)
    assert np.allclose(y[1, :128], np.where(np.arange(128) % 2, 1.0, -1.0) * math.sqrt(2.0) * gd[:128],
                       rtol=1e-15, atol=0)
    assert not y[1, 128:].any()
    y = oracle_lib.rmsnorm_f64(_bf16(x), g, 1e-5)      # all-zero row with eps > 0
    assert not y[2].any()
    q, s = oracle_lib.rmsnorm_quant_1x128(_bf16(x), g, 1e-5)
    assert not (q[2] & 0x7F).any() and np.all(s[2] == 1.0)


def test_power_of_two_scaling_and_eps(oracle_lib):
    rng = np.random.default_rng(2)
    M, K = 8, 384
    xb = _bf16(rng.standard_normal((M, K)).astype(np.float32))
    gb = _bf16(rng.uniform(0.5, 1.5, K).astype(np.float32))
    y0 = oracle_lib.rmsnorm_f64(xb, gb, 0.0)
    for j in (-20, -3, 5):
        xs = _bf16((_dec(xb) * 2.0 ** j).astype(np.float32))   # exact: bf16 keeps its 8 bits
        assert np.array_equal(oracle_lib.rmsnorm_f64(xs, gb, 0.0), y0), j
    eps = 0.25
    ms = np.mean(_dec(xb) ** 2, axis=1, keepdims=True)
    assert np.allclose(oracle_lib.rmsnorm_f64(xb, gb, eps), y0 * np.sqrt(ms / (ms + eps)), rtol=1e-14, atol=0)


def test_quantized_output_composition(oracle_lib):
    rng = np.random.default_rng(3)
    M, K = 16, 512
    xb = _rows(rng, M, K)
    gb = _bf16(rng.uniform(0.2, 3.0, K).astype(np.float32))
    ref = torch.nn.functional.rms_norm(torch.from_numpy(_dec(xb)), (K,), weight=torch.from_numpy(_dec(gb)),
                                       eps=float(np.float32(1e-5))).numpy()
    for mode in (0, 1):
        q, s = oracle_lib.rmsnorm_quant_1x128(xb, gb, 1e-5, mode)
        q2, s2 = oracle_lib.quant_act_1x128(oracle_lib.round_bf16(ref), mode)
        # torch's float64 result may differ from the oracle's in the last bit;
        # the bf16 rounding hides that except at a rounding midpoint
        assert np.count_nonzero(q != q2) <= 2 and np.count_nonzero(s != s2) <= 1, mode
