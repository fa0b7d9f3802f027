"""Pins of the oracle's fused gate+up GEMM with SwiGLU and output quantization.

The activation's quantization is part of the quantization-kernel overhead the
page blames for the gap to 2x (page "NVIDIA NeMo RL erreicht 48%
Geschwindigkeitssteigerung ...", section "Leistungsgewinne in der
Praxis").  Pins, independent of the functions under test:
  - the 128-block interleave against explicit index arithmetic;
  - h against torch's silu in float64 on the bf16-rounded gate and up taken
    from the plain GEMM by that index arithmetic;
  - closed forms: g = 0 gives 0, exact-integer products give h from math.exp;
  - the quantized output against the pinned row quantizer of bf16(h);
  - the grouped (mixture-of-experts) form against the dense form on each
    group's rows, explicit gathering by index, and a zero row's closed form.
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


# ---------------------------------------------------------------------------
# The grouped (mixture-of-experts) form.  Pins, independent of the code under
# test: the dense oracle above on each group's rows alone (its C GEMM loop is
# a different routine from the grouped one), explicit gathering by index, and
# the closed form of a zero row.
# ---------------------------------------------------------------------------

def _expert_operands(rng, G, F, K, M):
    aq = _codes(rng, (M, K))
    as_ = rng.uniform(1e-3, 1e-2, size=(M, K // 128)).astype(np.float32)
    bq = _codes(rng, (G, 2 * F, K))
    bs = rng.uniform(1e-3, 1e-2, size=(G, 2 * F // 128, K // 128)).astype(np.float32)
    return aq, as_, bq, bs


def test_grouped_equals_dense_per_group(oracle_lib):
    """Ragged groups, one of them empty: every group's rows equal the dense
    fused oracle on those rows with that expert's weight."""
    rng = np.random.default_rng(11)
    G, F, K = 4, 256, 256
    offsets = np.array([0, 37, 37, 140, 205], dtype=np.int32)
    aq, as_, bq, bs = _expert_operands(rng, G, F, K, int(offsets[-1]))
    for mode in (0, 1):
        hq, hs = oracle_lib.grouped_gemm_swiglu_quant(aq, as_, bq, bs, offsets, mode)
        assert hq.shape == (205, F) and hs.shape == (205, F // 128)
        for g in range(G):
            a, b = offsets[g], offsets[g + 1]
            if a == b:
                continue
            dq, ds = oracle_lib.gemm_swiglu_quant(aq[a:b], as_[a:b], bq[g], bs[g], mode)
            assert np.array_equal(hq[a:b], dq) and np.array_equal(hs[a:b], ds), (mode, g)


def test_grouped_gather_by_index(oracle_lib):
    """Routed rows read token rows by index: the result equals the grouped
    oracle on the explicitly gathered rows; an index outside the tokens is a
    zero row, whose h is 0 (codes 0, the all-zero block's scale 1)."""
    rng = np.random.default_rng(12)
    G, F, K, T = 3, 128, 384, 50
    aq, as_, bq, bs = _expert_operands(rng, G, F, K, T)
    idx = rng.integers(0, T, size=90).astype(np.int32)
    idx[[5, 61]] = [-1, T]                                  # outside the token matrix
    offsets = np.array([0, 30, 31, 90], dtype=np.int32)
    hq, hs = oracle_lib.grouped_gemm_swiglu_quant(aq, as_, bq, bs, offsets, 0, row_index=idx)
    gq = np.stack([aq[i] if 0 <= i < T else np.zeros(K, np.uint8) for i in idx])
    gs = np.stack([as_[i] if 0 <= i < T else np.zeros(K // 128, np.float32) for i in idx])
    rq, rs = oracle_lib.grouped_gemm_swiglu_quant(gq, gs, bq, bs, offsets, 0)
    assert np.array_equal(hq, rq) and np.array_equal(hs, rs)
    for r in (5, 61):
        assert (hq[r] == 0).all() and (hs[r] == 1.0).all()


def test_grouped_rows_equal_full(oracle_lib):
    """The sampled-rows form gives the full form's rows."""
    rng = np.random.default_rng(13)
    G, F, K = 3, 128, 256
    offsets = np.array([0, 20, 64, 100], dtype=np.int32)
    aq, as_, bq, bs = _expert_operands(rng, G, F, K, 100)
    hq, hs = oracle_lib.grouped_gemm_swiglu_quant(aq, as_, bq, bs, offsets, 1)
    rows = np.array([0, 19, 20, 63, 64, 99])
    groups = np.searchsorted(offsets, rows, side="right") - 1
    sq, ss = oracle_lib.grouped_gemm_swiglu_quant_rows(aq, as_, bq, bs, groups, rows, 1)
    assert np.array_equal(sq, hq[rows]) and np.array_equal(ss, hs[rows])
