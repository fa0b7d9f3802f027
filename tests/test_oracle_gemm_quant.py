"""Pins of the oracle's GEMM with a quantized output: Y rounded once to bf16,
then quantized in 1x128 blocks along N by the activation-quantization rule
(linear layers in FP8 with 1x128 activation blocks: page "NVIDIA NeMo RL
erreicht 48% Geschwindigkeitssteigerung ...", section "Der technische
Durchbruch"; the quantization of a layer's output for the next one is the
quantization-kernel work that page's section "Leistungsgewinne in der Praxis"
counts as overhead).

Pins: torch's float32 -> bfloat16 conversion (round to nearest even) for
values it represents exactly, a hand-made value where rounding through
float32 first would give a different bf16, the subnormal bf16 grid, and exact
integer GEMMs whose bf16 output is known without the oracle.
"""
import numpy as np
import pytest
import torch


def _torch_bf16_bits(x32):
    t = torch.from_numpy(np.ascontiguousarray(x32.astype(np.float32))).to(torch.bfloat16)
    return t.view(torch.int16).numpy().astype(np.uint16)


def test_round_bf16_matches_torch_on_float32_values(oracle_lib):
    rng = np.random.default_rng(11)
    x = np.concatenate([
        rng.standard_normal(20000) * np.exp2(rng.uniform(-30, 30, 20000)),
        np.exp2(rng.uniform(-140, -120, 2000)) * rng.choice([-1, 1], 2000),   # bf16 subnormals
        (1.0 + (2 * rng.integers(0, 128, 2000) + 1) * 2.0 ** -8) * rng.choice([-1, 1], 2000),  # exact ties
    ]).astype(np.float32)
    assert np.array_equal(oracle_lib.round_bf16(x.astype(np.float64)), _torch_bf16_bits(x))


def test_round_bf16_rounds_once(oracle_lib):
    # 1 + 2^-8 + 2^-40 lies above the tie between 1 and 1 + 2^-7.  Rounded once
    # it goes up (0x3F81); rounded to fp32 first it would become the tie 1 + 2^-8
    # and then go to the even neighbour 1.0 (0x3F80).
    x = np.array([1.0 + 2.0 ** -8 + 2.0 ** -40, -(1.0 + 2.0 ** -8 + 2.0 ** -40)])
    assert list(oracle_lib.round_bf16(x)) == [0x3F81, 0xBF81]
    assert _torch_bf16_bits(x)[0] == 0x3F80  # the double-rounded value, for contrast


def test_round_bf16_subnormal_grid_and_zero_sign(oracle_lib):
    k = np.arange(0, 128)
    x = k * 2.0 ** -133                       # every bf16 subnormal, exactly
    assert np.array_equal(oracle_lib.round_bf16(x), k.astype(np.uint16))
    assert list(oracle_lib.round_bf16(np.array([0.5 * 2.0 ** -133, 1.5 * 2.0 ** -133, -0.0]))) == [0, 2, 0x8000]


def _int_operands(rng, M, N, K):
    # E4M3 codes of -1, 0, +1 (0xB8, 0x00, 0x38) with unit scales: Y is an exact
    # integer with |Y| <= K, so bf16(Y) is exact for K <= 256.
    codes = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)
    vals = np.array([-1, 0, 1])
    ia = rng.integers(0, 3, size=(M, K))
    ib = rng.integers(0, 3, size=(N, K))
    y = vals[ia] @ vals[ib].T
    return codes[ia], np.ones((M, K // 128), np.float32), codes[ib], np.ones((N // 128, K // 128), np.float32), y


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M,N,K", [(5, 128, 128), (33, 384, 256)])
def test_gemm_quant_of_exact_integers(oracle_lib, mode, M, N, K):
    rng = np.random.default_rng(M * 7 + N + mode)
    aq, as_, bq, bs, y = _int_operands(rng, M, N, K)
    q, s = oracle_lib.gemm_quant_1x128(aq, as_, bq, bs, mode)
    # The bf16 output is the integer matrix itself (torch converts it exactly);
    # quantizing it must give the same bytes and scales.
    q_ref, s_ref = oracle_lib.quant_act_1x128(_torch_bf16_bits(y.astype(np.float32)), mode)
    assert np.array_equal(q, q_ref) and np.array_equal(s, s_ref)
    # Closed form of the scales: amax / 448 (amax mode), else the least 2^e with 448 * 2^e >= amax.
    amax = np.abs(y).reshape(M, N // 128, 128).max(axis=2).astype(np.float64)
    if mode == 0:
        want = np.where(amax == 0, 1.0, (amax / 448.0)).astype(np.float32)
    else:
        e = np.ceil(np.log2(np.where(amax == 0, 1.0, amax) / 448.0))
        want = np.where(amax == 0, 1.0, np.exp2(e)).astype(np.float32)
    assert np.array_equal(s, want)


def test_gemm_quant_dequantizes_to_the_product(oracle_lib):
    # Random operands: the dequantized output is within half an E4M3 step of
    # bf16(Y), and the block maximum maps to +-448 in amax mode.
    rng = np.random.default_rng(5)
    M, N, K = 40, 256, 384
    codes = [c for c in range(256) if c not in (0x7F, 0xFF)]
    aq = rng.choice(codes, size=(M, K)).astype(np.uint8)
    bq = rng.choice(codes, size=(N, K)).astype(np.uint8)
    as_ = np.exp2(rng.uniform(-8, 0, size=(M, K // 128))).astype(np.float32)
    bs = np.exp2(rng.uniform(-8, 0, size=(N // 128, K // 128))).astype(np.float32)
    q, s = oracle_lib.gemm_quant_1x128(aq, as_, bq, bs, 0)
    yb = oracle_lib.round_bf16(oracle_lib.gemm_f64(aq, as_, bq, bs))
    ybf = (yb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dec = torch.from_numpy(q).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    deq = dec * np.repeat(s.astype(np.float64), 128, axis=1)
    # E4M3 has 3 mantissa bits: half a step is 2^-4 of the value (2^-10 * s below 2^-6 * s).
    tol = np.maximum(np.abs(ybf) * 2.0 ** -4, np.repeat(s.astype(np.float64), 128, axis=1) * 2.0 ** -10) * 1.0001
    assert np.all(np.abs(deq - ybf) <= tol)
    assert np.all(np.abs(dec).reshape(M, N // 128, 128).max(axis=2) == 448.0)
