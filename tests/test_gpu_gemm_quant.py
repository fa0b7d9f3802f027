"""GPU parity of the GEMM whose epilogue quantizes its output for the next FP8
layer (E4M3, 1x128 blocks along N; activation blocks from page "NVIDIA NeMo
RL erreicht 48% Geschwindigkeitssteigerung ...", section "Der technische
Durchbruch"; the separate quantization pass it replaces is the
quantization-kernel overhead named in section "Leistungsgewinne in der
Praxis").

Per case:
  1. Bit-exact: bytes and scales equal the oracle's activation quantizer applied
     to the bf16 output of fp8_blockscaled_gemm on the same inputs (the two GPU
     entry points share one main loop, so their bf16 outputs are identical; the
     check pins the fused block max, scale and element rule to the oracle).
  2. Against the oracle's own composition: the dequantized output lies within
     half an E4M3 step of the GPU's bf16 Y, which is within the GEMM tolerance
     of the fp64 oracle (checked by the GEMM tests and again here).
  3. Exact-integer products: equal to the oracle composition bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (assert_bytes_equal, assert_scales_equal, gemm_tolerance_check, host_f32, host_u8,
                        lib, require_gpu, say)

pytestmark = pytest.mark.gpu

MODES = {0: "amax", 1: "pow2"}


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def _operands(M, N, K, seed, outliers=0.01):
    x = synth.normal_bf16((M, K), 1.0, synth.seed_of(12, seed, 0), outlier_frac=outliers)
    w = synth.normal_bf16((N, K), 0.02, synth.seed_of(12, seed, 1))
    aq, as_ = oracle.quant_act_1x128(synth.bf16_bits(x))
    bq, bs = oracle.quant_weight_128x128(synth.bf16_bits(w))
    return aq, as_, bq, bs


def _run(aq, as_, bq, bs, mode):
    fp8q = lib()
    args = (_dev_u8(aq), _dev_f32(as_), _dev_u8(bq), _dev_f32(bs))
    yq, ys = fp8q.fp8_blockscaled_gemm_quant(*args, mode=MODES[mode])
    y = fp8q.fp8_blockscaled_gemm(*args)
    torch.cuda.synchronize()
    ybits = y.detach().to("cpu").contiguous().view(torch.int16).numpy().view(np.uint16)
    return host_u8(yq), host_f32(ys), ybits


def _dequant(q, s):
    dec = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return dec * np.repeat(s.astype(np.float64), 128, axis=1)


def _check_half_step(q, s, ybits, what):
    ybf = (ybits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    tol = np.maximum(np.abs(ybf) * 2.0 ** -4, srep * 2.0 ** -10) * (1 + 1e-6)
    bad = np.flatnonzero(np.abs(_dequant(q, s) - ybf).reshape(-1) > tol.reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} elements beyond half an E4M3 step"


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M,N,K", [
    (256, 256, 512), (1, 128, 128), (129, 384, 256), (300, 640, 384), (1000, 1280, 1024), (257, 2816, 640),
])
def test_fused_output_quantization(M, N, K, mode):
    require_gpu()
    aq, as_, bq, bs = _operands(M, N, K, seed=M + 3 * N + 7 * K + mode)
    say("gemm_quant", M, N, K, MODES[mode])
    q, s, ybits = _run(aq, as_, bq, bs, mode)
    q_ref, s_ref = oracle.quant_act_1x128(ybits, mode)
    assert_bytes_equal(q, q_ref, f"{M}x{N}x{K} bytes")
    assert_scales_equal(s, s_ref, f"{M}x{N}x{K} scales")
    gemm_tolerance_check((ybits.astype(np.uint32) << 16).view(np.float32), oracle.gemm_f64(aq, as_, bq, bs),
                         f"{M}x{N}x{K} bf16 Y")
    _check_half_step(q, s, ybits, f"{M}x{N}x{K}")


@pytest.mark.parametrize("mode", [0, 1])
def test_fused_exact_integer_products(mode):
    require_gpu()
    rng = np.random.default_rng(9 + mode)
    M, N, K = 200, 512, 256
    codes = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)   # -1, 0, +1
    aq = codes[rng.integers(0, 3, size=(M, K))]
    bq = codes[rng.integers(0, 3, size=(N, K))]
    as_ = np.ones((M, K // 128), np.float32)
    bs = np.ones((N // 128, K // 128), np.float32)
    say("gemm_quant exact", M, N, K, MODES[mode])
    q, s, _ = _run(aq, as_, bq, bs, mode)
    q_ref, s_ref = oracle.gemm_quant_1x128(aq, as_, bq, bs, mode)
    assert_bytes_equal(q, q_ref, "exact bytes")
    assert_scales_equal(s, s_ref, "exact scales")


@pytest.mark.parametrize("mode", [0, 1])
def test_fused_llama_qkv_panel_split(mode):
    # The QKV projection at 4096 tokens: 16 weight panels on 256-row tiles and
    # 8 on 128-row tiles (8 waves, each holding half of a 1x128 block), one
    # launch into column slices of the codes and scales.  Whole output, bit
    # for bit against quantizing the bf16 output.
    require_gpu()
    M, N, K = 4096, 6144, 4096
    rows, big = lib().fp8_blockscaled_gemm_tile_plan(M, N)
    assert rows == M and 0 < big < N // 256, (rows, big)
    aq, as_, bq, bs = _operands(M, N, K, seed=43 + mode)
    say("gemm_quant qkv split", M, N, K, MODES[mode], rows, big)
    q, s, ybits = _run(aq, as_, bq, bs, mode)
    q_ref, s_ref = oracle.quant_act_1x128(ybits, mode)
    assert_bytes_equal(q, q_ref, "qkv bytes")
    assert_scales_equal(s, s_ref, "qkv scales")
    _check_half_step(q, s, ybits, "qkv")
    rows = np.arange(3, M, 89)
    cols = np.concatenate([np.arange(7, N, 61), [big * 256 - 1, big * 256, N - 1]])
    ms, ns = np.meshgrid(rows, cols, indexing="ij")
    ref = oracle.gemm_sampled_f64(aq, as_, bq, bs, ms.reshape(-1), ns.reshape(-1))
    ybf = (ybits.astype(np.uint32) << 16).view(np.float32)[ms.reshape(-1), ns.reshape(-1)]
    gemm_tolerance_check(ybf, ref, "qkv sampled bf16 Y", frob=2e-3)


@pytest.mark.parametrize("mode", [0, 1])
def test_fused_llama_o_full_size(mode):
    # The Llama-3.1-8B O projection at 4096 tokens (256x256 tiles, one per CU).
    require_gpu()
    M, N, K = 4096, 4096, 4096
    aq, as_, bq, bs = _operands(M, N, K, seed=41 + mode)
    say("gemm_quant full", M, N, K, MODES[mode])
    q, s, ybits = _run(aq, as_, bq, bs, mode)
    q_ref, s_ref = oracle.quant_act_1x128(ybits, mode)
    assert_bytes_equal(q, q_ref, "full bytes")
    assert_scales_equal(s, s_ref, "full scales")
    _check_half_step(q, s, ybits, "full")
    rows = np.arange(0, M, 97)
    cols = np.arange(5, N, 131)
    ms, ns = np.meshgrid(rows, cols, indexing="ij")
    ref = oracle.gemm_sampled_f64(aq, as_, bq, bs, ms.reshape(-1), ns.reshape(-1))
    ybf = (ybits.astype(np.uint32) << 16).view(np.float32)[ms.reshape(-1), ns.reshape(-1)]
    gemm_tolerance_check(ybf, ref, "full sampled bf16 Y", frob=2e-3)


@pytest.mark.parametrize("mode", [0, 1])
def test_fused_split_by_token_rows(mode):
    """A shape that the tile plan splits by token rows (6144 x 4096: rows
    0..4095 on 256-row tiles, the rest on 128-row tiles of 8 waves, one
    launch), and a ragged one split by weight panels with a half last panel
    (4000 x 6016): the whole output bit for bit against quantizing the bf16
    output, and sampled bf16 values against the oracle."""
    require_gpu()
    for M, N, K in ((6144, 4096, 512), (4000, 6016, 384)):
        rows, big = lib().fp8_blockscaled_gemm_tile_plan(M, N)
        assert (rows, big) != (M, (N + 255) // 256) and rows > 0, (M, N, rows, big)
        aq, as_, bq, bs = _operands(M, N, K, seed=M + N + mode)
        say("gemm_quant split", M, N, K, MODES[mode], rows, big)
        q, s, ybits = _run(aq, as_, bq, bs, mode)
        q_ref, s_ref = oracle.quant_act_1x128(ybits, mode)
        assert_bytes_equal(q, q_ref, f"{M}x{N} bytes")
        assert_scales_equal(s, s_ref, f"{M}x{N} scales")
        _check_half_step(q, s, ybits, f"{M}x{N}")
        ms = np.concatenate([np.arange(5, M, 97), [rows - 1, rows, M - 1]])
        ns = np.concatenate([np.arange(3, N, 53), [N - 1]])
        mm, nn = np.meshgrid(ms[ms < M], ns, indexing="ij")
        ref = oracle.gemm_sampled_f64(aq, as_, bq, bs, mm.reshape(-1), nn.reshape(-1))
        ybf = (ybits.astype(np.uint32) << 16).view(np.float32)[mm.reshape(-1), nn.reshape(-1)]
        gemm_tolerance_check(ybf, ref, f"{M}x{N} sampled bf16 Y")
