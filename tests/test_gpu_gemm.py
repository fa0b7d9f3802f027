"""GPU parity of the block-scaled FP8 GEMM (dense) against the fp64 oracle.

Tolerance: |Y_gpu - Y_ref| <= 8e-3*|Y_ref| + 1e-3*rms(Y_ref) element-wise and
relative Frobenius error <= 2e-3 (bf16 output rounding alone costs ~1.7e-3 of
the latter).  Exact-integer products must match bit for bit.  Linear layers
in FP8 with 1x128 / 128x128 scale blocks: page "NVIDIA NeMo RL erreicht 48%
Geschwindigkeitssteigerung ...", section "Der technische Durchbruch".
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (gemm_tolerance_check, host_bf16_as_f64, lib, require_gpu, say)

pytestmark = pytest.mark.gpu


def _dev_u8(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to("cuda:0")


def _run_gemm(aq, as_, bq, bs):
    fp8q = lib()
    y = fp8q.fp8_blockscaled_gemm(_dev_u8(aq), _dev_f32(as_), _dev_u8(bq), _dev_f32(bs))
    torch.cuda.synchronize()
    return host_bf16_as_f64(y)


def _quantized(M, N, K, seed, xstd=1.0, wstd=0.02, outliers=0.0, mode=0):
    x = synth.normal_bf16((M, K), xstd, synth.seed_of(10, seed, 0), outlier_frac=outliers)
    w = synth.normal_bf16((N, K), wstd, synth.seed_of(10, seed, 1))
    aq, as_ = oracle.quant_act_1x128(synth.bf16_bits(x), mode)
    bq, bs = oracle.quant_weight_128x128(synth.bf16_bits(w), mode)
    return aq, as_, bq, bs


def test_tiny_config():
    require_gpu()
    x, w = synth.tiny_inputs()
    aq, as_ = oracle.quant_act_1x128(synth.bf16_bits(x))
    bq, bs = oracle.quant_weight_128x128(synth.bf16_bits(w))
    say("gemm tiny 256x256x512")
    y = _run_gemm(aq, as_, bq, bs)
    ref = oracle.gemm_f64(aq, as_, bq, bs)
    gemm_tolerance_check(y, ref, "tiny")


@pytest.mark.parametrize("M,N,K", [
    (1, 128, 128), (17, 256, 384), (128, 256, 128), (129, 384, 256), (300, 640, 1024),
    (255, 512, 640), (513, 1280, 256), (64, 2816, 1408),
])
def test_shapes_and_ragged_tails(M, N, K):
    require_gpu()
    aq, as_, bq, bs = _quantized(M, N, K, seed=M * 31 + N + K, outliers=0.01)
    say("gemm", M, N, K)
    y = _run_gemm(aq, as_, bq, bs)
    ref = oracle.gemm_f64(aq, as_, bq, bs)
    gemm_tolerance_check(y, ref, f"{M}x{N}x{K}")


@pytest.mark.parametrize("pow2", [False, True])
def test_exact_integer_products(pow2):
    """Codes for -1, 0, +1 with power-of-two scales: every partial sum is an
    exact small dyadic number, so fp32 accumulation and the bf16 rounding of
    |Y| <= 256 are exact -- the GPU must match the integer product bit for bit."""
    require_gpu()
    rng = np.random.default_rng(17 + pow2)
    M, N, K = 200, 384, 256
    lut = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)
    ia = rng.integers(-1, 2, size=(M, K))
    ib = rng.integers(-1, 2, size=(N, K))
    as_ = np.ones((M, K // 128), np.float32)
    bs = np.ones((N // 128, K // 128), np.float32)
    if pow2:
        as_ *= np.float32(2.0 ** -3)
        bs *= np.float32(2.0 ** 3)
    say("gemm exact integers pow2", pow2)
    y = _run_gemm(lut[ia + 1], as_, lut[ib + 1], bs)
    assert np.array_equal(y, (ia @ ib.T).astype(np.float64))


def test_row_permutation_equivariance():
    require_gpu()
    aq, as_, bq, bs = _quantized(384, 512, 512, seed=5)
    perm = np.random.default_rng(5).permutation(384)
    say("gemm permutation")
    y = _run_gemm(aq, as_, bq, bs)
    yp = _run_gemm(aq[perm], as_[perm], bq, bs)
    assert np.array_equal(yp, y[perm])


def test_deterministic_and_in_bounds():
    require_gpu()
    fp8q = lib()
    aq, as_, bq, bs = _quantized(130, 384, 256, seed=6)
    A, AS, B, BS = _dev_u8(aq), _dev_f32(as_), _dev_u8(bq), _dev_f32(bs)
    ybuf = torch.full((130 * 384 + 2048,), 7.5, dtype=torch.bfloat16, device="cuda")
    y1 = fp8q.fp8_blockscaled_gemm(A, AS, B, BS, out=ybuf[: 130 * 384].view(130, 384))
    y2 = fp8q.fp8_blockscaled_gemm(A, AS, B, BS)
    torch.cuda.synchronize()
    assert torch.equal(y1.view(torch.int16), y2.view(torch.int16))
    assert torch.all(ybuf[130 * 384:] == 7.5)


@pytest.mark.parametrize("layer", range(4))
def test_llama_layers_full_size_sampled(layer):
    """Full-size Llama-3.1-8B-shaped layers (4096 tokens), in the configuration
    the benchmark times: quantized on the GPU, multiplied on the GPU, checked
    on sampled outputs (whole rows and scattered elements) against the oracle
    applied to the GPU's own quantized operands -- whose bytes the quantizer
    tests pin to the oracle."""
    require_gpu()
    fp8q = lib()
    name, N, K = synth.LLAMA_LAYERS[layer]
    x, w = synth.llama_layer_inputs(layer, device="cuda")
    say("gemm llama", name, x.shape, w.shape)
    aq, as_ = fp8q.fp8_quant_act_1x128(x)
    bq, bs = fp8q.fp8_quant_weight_128x128(w)
    y = fp8q.fp8_blockscaled_gemm(aq, as_, bq, bs)
    torch.cuda.synchronize()
    haq, has = aq.cpu().numpy(), as_.cpu().numpy()
    hbq, hbs = bq.cpu().numpy(), bs.cpu().numpy()
    # the GPU quantization must equal the oracle's on these inputs as well
    oaq, oas = oracle.quant_act_1x128(synth.bf16_bits(x))
    assert np.array_equal(haq, oaq) and np.array_equal(has.view(np.uint32), oas.view(np.uint32))
    rng = np.random.default_rng(layer)
    M = x.shape[0]
    rows = np.concatenate([[0, 1, 127, 128, M - 1], rng.choice(M, 3, replace=False)])
    ms = np.repeat(rows, N)
    ns = np.tile(np.arange(N), rows.size)
    ms = np.concatenate([ms, rng.integers(0, M, 20000)])
    ns = np.concatenate([ns, rng.integers(0, N, 20000)])
    ref = oracle.gemm_sampled_f64(haq, has, hbq, hbs, ms, ns)
    got = y.float().cpu().numpy().astype(np.float64)[ms, ns]
    gemm_tolerance_check(got, ref, f"llama {name} sampled")


@pytest.mark.parametrize("M,N,K", [
    (300, 32640, 128), (300, 32640, 256), (257, 32768, 384), (513, 16512, 640), (4096, 4096, 1408),
])
def test_wide_shapes_ragged(M, N, K):
    """Shapes with at least 256 output tiles of 256 x 256 (the configuration of
    the large-M kernel): ragged token and weight tiles, 1, 2, 3, 5 and 11 K
    blocks (every remainder of the three-block main loop)."""
    require_gpu()
    aq, as_, bq, bs = _quantized(M, N, K, seed=M + N + K, outliers=0.01)
    say("gemm wide", M, N, K)
    y = _run_gemm(aq, as_, bq, bs)
    rng = np.random.default_rng(M + N)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, M - 1], rng.integers(0, M, 6)]))
    ms = np.concatenate([np.repeat(rows, N), rng.integers(0, M, 20000)])
    ns = np.concatenate([np.tile(np.arange(N), rows.size), rng.integers(0, N, 20000)])
    ref = oracle.gemm_sampled_f64(aq, as_, bq, bs, ms, ns)
    gemm_tolerance_check(y[ms, ns], ref, f"{M}x{N}x{K}")


@pytest.mark.parametrize("variant", ["amax", "pow2", "per_row_scales"])
def test_split_by_weight_panels(variant):
    """Shapes whose 256x256 tiles would leave a partly empty last round are
    split by weight panels: the first panels on 256-row tiles, the rest on
    128-row tiles, as two launches into column slices of Y (4000 x 6016:
    16 panels + 7.5 panels, ragged tokens and a half last panel).  Whole rows
    and scattered elements against the oracle, for the amax and power-of-two
    GEMMs and for the GEMM with one scale per row on both operands."""
    require_gpu()
    fp8q = lib()
    M, N, K = 4000, 6016, 256
    mode = 1 if variant == "pow2" else 0
    if variant == "per_row_scales":
        x = synth.normal_bf16((M, K), 1.0, synth.seed_of(10, 77, 0), outlier_frac=0.01)
        w = synth.normal_bf16((N, K), 0.02, synth.seed_of(10, 77, 1))
        aq, as_ = oracle.quant_act_1x128(synth.bf16_bits(x))
        bq, bs = oracle.quant_act_1x128(synth.bf16_bits(w))
    else:
        aq, as_, bq, bs = _quantized(M, N, K, seed=77, outliers=0.01, mode=mode)
    fn = {"amax": fp8q.fp8_blockscaled_gemm, "pow2": fp8q.fp8_blockscaled_gemm_pow2,
          "per_row_scales": fp8q.fp8_blockscaled_gemm_wgrad}[variant]
    say("gemm split by panels", variant, M, N, K)
    y = fn(_dev_u8(aq), _dev_f32(as_), _dev_u8(bq), _dev_f32(bs))
    torch.cuda.synchronize()
    y = host_bf16_as_f64(y)
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([[0, 1, 255, 256, 3999], rng.integers(0, M, 5)]))
    ms = np.concatenate([np.repeat(rows, N), rng.integers(0, M, 20000)])
    ns = np.concatenate([np.tile(np.arange(N), rows.size), rng.integers(0, N, 20000)])
    if variant == "per_row_scales":
        ref = oracle.gemm_wgrad_sampled_f64(aq, as_, bq, bs, ms, ns)
    else:
        ref = oracle.gemm_sampled_f64(aq, as_, bq, bs, ms, ns)
    gemm_tolerance_check(y[ms, ns], ref, f"split {variant}")


@pytest.mark.parametrize("M,N,K", [(2048, 6144, 256), (2048, 4096, 384), (2000, 4096, 128)])
def test_tile_choice_at_2048_tokens(M, N, K):
    """At 2048 tokens the tile shape follows the estimated rounds: QKV-wide
    outputs (192 tiles of 256 x 256, one round) on 256-row tiles, O-wide ones
    (128 such tiles) on 128-row tiles.  Whole rows and scattered elements
    against the oracle."""
    require_gpu()
    aq, as_, bq, bs = _quantized(M, N, K, seed=M + 3 * N + K, outliers=0.01)
    say("gemm tile choice", M, N, K)
    y = _run_gemm(aq, as_, bq, bs)
    rng = np.random.default_rng(M + N + K)
    rows = np.unique(np.concatenate([[0, 127, 128, 255, 256, M - 1], rng.integers(0, M, 5)]))
    ms = np.concatenate([np.repeat(rows, N), rng.integers(0, M, 20000)])
    ns = np.concatenate([np.tile(np.arange(N), rows.size), rng.integers(0, N, 20000)])
    ref = oracle.gemm_sampled_f64(aq, as_, bq, bs, ms, ns)
    gemm_tolerance_check(y[ms, ns], ref, f"{M}x{N}x{K}")
