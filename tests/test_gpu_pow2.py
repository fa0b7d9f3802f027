"""GPU parity of the power-of-two-scale GEMMs (fp8_blockscaled_gemm_pow2,
fp8_grouped_gemm_pow2): operands quantized with power-of-two scales (page
"NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung ...", section "Warum
dies fuer die KI-Oekonomie wichtig ist"), whose scales the gfx950 matrix
cores apply as E8M0 block scales.  Same tolerance as the general GEMM; exact
products bit for bit; a scale outside the contract turns exactly the outputs
that depend on it into NaN."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import gemm_tolerance_check, host_bf16_as_f64, lib, require_gpu, say

pytestmark = pytest.mark.gpu
POW2 = oracle.MODE_POW2


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _quantized(M, N, K, seed, outliers=0.01):
    x = synth.normal_bf16((M, K), 1.0, synth.seed_of(12, seed, 0), outlier_frac=outliers)
    w = synth.normal_bf16((N, K), 0.02, synth.seed_of(12, seed, 1))
    aq, as_ = oracle.quant_act_1x128(synth.bf16_bits(x), POW2)
    bq, bs = oracle.quant_weight_128x128(synth.bf16_bits(w), POW2)
    return aq, as_, bq, bs


def _run(aq, as_, bq, bs):
    fp8q = lib()
    y = fp8q.fp8_blockscaled_gemm_pow2(_dev(aq), _dev(as_), _dev(bq), _dev(bs))
    torch.cuda.synchronize()
    return host_bf16_as_f64(y)


@pytest.mark.parametrize("M,N,K", [
    (1, 128, 128), (129, 384, 256), (300, 640, 1024), (513, 1280, 256),
    (300, 32640, 256), (4096, 4096, 640),
])
def test_pow2_gemm_matches_oracle(M, N, K):
    """Both tile configurations (the last two shapes have >= 256 tiles of
    256 x 256), ragged token and weight tiles."""
    require_gpu()
    aq, as_, bq, bs = _quantized(M, N, K, seed=M + N + K)
    say("gemm pow2", M, N, K)
    y = _run(aq, as_, bq, bs)
    if M * N * K <= 2 ** 28:
        gemm_tolerance_check(y, oracle.gemm_f64(aq, as_, bq, bs), f"pow2 {M}x{N}x{K}")
    else:
        rng = np.random.default_rng(M)
        ms, ns = rng.integers(0, M, 40000), rng.integers(0, N, 40000)
        ref = oracle.gemm_sampled_f64(aq, as_, bq, bs, ms, ns)
        gemm_tolerance_check(y[ms, ns], ref, f"pow2 {M}x{N}x{K} sampled")


def test_pow2_exact_products():
    """Codes for -1/0/+1 with scales 2^e (e in [-3, 3], per token row and K
    block, per weight block): every partial sum is a multiple of 2^-6 below
    2^14, so fp32 accumulation is exact and Y is the exact product rounded
    once to bf16 (RNE) -- compared bit for bit."""
    require_gpu()
    rng = np.random.default_rng(31)
    M, N, K = 300, 640, 512
    lut = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)
    ia, ib = rng.integers(-1, 2, size=(M, K)), rng.integers(-1, 2, size=(N, K))
    ea = rng.integers(-3, 4, size=(M, K // 128))
    eb = rng.integers(-3, 4, size=(N // 128, K // 128))
    as_ = np.ldexp(1.0, ea).astype(np.float32)
    bs = np.ldexp(1.0, eb).astype(np.float32)
    exact = (ia * np.repeat(np.ldexp(1.0, ea), 128, axis=1)) @ (ib * np.repeat(np.repeat(np.ldexp(1.0, eb), 128, axis=0), 128, axis=1)).T
    want = torch.from_numpy(exact).float().to(torch.bfloat16).double().numpy()
    say("gemm pow2 exact")
    y = _run(lut[ia + 1], as_, lut[ib + 1], bs)
    assert np.array_equal(y, want)


def test_pow2_agrees_with_general_gemm():
    """On power-of-two inputs the E8M0 path and the general path compute the
    same product (up to summation order)."""
    require_gpu()
    fp8q = lib()
    aq, as_, bq, bs = _quantized(1024, 8192, 1024, seed=77)
    A, AS, B, BS = _dev(aq), _dev(as_), _dev(bq), _dev(bs)
    say("gemm pow2 vs general")
    y1 = fp8q.fp8_blockscaled_gemm_pow2(A, AS, B, BS).double()
    y2 = fp8q.fp8_blockscaled_gemm(A, AS, B, BS).double()
    torch.cuda.synchronize()
    rel = (torch.linalg.norm(y1 - y2) / torch.linalg.norm(y2)).item()
    assert rel <= 2e-3, rel


def test_pow2_invalid_scale_gives_nan_exactly_where_used():
    """A token-row scale of 3 (not a power of two) and a zero weight scale:
    exactly the outputs of that row, and of that weight block, are NaN."""
    require_gpu()
    aq, as_, bq, bs = _quantized(200, 512, 384, seed=5)
    as_ = as_.copy()
    bs = bs.copy()
    as_[17, 1] = 3.0
    bs[2, 0] = 0.0          # weight rows 256..383
    say("gemm pow2 invalid scales")
    y = _run(aq, as_, bq, bs)
    nan = np.isnan(y)
    expect = np.zeros_like(nan)
    expect[17, :] = True
    expect[:, 256:384] = True
    assert np.array_equal(nan, expect)
    keep = ~expect
    ref = oracle.gemm_f64(aq, as_, bq, bs)
    gemm_tolerance_check(y[keep], ref[keep], "pow2 valid outputs")


@pytest.mark.parametrize("sizes,N,K", [
    ([3, 0, 130, 1, 0, 255, 128], 256, 256),
    ([600, 0, 257, 1024, 1, 300, 256], 384, 640),
])
def test_pow2_grouped(sizes, N, K):
    require_gpu()
    fp8q = lib()
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    G, M = len(sizes), int(off[-1])
    x = synth.normal_bf16((M, K), 1.0, synth.seed_of(13, M, 0))
    w = synth.normal_bf16((G, N, K), 0.02, synth.seed_of(13, M, 1))
    aq, as_ = oracle.quant_act_1x128(synth.bf16_bits(x), POW2)
    bq, bs = zip(*[oracle.quant_weight_128x128(synth.bf16_bits(w[g]), POW2) for g in range(G)])
    bq, bs = np.stack(bq), np.stack(bs)
    say("grouped pow2", sizes, N, K)
    y = fp8q.fp8_grouped_gemm_pow2(_dev(aq), _dev(as_), _dev(bq), _dev(bs), _dev(off))
    torch.cuda.synchronize()
    gemm_tolerance_check(host_bf16_as_f64(y), oracle.grouped_gemm_f64(aq, as_, bq, bs, off), f"grouped pow2 {sizes}")


def test_pow2_llama_full_size_sampled():
    """Full-size Llama-3.1-8B gate+up layer, quantized on the GPU in pow2 mode."""
    require_gpu()
    fp8q = lib()
    name, N, K = synth.LLAMA_LAYERS[2]
    x, w = synth.llama_layer_inputs(2, device="cuda")
    say("gemm pow2 llama", name)
    aq, as_ = fp8q.fp8_quant_act_1x128(x, "pow2")
    bq, bs = fp8q.fp8_quant_weight_128x128(w, "pow2")
    y = fp8q.fp8_blockscaled_gemm_pow2(aq, as_, bq, bs)
    torch.cuda.synchronize()
    haq, has, hbq, hbs = aq.cpu().numpy(), as_.cpu().numpy(), bq.cpu().numpy(), bs.cpu().numpy()
    rng = np.random.default_rng(2)
    M = x.shape[0]
    ms, ns = rng.integers(0, M, 30000), rng.integers(0, N, 30000)
    ref = oracle.gemm_sampled_f64(haq, has, hbq, hbs, ms, ns)
    gemm_tolerance_check(y.float().cpu().numpy().astype(np.float64)[ms, ns], ref, "pow2 llama sampled")
