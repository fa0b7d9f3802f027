"""GPU parity of RMS normalization fused with the 1x128 quantization of its
output (activation blocks: page "NVIDIA NeMo RL erreicht 48%
Geschwindigkeitssteigerung ...", section "Der technische Durchbruch"; the
separate quantization pass it replaces is overhead named in section
"Leistungsgewinne in der Praxis").

The kernel forms y in fp32 (sum of squares, 1/sqrt, two products); the oracle
forms it exactly.  Their bf16 roundings agree except where y lies within a few
fp32 ulp of a bf16 midpoint, and only such a change can move a code.  Per
case: at most 5e-4 of the bytes and 2e-3 of the scales differ from the
oracle's, every dequantized value is within one E4M3 step of the oracle's, and
within half a step (plus one bf16 ulp) of the exact y.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import dev_bf16, host_f32, host_u8, lib, require_gpu, say

pytestmark = pytest.mark.gpu

MODES = {0: "amax", 1: "pow2"}


def _inputs(M, K, seed, std=1.0, small_rows=True):
    x = synth.normal_bf16((M, K), std, synth.seed_of(29, seed, 0), outlier_frac=0.01)
    if small_rows and M > 1:
        x[M // 2:] *= 1e-3                      # rows where eps matters
    g = synth.normal_bf16((K,), 0.3, synth.seed_of(29, seed, 1)).float() + 1.0
    return synth.bf16_bits(x), synth.bf16_bits(g.to(torch.bfloat16))


def _run(xb, gb, eps, mode):
    fp8q = lib()
    q, s = fp8q.fp8_rmsnorm_quant_1x128(dev_bf16(xb), dev_bf16(gb), eps, MODES[mode])
    torch.cuda.synchronize()
    return host_u8(q), host_f32(s)


def _dequant(q, s):
    dec = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return dec * np.repeat(np.asarray(s, np.float64), 128, axis=1)


def _check(q, s, xb, gb, eps, mode, what):
    q_ref, s_ref = oracle.rmsnorm_quant_1x128(xb, gb, eps, mode)
    n_bytes = int(np.count_nonzero(q != q_ref))
    n_scales = int(np.count_nonzero(s.view(np.uint32) != s_ref.view(np.uint32)))
    assert n_bytes <= max(4, 5e-4 * q.size), f"{what}: {n_bytes} of {q.size} bytes differ"
    assert n_scales <= max(2, 2e-3 * s.size), f"{what}: {n_scales} of {s.size} scales differ"
    a, b = _dequant(q, s), _dequant(q_ref, s_ref)
    smax = np.repeat(np.maximum(s, s_ref).astype(np.float64), 128, axis=1)
    step = (2.0 ** -3 + 2.0 ** -7) * np.maximum(np.abs(a), np.abs(b)) + 2.0 ** -9 * smax
    bad = np.flatnonzero((np.abs(a - b) > step).reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} values more than one E4M3 step from the oracle's"
    y = oracle.rmsnorm_f64(xb, gb, eps)
    srep = np.repeat(s.astype(np.float64), 128, axis=1)
    half = (2.0 ** -4 + 2.0 ** -8) * np.abs(y) * (1 + 2.0 ** -7) + 2.0 ** -10 * srep
    bad = np.flatnonzero((np.abs(a - y) > half).reshape(-1))
    assert bad.size == 0, f"{what}: {bad.size} values beyond half an E4M3 step of the exact y"


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("M,K", [(1, 128), (7, 256), (300, 384), (129, 640), (1000, 4096), (513, 2048),
                                 (64, 8192), (33, 1152), (2, 7680)])
def test_rmsnorm_quant(M, K, mode):
    require_gpu()
    xb, gb = _inputs(M, K, seed=M + 7 * K + mode)
    for eps in (1e-5, 1e-6):
        say("rmsnorm_quant", M, K, eps, MODES[mode])
        q, s = _run(xb, gb, eps, mode)
        _check(q, s, xb, gb, eps, mode, f"{M}x{K} eps={eps}")


@pytest.mark.parametrize("mode", [0, 1])
def test_rmsnorm_special_rows(mode):
    """A constant row (y = +-gamma exactly with eps = 0), a zero row with
    eps > 0 (codes 0 with the sign of the product, scale 1), a row of one
    outlier among tiny values, and rows of large and of tiny (1e-37) bf16
    values."""
    require_gpu()
    K = 512
    x = np.zeros((6, K), np.float32)
    x[0] = -3.0
    x[2, :] = 1e-6
    x[2, 77] = 50.0
    x[3] = np.linspace(-3e4, 3e4, K)
    x[4] = np.linspace(-1e-37, 1e-37, K)
    x[5] = np.random.default_rng(mode).standard_normal(K)
    xb = synth.bf16_bits(torch.from_numpy(x).to(torch.bfloat16))
    gb = synth.bf16_bits(torch.ones(K, dtype=torch.bfloat16))
    say("rmsnorm special rows", MODES[mode])
    # (row 4's squares underflow fp32: with eps = 0 it is outside the contract)
    q, s = _run(xb[[0, 2, 3, 5]], gb, 0.0, mode)
    _check(q, s, xb[[0, 2, 3, 5]], gb, 0.0, mode, "special rows, eps 0")
    q_ref, s_ref = oracle.rmsnorm_quant_1x128(xb[[0]], gb, 0.0, mode)
    assert np.array_equal(q[0], q_ref[0]) and np.array_equal(s[0], s_ref[0]), "constant row"
    q, s = _run(xb, gb, 1e-5, mode)
    _check(q, s, xb, gb, 1e-5, mode, "special rows, eps 1e-5")
    assert not (q[1] & 0x7F).any() and np.all(s[1] == 1.0), "zero row"


@pytest.mark.parametrize("mode", [0, 1])
def test_rmsnorm_llama_hidden_full_size(mode):
    """The Llama-3.1-8B hidden state at 4096 tokens (K = 4096), every row."""
    require_gpu()
    xb, gb = _inputs(4096, 4096, seed=88 + mode, small_rows=False)
    say("rmsnorm full", MODES[mode])
    q, s = _run(xb, gb, 1e-5, mode)
    _check(q, s, xb, gb, 1e-5, mode, "llama hidden")
