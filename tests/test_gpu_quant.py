"""GPU parity of the activation (1x128) and weight (128x128) quantizers.

The HIP path must reproduce the oracle's E4M3 bytes and fp32 scales bit for
bit (blocks of 1x128 / 128x128, E4M3: page "NVIDIA NeMo RL erreicht 48%
Geschwindigkeitssteigerung ...", section "Der technische Durchbruch"; +-448:
page "FP8 Trainingsinfrastructuur", section "Het landschap van numerieke
precisie").
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (assert_bytes_equal, assert_scales_equal, dev_bf16, host_f32, host_u8,
                        lib, require_gpu, say)

pytestmark = pytest.mark.gpu
MODES = (0, 1)


def _act_parity(x_bits, mode, what):
    fp8q = lib()
    say("quant_act", what, x_bits.shape, "mode", mode)
    q, s = fp8q.fp8_quant_act_1x128(dev_bf16(x_bits), mode)
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_act_1x128(x_bits, mode)
    assert_scales_equal(host_f32(s), os_, what + " scales")
    assert_bytes_equal(host_u8(q), oq, what + " bytes")


def _weight_parity(w_bits, mode, what):
    fp8q = lib()
    say("quant_weight", what, w_bits.shape, "mode", mode)
    q, s = fp8q.fp8_quant_weight_128x128(dev_bf16(w_bits), mode)
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_weight_128x128(w_bits, mode)
    assert_scales_equal(host_f32(s), os_, what + " scales")
    assert_bytes_equal(host_u8(q), oq, what + " bytes")


@pytest.mark.parametrize("mode", MODES)
def test_tiny_config(mode):
    require_gpu()
    x, w = synth.tiny_inputs()
    _act_parity(synth.bf16_bits(x), mode, "tiny X")
    _weight_parity(synth.bf16_bits(w), mode, "tiny W")


def _exhaustive_blocks():
    """One 1x128 block per row: element 0 is amax (every positive finite bf16,
    subnormals included), the other 127 slots walk through every bf16 x with
    |x| <= amax, both signs (padding slots hold +0).  ~1.07e9 (x, amax) pairs."""
    rows = []
    for a in range(1, 0x7F80):
        xs = np.arange(0, a + 1, dtype=np.uint16)
        vals = np.concatenate([xs, xs | np.uint16(0x8000)])
        nb = -(-vals.size // 127)
        blk = np.zeros((nb, 128), dtype=np.uint16)
        blk[:, 0] = a
        flat = blk[:, 1:].reshape(-1)
        flat[: vals.size] = vals
        blk[:, 1:] = flat.reshape(nb, 127)
        rows.append(blk)
    return np.concatenate(rows)


@pytest.fixture(scope="module")
def exhaustive_input():
    return _exhaustive_blocks()


_EXHAUSTIVE_ORACLE = {}


def _exhaustive_oracle(x_bits, mode):
    """The oracle's codes and scales of the exhaustive input (computed once
    per mode and shared by the tests below)."""
    if mode not in _EXHAUSTIVE_ORACLE:
        _EXHAUSTIVE_ORACLE[mode] = oracle.quant_act_1x128(x_bits, mode)
    return _EXHAUSTIVE_ORACLE[mode]


@pytest.mark.parametrize("mode", MODES)
def test_exhaustive_element_rule(exhaustive_input, mode):
    """The byte of an element depends only on (x, amax of its block); this
    covers every such pair of bf16 values, i.e. the whole element rule,
    including the blocks that take the exact-division path."""
    require_gpu()
    fp8q = lib()
    say("quant_act exhaustive (x, amax)", exhaustive_input.shape, "mode", mode)
    q, s = fp8q.fp8_quant_act_1x128(dev_bf16(exhaustive_input), mode)
    torch.cuda.synchronize()
    oq, os_ = _exhaustive_oracle(exhaustive_input, mode)
    assert_scales_equal(host_f32(s), os_, "exhaustive scales")
    assert_bytes_equal(host_u8(q), oq, "exhaustive bytes")


@pytest.mark.parametrize("mode", MODES)
def test_exhaustive_element_rule_dual(exhaustive_input, mode):
    """The same sweep through the two-layout quantizer's row blocks, whose
    blocks with a normal scale convert without the explicit +-448 clamp: every
    (x, amax) pair gives the 1x128 quantizer's byte and scale."""
    require_gpu()
    fp8q = lib()
    say("quant_act_dual exhaustive (x, amax)", exhaustive_input.shape, "mode", mode)
    q, s, _, _ = fp8q.fp8_quant_act_dual(dev_bf16(exhaustive_input), mode, rowwise=True)
    torch.cuda.synchronize()
    oq, os_ = _exhaustive_oracle(exhaustive_input, mode)
    assert_scales_equal(host_f32(s), os_, "exhaustive dual scales")
    assert_bytes_equal(host_u8(q), oq, "exhaustive dual bytes")


@pytest.mark.parametrize("mode", MODES)
def test_special_blocks(mode):
    require_gpu()
    rng = np.random.default_rng(123)
    torch.manual_seed(123)
    rows = np.zeros((12, 256), dtype=np.uint16)
    rows[1, :] = 0x8000                                       # -0.0 everywhere
    rows[2, :] = rng.integers(1, 0x80, 256).astype(np.uint16)  # subnormals
    rows[2, ::5] |= 0x8000
    rows[3, :] = 0x7F7F                                        # bf16 max
    rows[3, 1::2] = 0xFF7F
    rows[4, :] = synth.bf16_bits(torch.linspace(-448, 448, 256).to(torch.bfloat16))
    rows[5, :] = synth.bf16_bits(torch.full((256,), 1e-35).to(torch.bfloat16))    # amax < 2^-100
    rows[5, 7] = 0x8001
    rows[6, :] = synth.bf16_bits((torch.randn(256) * 1e30).to(torch.bfloat16))
    rows[7, :128] = 0x0001                                     # min subnormal block
    rows[8, :] = synth.bf16_bits(torch.randn(256).to(torch.bfloat16))
    rows[8, 3] = synth.bf16_bits(torch.tensor([3.0e4]).to(torch.bfloat16))[0]     # one large outlier
    rows[9, :] = synth.bf16_bits((torch.randn(256) * 2.0 ** -110).to(torch.bfloat16))
    rows[10, :] = synth.bf16_bits((torch.randn(256) * 2.0 ** -101).to(torch.bfloat16))
    rows[11, :] = synth.bf16_bits((torch.randn(256) * 2.0 ** 100).to(torch.bfloat16))
    _act_parity(rows, mode, "special blocks")
    # one 128x128 weight tile per special pattern: tile j repeats row j's first
    # 128 values, rotated by one more position on every row
    tiles = [np.stack([np.roll(rows[j, :128], i) for i in range(128)]) for j in range(rows.shape[0])]
    _weight_parity(np.ascontiguousarray(np.concatenate(tiles, axis=1)), mode, "special tiles")


@pytest.mark.parametrize("M", [1, 7, 33, 257])
def test_ragged_rows(M):
    require_gpu()
    x = synth.normal_bf16((M, 384), 1.0, synth.seed_of(9, M, 0))
    _act_parity(synth.bf16_bits(x), 0, f"ragged M={M}")


def test_empty_input_is_noop():
    require_gpu()
    fp8q = lib()
    x = torch.empty((0, 256), dtype=torch.bfloat16, device="cuda")
    q, s = fp8q.fp8_quant_act_1x128(x)
    assert q.shape == (0, 256) and s.shape == (0, 2)


@pytest.mark.parametrize("layer", range(4))
def test_llama_activation_full_size(layer):
    """Full-size activations of the four Llama-3.1-8B-shaped layers at 4096
    tokens (1% outlier channels x20), bit-exact over every element."""
    require_gpu()
    x, _ = synth.llama_layer_inputs(layer, device="cuda")
    _act_parity(synth.bf16_bits(x), 0, f"llama act {synth.LLAMA_LAYERS[layer][0]}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("kind", range(4))
def test_recalibration_weights_full_size(mode, kind):
    """Full-size weights of the recalibration pass (layer 0 and layer 31 of the
    32-layer Llama-3.1-8B shape), both scale modes, bit-exact."""
    require_gpu()
    for layer in (0, 31):
        w = synth.llama_weight(layer, kind, device="cuda")
        _weight_parity(synth.bf16_bits(w), mode, f"recal L{layer} {synth.LLAMA_LAYERS[kind][0]}")


def test_outputs_stay_in_bounds_and_deterministic():
    """Guard bytes past the outputs stay untouched; two calls give identical bits."""
    require_gpu()
    fp8q = lib()
    M, K = 77, 640
    x = synth.normal_bf16((M, K), 1.0, synth.seed_of(9, 1, 1), device="cuda")
    qbuf = torch.full((M * K + 4096,), 0xA5, dtype=torch.uint8, device="cuda")
    sbuf = torch.full((M * K // 128 + 1024,), -7.0, dtype=torch.float32, device="cuda")
    q = qbuf[: M * K].view(M, K)
    s = sbuf[: M * K // 128].view(M, K // 128)
    fp8q.fp8_quant_act_1x128(x, out=(q, s))
    q2, s2 = fp8q.fp8_quant_act_1x128(x)
    torch.cuda.synchronize()
    assert torch.all(qbuf[M * K:] == 0xA5) and torch.all(sbuf[M * K // 128:] == -7.0)
    assert torch.equal(q, q2) and torch.equal(s.view(torch.int32), s2.view(torch.int32))
    w = synth.normal_bf16((256, 384), 0.02, synth.seed_of(9, 2, 1), device="cuda")
    qw = torch.full((256 * 384 + 4096,), 0x5A, dtype=torch.uint8, device="cuda")
    sw = torch.full((6 + 64,), -3.0, dtype=torch.float32, device="cuda")
    fp8q.fp8_quant_weight_128x128(w, out=(qw[: 256 * 384].view(256, 384), sw[:6].view(2, 3)))
    torch.cuda.synchronize()
    assert torch.all(qw[256 * 384:] == 0x5A) and torch.all(sw[6:] == -3.0)
