"""GPU parity of the backward pass of the FP8 linear layer.

Training runs end to end in FP8 (page "NVIDIA NeMo RL erreicht 48%
Geschwindigkeitssteigerung ...", title and section "Der technische
Durchbruch").  The quantizers that write both layouts must reproduce the
oracle's bytes and scales bit for bit; the data gradient dX = dY W (the dense
GEMM on W's transposed tiles) and the weight gradient dW = dY^T X (1x128 blocks
on both operands, contracted over the tokens) must meet the GEMM tolerance
against the fp64 oracle, and exact-integer products must match bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (assert_bytes_equal, assert_scales_equal, dev_bf16, gemm_tolerance_check,
                        host_bf16_as_f64, host_f32, host_u8, lib, require_gpu, say)

pytestmark = pytest.mark.gpu
MODES = (0, 1)


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _act_dual_parity(x_bits, mode, what, rowwise=True):
    fp8q = lib()
    say("quant_act_dual", what, x_bits.shape, "mode", mode, "rowwise", rowwise)
    q, s, qt, st = fp8q.fp8_quant_act_dual(dev_bf16(x_bits), mode, rowwise=rowwise)
    torch.cuda.synchronize()
    oqt, ost = oracle.quant_act_colwise_t(x_bits, mode)
    assert_scales_equal(host_f32(st), ost, what + " column scales")
    assert_bytes_equal(host_u8(qt), oqt, what + " column bytes")
    if rowwise:
        oq, os_ = oracle.quant_act_1x128(x_bits, mode)
        assert_scales_equal(host_f32(s), os_, what + " row scales")
        assert_bytes_equal(host_u8(q), oq, what + " row bytes")
    else:
        assert q is None and s is None


def _weight_dual_parity(w_bits, mode, what):
    fp8q = lib()
    say("quant_weight_dual", what, w_bits.shape, "mode", mode)
    q, s, qt, st = fp8q.fp8_quant_weight_128x128_dual(dev_bf16(w_bits), mode)
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_weight_128x128(w_bits, mode)
    oqt, ost = oracle.quant_weight_128x128_t(w_bits, mode)
    assert_scales_equal(host_f32(s), os_, what + " scales")
    assert_bytes_equal(host_u8(q), oq, what + " bytes")
    assert_scales_equal(host_f32(st), ost, what + " transposed scales")
    assert_bytes_equal(host_u8(qt), oqt, what + " transposed bytes")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("M,K", [(1, 128), (128, 256), (200, 384), (300, 1024), (1000, 640), (129, 128)])
def test_act_dual_shapes(M, K, mode):
    require_gpu()
    x = synth.normal_bf16((M, K), 1.0, synth.seed_of(13, M, K), outlier_frac=0.01)
    _act_dual_parity(synth.bf16_bits(x), mode, f"{M}x{K}")


def test_act_dual_transposed_only():
    require_gpu()
    x = synth.normal_bf16((333, 512), 1e-3, synth.seed_of(13, 333, 1))
    _act_dual_parity(synth.bf16_bits(x), 0, "333x512 transposed only", rowwise=False)


@pytest.mark.parametrize("mode", MODES)
def test_act_dual_special_columns(mode):
    """Columns that are all -0, bf16 subnormals, bf16 max, below 2^-100 (the
    exact-division path), one huge outlier, and values of 2^100; laid out as
    columns so each is one 128x1 block (and its transposed row)."""
    require_gpu()
    rng = np.random.default_rng(321)
    torch.manual_seed(321)
    cols = np.zeros((256, 10), dtype=np.uint16)
    cols[:, 1] = 0x8000
    cols[:, 2] = rng.integers(1, 0x80, 256).astype(np.uint16)
    cols[::3, 2] |= 0x8000
    cols[:, 3] = 0x7F7F
    cols[1::2, 3] = 0xFF7F
    cols[:, 4] = synth.bf16_bits(torch.linspace(-448, 448, 256).to(torch.bfloat16))
    cols[:, 5] = synth.bf16_bits(torch.full((256,), 1e-35).to(torch.bfloat16))
    cols[9, 5] = 0x8001
    cols[:, 6] = synth.bf16_bits(torch.randn(256).to(torch.bfloat16))
    cols[40, 6] = synth.bf16_bits(torch.tensor([3.0e4]).to(torch.bfloat16))[0]
    cols[:, 7] = synth.bf16_bits((torch.randn(256) * 2.0 ** -110).to(torch.bfloat16))
    cols[:, 8] = synth.bf16_bits((torch.randn(256) * 2.0 ** 100).to(torch.bfloat16))
    cols[:128, 9] = 0x0001
    x = np.zeros((256, 128), dtype=np.uint16)
    x[:, :10] = cols
    x[:, 10:] = synth.bf16_bits(torch.randn(256, 118).to(torch.bfloat16))
    _act_dual_parity(np.ascontiguousarray(x), mode, "special columns")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("N,K", [(128, 128), (256, 384), (384, 1024)])
def test_weight_dual_shapes(N, K, mode):
    require_gpu()
    w = synth.normal_bf16((N, K), 0.02, synth.seed_of(14, N, K))
    _weight_dual_parity(synth.bf16_bits(w), mode, f"{N}x{K}")


def test_weight_dual_equals_plain_weight_quantizer():
    require_gpu()
    fp8q = lib()
    w = synth.llama_weight(0, 1, device="cuda")
    say("weight dual vs plain", w.shape)
    q1, s1 = fp8q.fp8_quant_weight_128x128(w)
    q2, s2, qt, st = fp8q.fp8_quant_weight_128x128_dual(w)
    torch.cuda.synchronize()
    assert torch.equal(q1, q2) and torch.equal(s1.view(torch.int32), s2.view(torch.int32))
    assert torch.equal(qt, q1.t().contiguous()) and torch.equal(st.view(torch.int32), s1.t().contiguous().view(torch.int32))


def _grad_operands(M, N, K, seed, mode=0):
    """Oracle-quantized dY [M, N] (rows and 128-token columns), W [N, K] (tiles
    and transposed tiles) and X [M, K] (128-token columns)."""
    x = synth.normal_bf16((M, K), 1.0, synth.seed_of(15, seed, 0), outlier_frac=0.01)
    w = synth.normal_bf16((N, K), 0.02, synth.seed_of(15, seed, 1))
    g = synth.normal_bf16((M, N), 1e-3, synth.seed_of(15, seed, 2))
    gb, wb, xb = synth.bf16_bits(g), synth.bf16_bits(w), synth.bf16_bits(x)
    ops = dict(g=oracle.quant_act_1x128(gb, mode), gt=oracle.quant_act_colwise_t(gb, mode),
               xt=oracle.quant_act_colwise_t(xb, mode))
    if N % 128 == 0:  # W's tiles exist only for whole 128-row blocks
        ops.update(w=oracle.quant_weight_128x128(wb, mode), wt=oracle.quant_weight_128x128_t(wb, mode))
    return ops


@pytest.mark.parametrize("M,N,K", [(1, 256, 1024), (300, 512, 384), (129, 256, 640), (1000, 384, 1280)])
def test_dgrad(M, N, K):
    """dX [M, K] = dY W: the dense GEMM on W's transposed tiles.  (A single
    row gets 1024 outputs: with only 128, the bf16 rounding of the exact
    result can by itself exceed the 2e-3 Frobenius bar.)"""
    require_gpu()
    fp8q = lib()
    ops = _grad_operands(M, N, K, M + N + K)
    (gq, gs), (wtq, wts) = ops["g"], ops["wt"]
    say("dgrad", M, N, K)
    y = fp8q.fp8_blockscaled_gemm(_dev(gq), _dev(gs), _dev(wtq), _dev(wts))
    torch.cuda.synchronize()
    ref = oracle.gemm_dgrad_f64(gq, gs, *ops["w"])
    gemm_tolerance_check(host_bf16_as_f64(y), ref, f"dgrad {M}x{N}x{K}")


@pytest.mark.parametrize("M,N,K,rows", [(1, 128, 128, None), (300, 256, 384, None), (128, 640, 256, None),
                                        (1000, 384, 512, None), (700, 256, 128, 200), (1200, 256, 384, None)])
def test_wgrad(M, N, K, rows):
    """dW [N, K] = dY^T X over Mp = 128*ceil(M/128) tokens (the ragged tail's
    padding codes are zeros); rows = 200 keeps the first 200 dY^T rows, which
    leaves a partial tile of dW rows.  The kernel loads both scale vectors in
    chunks of four 128-token blocks, two chunk buffers in turn: 1, 3, 6, 8 and
    10 blocks cover a lone partial chunk, a partial second one, two whole ones
    and a third chunk that reuses the first one's buffer."""
    require_gpu()
    fp8q = lib()
    ops = _grad_operands(M, N, K, 3 * M + N + K)
    (gtq, gts), (xtq, xts) = ops["gt"], ops["xt"]
    if rows is not None:
        gtq, gts = gtq[:rows], gts[:rows]
    say("wgrad", M, N, K)
    y = fp8q.fp8_blockscaled_gemm_wgrad(_dev(gtq), _dev(gts), _dev(xtq), _dev(xts))
    torch.cuda.synchronize()
    ref = oracle.gemm_wgrad_f64(gtq, gts, xtq, xts)
    gemm_tolerance_check(host_bf16_as_f64(y), ref, f"wgrad {M}x{N}x{K}")


def test_wgrad_per_row_scales_reach_the_right_rows():
    """Codes for -1/0/+1 and scales 2^e, e drawn per row and block on both
    sides over 21 binades: a scale applied to a wrong row or block changes an
    output by a power of two, far outside the GEMM tolerance."""
    require_gpu()
    fp8q = lib()
    rng = np.random.default_rng(77)
    N, K, Mp = 256, 384, 256
    lut = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)
    ia = rng.integers(-1, 2, size=(N, Mp))
    ib = rng.integers(-1, 2, size=(K, Mp))
    as_ = np.exp2(rng.integers(-20, 1, size=(N, 2))).astype(np.float32)
    bs = np.exp2(rng.integers(-20, 1, size=(K, 2))).astype(np.float32)
    say("wgrad per-row scales")
    y = fp8q.fp8_blockscaled_gemm_wgrad(_dev(lut[ia + 1]), _dev(as_), _dev(lut[ib + 1]), _dev(bs))
    torch.cuda.synchronize()
    ref = oracle.gemm_wgrad_f64(lut[ia + 1], as_, lut[ib + 1], bs)
    gemm_tolerance_check(host_bf16_as_f64(y), ref, "wgrad per-row scales")


@pytest.mark.parametrize("pow2_scales", [False, True])
def test_wgrad_exact_integer_products(pow2_scales):
    require_gpu()
    fp8q = lib()
    rng = np.random.default_rng(55 + pow2_scales)
    N, K, Mp = 256, 384, 256
    lut = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)
    ia = rng.integers(-1, 2, size=(N, Mp))
    ib = rng.integers(-1, 2, size=(K, Mp))
    as_ = np.ones((N, 2), np.float32)
    bs = np.ones((K, 2), np.float32)
    if pow2_scales:   # one power of two per dY row: the output row is scaled exactly
        e = rng.integers(-6, 7, size=(N, 1))
        as_ = np.exp2(np.repeat(e, 2, axis=1)).astype(np.float32)
    say("wgrad exact integers", pow2_scales)
    y = fp8q.fp8_blockscaled_gemm_wgrad(_dev(lut[ia + 1]), _dev(as_), _dev(lut[ib + 1]), _dev(bs))
    torch.cuda.synchronize()
    ref = (ia @ ib.T).astype(np.float64) * as_[:, :1].astype(np.float64)
    assert np.array_equal(host_bf16_as_f64(y), ref)


@pytest.mark.parametrize("layer", [0, 1, 3])
def test_llama_backward_full_size_sampled(layer):
    """Full-size Llama-3.1-8B-shaped QKV (6144x4096), O (4096x4096) and down
    (4096x14336) layers at 4096 tokens: dY ~ N(0, 1e-3), quantized on the GPU
    in both layouts (checked bit for bit on sampled rows against the oracle),
    then dgrad and wgrad checked on sampled outputs against the fp64 oracle,
    with rows on both sides of a split tile plan (QKV's weight gradient runs
    rows 0..4095 on 256-row tiles and 4096..6143 on 128-row tiles)."""
    require_gpu()
    fp8q = lib()
    name, N, K = synth.LLAMA_LAYERS[layer]
    x, w = synth.llama_layer_inputs(layer, device="cuda")
    M = x.shape[0]
    g = synth.normal_bf16((M, N), 1e-3, synth.seed_of(16, layer, 2), device="cuda")
    say("llama backward", name, M, N, K)
    gq, gs, gtq, gts = fp8q.fp8_quant_act_dual(g)
    _, _, xtq, xts = fp8q.fp8_quant_act_dual(x, rowwise=False)
    wq, ws, wtq, wts = fp8q.fp8_quant_weight_128x128_dual(w)
    dx = fp8q.fp8_blockscaled_gemm(gq, gs, wtq, wts)
    dw = fp8q.fp8_blockscaled_gemm_wgrad(gtq, gts, xtq, xts)
    torch.cuda.synchronize()
    rng = np.random.default_rng(layer)
    # the transposed quantization of dY on 64 sampled columns, bit for bit
    cols = np.sort(rng.choice(N, 64, replace=False))
    gcols = synth.bf16_bits(g[:, torch.from_numpy(cols).to("cuda")].contiguous())
    oqt, ost = oracle.quant_act_colwise_t(gcols)
    assert_bytes_equal(host_u8(gtq)[cols], oqt, f"{name} dY column bytes")
    assert_scales_equal(host_f32(gts)[cols], ost, f"{name} dY column scales")
    hgq, hgs, hwq, hws = host_u8(gq), host_f32(gs), host_u8(wq), host_f32(ws)
    ms, ks = rng.integers(0, M, 400), rng.integers(0, K, 400)
    ref = oracle.gemm_dgrad_sampled_f64(hgq, hgs, hwq, hws, ms, ks)
    gemm_tolerance_check(dx.float().cpu().numpy().astype(np.float64)[ms, ks], ref, f"{name} dgrad sampled")
    edge = np.array([0, 4095, 4096, N - 1])
    ns = np.concatenate([rng.integers(0, N, 400), np.repeat(edge[edge < N], 8)])
    ks = rng.integers(0, K, ns.size)
    ref = oracle.gemm_wgrad_sampled_f64(host_u8(gtq), host_f32(gts), host_u8(xtq), host_f32(xts), ns, ks)
    gemm_tolerance_check(dw.float().cpu().numpy().astype(np.float64)[ns, ks], ref, f"{name} wgrad sampled")


@pytest.mark.parametrize("M,N,K,rows", [(300, 256, 384, None), (128, 640, 256, None), (700, 256, 128, 200),
                                        (1200, 256, 384, None)])
def test_wgrad_pow2(M, N, K, rows):
    """Power-of-two scales applied by the matrix cores (per-row E8M0 on both
    operands) against the oracle."""
    require_gpu()
    fp8q = lib()
    ops = _grad_operands(M, N, K, 5 * M + N + K, mode=1)
    (gtq, gts), (xtq, xts) = ops["gt"], ops["xt"]
    if rows is not None:
        gtq, gts = gtq[:rows], gts[:rows]
    say("wgrad pow2", M, N, K)
    y = fp8q.fp8_blockscaled_gemm_wgrad_pow2(_dev(gtq), _dev(gts), _dev(xtq), _dev(xts))
    torch.cuda.synchronize()
    gemm_tolerance_check(host_bf16_as_f64(y), oracle.gemm_wgrad_f64(gtq, gts, xtq, xts), f"wgrad pow2 {M}x{N}x{K}")


def test_wgrad_pow2_exact_per_row_scales():
    """Codes for -1/0/+1 and scales 2^e per row and block on both sides: every
    partial sum is exact in fp32, so the bf16 output is the exact product
    rounded once, bit for bit."""
    require_gpu()
    fp8q = lib()
    rng = np.random.default_rng(91)
    N, K, Mp = 256, 384, 384
    lut = np.array([0xB8, 0x00, 0x38], dtype=np.uint8)
    aq, bq = lut[rng.integers(-1, 2, size=(N, Mp)) + 1], lut[rng.integers(-1, 2, size=(K, Mp)) + 1]
    as_ = np.exp2(rng.integers(-3, 4, size=(N, 3))).astype(np.float32)
    bs = np.exp2(rng.integers(-3, 4, size=(K, 3))).astype(np.float32)
    say("wgrad pow2 exact")
    y = fp8q.fp8_blockscaled_gemm_wgrad_pow2(_dev(aq), _dev(as_), _dev(bq), _dev(bs))
    torch.cuda.synchronize()
    want = oracle.round_bf16(oracle.gemm_wgrad_f64(aq, as_, bq, bs))
    assert_bytes_equal(y.cpu().contiguous().view(torch.int16).numpy().view(np.uint16), want, "wgrad pow2 exact")


def test_wgrad_pow2_nan_rule():
    """A scale that is not a power of two turns exactly the outputs that depend
    on it into NaN: a dY^T row's scale its output row, an X^T row's scale its
    output column; everything else is unchanged."""
    require_gpu()
    fp8q = lib()
    ops = _grad_operands(256, 256, 384, 7, mode=1)
    (gtq, gts), (xtq, xts) = ops["gt"], ops["xt"]
    gts, xts = gts.copy(), xts.copy()
    gts[37, 1] = 3.0
    xts[200, 0] = 0.75
    say("wgrad pow2 nan rule")
    y = host_bf16_as_f64(fp8q.fp8_blockscaled_gemm_wgrad_pow2(_dev(gtq), _dev(gts), _dev(xtq), _dev(xts)))
    torch.cuda.synchronize()
    bad = np.zeros(y.shape, bool)
    bad[37, :] = True
    bad[:, 200] = True
    assert np.isnan(y[bad]).all()
    assert not np.isnan(y[~bad]).any()
    ref = oracle.gemm_wgrad_f64(gtq, gts, xtq, xts)
    gemm_tolerance_check(np.where(bad, 0.0, y), np.where(bad, 0.0, ref), "wgrad pow2 other outputs")


def test_tiny_gradient_blocks_pow2():
    """Gradient blocks far below 448 * 2^-127 (down to bf16 subnormals) get the
    E8M0 floor 2^-127 as their power-of-two scale; the two-layout quantizer
    matches the oracle and the weight gradient on the matrix cores stays
    finite and within tolerance (a scale of 2^-127 is E8M0 byte 0x00)."""
    require_gpu()
    fp8q = lib()
    M, N, K = 256, 256, 384
    g = synth.normal_bf16((M, N), 1e-3, synth.seed_of(15, 901, 2))
    gb = synth.bf16_bits(g).copy()
    tiny = synth.bf16_bits(synth.normal_bf16((M, N), 2.0 ** -128, synth.seed_of(15, 901, 3)))
    gb[:128, :128] = tiny[:128, :128]          # one column block and rows 0..127's first row block
    gb[200, :] = 0x0001                        # a row of the smallest bf16 subnormal
    x = synth.normal_bf16((M, K), 1.0, synth.seed_of(15, 901, 0))
    xb = synth.bf16_bits(x)
    say("tiny gradient pow2 dual + wgrad_pow2")
    gq, gs, gtq, gts = fp8q.fp8_quant_act_dual(dev_bf16(gb), 1)
    _, _, xtq, xts = fp8q.fp8_quant_act_dual(dev_bf16(xb), 1, rowwise=False)
    y = fp8q.fp8_blockscaled_gemm_wgrad_pow2(gtq, gts, xtq, xts)
    torch.cuda.synchronize()
    ogq, ogs = oracle.quant_act_1x128(gb, 1)
    ogtq, ogts = oracle.quant_act_colwise_t(gb, 1)
    oxtq, oxts = oracle.quant_act_colwise_t(xb, 1)
    assert float(ogts.min()) == 2.0 ** -127 and float(ogs.min()) == 2.0 ** -127
    assert_bytes_equal(host_u8(gq), ogq, "tiny dY row codes")
    assert_scales_equal(host_f32(gs), ogs, "tiny dY row scales")
    assert_bytes_equal(host_u8(gtq), ogtq, "tiny dY column codes")
    assert_scales_equal(host_f32(gts), ogts, "tiny dY column scales")
    yh = host_bf16_as_f64(y)
    assert np.isfinite(yh).all()
    gemm_tolerance_check(yh, oracle.gemm_wgrad_f64(ogtq, ogts, oxtq, oxts), "wgrad pow2 with 2^-127 scales")
