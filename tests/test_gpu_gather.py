"""GPU parity of the grouped GEMM that gathers routed rows from a token matrix
quantized before dispatch.

MoE expert layers run the same block-scaled linear layer as the dense model
(page "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung ...", sections
"Leistungsgewinne in der Praxis" and "Warum dies fuer die KI-Oekonomie wichtig
ist"); a 1x128 activation block lies inside one token row, so quantizing the
tokens and then selecting rows gives the same codes and scales as selecting
rows and then quantizing.  The gathered GEMM is therefore checked bit for bit
against the grouped GEMM on explicitly gathered operands, and against the
oracle within the GEMM tolerance.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (assert_bytes_equal, assert_scales_equal, gemm_tolerance_check, host_bf16_as_f64,
                        host_f32, host_u8, lib, moe_rows, moe_whole_rows_check, require_gpu, say)

pytestmark = pytest.mark.gpu

MODES = ("amax", "pow2")


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _bits(y):
    return y.detach().cpu().contiguous().view(torch.int16).numpy()


def _case(T, sizes, N, K, seed, mode, bad_rows=0):
    """Oracle-quantized tokens [T, K], per-group weights, offsets, and a routed
    row -> token index with repeats (plus bad_rows indices outside [0, T))."""
    m = oracle.MODE_POW2 if mode == "pow2" else oracle.MODE_AMAX
    G = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(off[-1])
    xt = synth.normal_bf16((T, K), 1.0, synth.seed_of(12, seed, 0), outlier_frac=0.01)
    w = synth.normal_bf16((G, N, K), 0.02, synth.seed_of(12, seed, 1))
    aq, as_ = oracle.quant_act_1x128(synth.bf16_bits(xt), m)
    bqs, bss = zip(*[oracle.quant_weight_128x128(synth.bf16_bits(w[g]), m) for g in range(G)])
    rng = np.random.default_rng(synth.seed_of(12, seed, 2))
    idx = rng.integers(0, T, M).astype(np.int32)
    if bad_rows:
        pos = rng.choice(M, bad_rows, replace=False)
        idx[pos] = rng.choice(np.array([-1, T, T + 7, 2 ** 31 - 1, -2 ** 31], dtype=np.int64),
                              bad_rows).astype(np.int32)
    return aq, as_, np.stack(bqs), np.stack(bss), off, idx


def _gather(aq, as_, bq, bs, off, idx, mode):
    fp8q = lib()
    y = fp8q.fp8_grouped_gemm_gather(_dev(aq), _dev(as_), _dev(bq), _dev(bs), _dev(off), _dev(idx), mode=mode)
    torch.cuda.synchronize()
    return y


def _grouped(aq, as_, bq, bs, off, mode):
    fp8q = lib()
    fn = fp8q.fp8_grouped_gemm_pow2 if mode == "pow2" else fp8q.fp8_grouped_gemm
    y = fn(_dev(aq), _dev(as_), _dev(bq), _dev(bs), _dev(off))
    torch.cuda.synchronize()
    return y


CASES = [
    (300, [3, 0, 130, 1, 0, 255, 128], 256, 256),
    (17, [0, 0, 0, 40], 384, 384),            # fewer tokens than routed rows: many repeats
    (1000, [129, 127, 128, 1, 256, 0, 64], 640, 512),
    (2000, [600, 0, 257, 1024, 1, 300, 256], 384, 640),   # 256-row tiles
    (1, [5], 128, 128),                       # one token
]


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T,sizes,N,K", CASES)
def test_equals_grouped_on_gathered_rows(T, sizes, N, K, mode):
    """Bit-exact against fp8_grouped_gemm(_pow2) on a_q[idx], a_s[idx]."""
    require_gpu()
    aq, as_, bq, bs, off, idx = _case(T, sizes, N, K, T + N, mode)
    say("gather vs grouped", T, sizes, N, K, mode)
    yg = _gather(aq, as_, bq, bs, off, idx, mode)
    yr = _grouped(aq[idx], as_[idx], bq, bs, off, mode)
    assert_bytes_equal(_bits(yg), _bits(yr), f"gather {T} {sizes} {mode}")


@pytest.mark.parametrize("mode", MODES)
@pytest.mark.parametrize("T,sizes,N,K", CASES[:3])
def test_against_oracle(T, sizes, N, K, mode):
    require_gpu()
    aq, as_, bq, bs, off, idx = _case(T, sizes, N, K, 7 * T + K, mode)
    say("gather vs oracle", T, sizes, N, K, mode)
    y = host_bf16_as_f64(_gather(aq, as_, bq, bs, off, idx, mode))
    ref = oracle.grouped_gemm_f64(aq[idx], as_[idx], bq, bs, off)
    gemm_tolerance_check(y, ref, f"gather {sizes} {mode}")


@pytest.mark.parametrize("mode", MODES)
def test_indices_outside_the_token_matrix_give_zero_rows(mode):
    """Rows whose index is outside [0, T) are zeros (also with power-of-two
    scales, where the zero scale such a row reads would otherwise mean NaN);
    every other row is unchanged."""
    require_gpu()
    T, sizes, N, K = 200, [40, 0, 300, 77], 384, 512
    aq, as_, bq, bs, off, idx = _case(T, sizes, N, K, 99, mode, bad_rows=60)
    say("gather bad indices", mode)
    y = _gather(aq, as_, bq, bs, off, idx, mode)
    bad = (idx < 0) | (idx >= T)
    assert bad.sum() == 60
    yb = _bits(y)
    assert not yb[bad].any(), "rows with an invalid index must be +0"
    safe = np.where(bad, 0, idx)
    yr = _bits(_grouped(aq[safe], as_[safe], bq, bs, off, mode))
    assert_bytes_equal(yb[~bad], yr[~bad], f"gather valid rows {mode}")


def test_quantize_before_dispatch_commutes():
    """Quantizing the T tokens on the GPU and gathering gives the same codes
    and scales as gathering the bf16 rows and quantizing them, and the two
    GEMM outputs are identical."""
    require_gpu()
    fp8q = lib()
    shape = synth.MoEShape("small", tokens=700, hidden=1024, routed_experts=16, top_k=4,
                           shared_experts=1, ffn=256, zipf_alpha=1.1)
    off, row_token, _ = oracle.moe_permute(synth.moe_routing(shape), shape.routed_experts,
                                           shape.shared_experts)
    xt = synth.moe_token_matrix(shape, "cuda")
    w = synth.moe_weights(shape, "gate_up", "cuda")
    G, N, K = w.shape
    say("gather commute", xt.shape, w.shape)
    bq = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for g in range(G):
        fp8q.fp8_quant_weight_128x128(w[g], out=(bq[g], bs[g]))
    idx64 = torch.from_numpy(row_token.astype(np.int64)).to("cuda")
    aq_t, as_t = fp8q.fp8_quant_act_1x128(xt)
    aq_r, as_r = fp8q.fp8_quant_act_1x128(xt[idx64].contiguous())
    torch.cuda.synchronize()
    assert_bytes_equal(host_u8(aq_t[idx64]), host_u8(aq_r), "codes")
    assert_scales_equal(host_f32(as_t[idx64]), host_f32(as_r), "scales")
    offd = torch.from_numpy(off).to("cuda")
    yg = fp8q.fp8_grouped_gemm_gather(aq_t, as_t, bq, bs, offd, idx64.to(torch.int32))
    yr = fp8q.fp8_grouped_gemm(aq_r, as_r, bq, bs, offd)
    torch.cuda.synchronize()
    assert_bytes_equal(_bits(yg), _bits(yr), "gather vs quantize-after-dispatch")


@pytest.mark.parametrize("shape", [synth.QWEN3, synth.MOONLIGHT], ids=lambda s: s.name)
def test_moe_full_size(shape):
    """Full-size Qwen3-30B-A3B and Moonlight-16B gate_up layers: the gathered
    GEMM equals the grouped GEMM on the gathered operands bit for bit, and in
    every group its first, last and two random rows match the oracle whole."""
    require_gpu()
    fp8q = lib()
    off, row_token, _ = oracle.moe_permute(synth.moe_routing(shape), shape.routed_experts,
                                           shape.shared_experts)
    xt = synth.moe_token_matrix(shape, "cuda")
    w = synth.moe_weights(shape, "gate_up", "cuda")
    G, N, K = w.shape
    say("gather moe", shape.name, xt.shape, w.shape)
    bq = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for g in range(G):
        fp8q.fp8_quant_weight_128x128(w[g], out=(bq[g], bs[g]))
    del w
    idx64 = torch.from_numpy(row_token.astype(np.int64)).to("cuda")
    offd = torch.from_numpy(off).to("cuda")
    aq, as_ = fp8q.fp8_quant_act_1x128(xt)
    yg = fp8q.fp8_grouped_gemm_gather(aq, as_, bq, bs, offd, idx64.to(torch.int32))
    yr = fp8q.fp8_grouped_gemm(aq[idx64].contiguous(), as_[idx64].contiguous(), bq, bs, offd)
    torch.cuda.synchronize()
    assert torch.equal(yg.view(torch.int16), yr.view(torch.int16)), f"{shape.name}: gather != grouped"
    ms, gs = moe_rows(off, seed=5)
    tok = row_token[ms]
    haq, has = aq.cpu().numpy()[tok], as_.cpu().numpy()[tok]   # the tokens the routed rows point at
    yr_rows = yg.float().cpu().numpy().astype(np.float64)[ms]
    moe_whole_rows_check(yr_rows, haq, has, bq.cpu().numpy(), bs.cpu().numpy(), gs, f"{shape.name} gather rows")
