"""GPU parity of the experts' fused gate+up GEMM with SwiGLU and the down
projection's 1x128 quantization in its epilogue (the recipe's MoE models,
page "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung ...", sections
"Leistungsgewinne in der Praxis" and "Warum dies fuer die KI-Oekonomie wichtig
ist"; the separate activation and quantization passes it replaces are the
quantization-kernel overhead named in "Leistungsgewinne in der Praxis").

Every row of the grouped kernel is the dense fused kernel's row for that
row's expert: same main loop, same epilogue.  So:
  1. bit for bit against fp8_blockscaled_gemm_swiglu_quant on each group's
     rows with its expert's weight (ragged and empty groups, both tile
     heights, both output modes);
  2. with gathered rows, bit for bit against the same call on explicitly
     gathered rows; an index outside the tokens gives h = 0 (codes 0, scale 1);
  3. against the oracle as the dense fused kernel is checked (its fp64 h
     against the kernel's fp32 exponential): dequantized values within one
     E4M3 step plus the GEMM tolerance carried through silu(g) * u, and at all
     but a few 1e-4 of the positions the oracle's SwiGLU and row quantizer on
     the GPU's own bf16 gate and up give the same bytes;
  4. at the full Qwen3-30B-A3B and Moonlight-16B gate+up shapes, routed rows
     gathered from the quantized tokens: whole rows (first, last and two
     random ones of every group) against the oracle.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import assert_bytes_equal, assert_scales_equal, host_f32, host_u8, lib, moe_rows, require_gpu, say

pytestmark = pytest.mark.gpu

MODES = {0: "amax", 1: "pow2"}


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _case(T, sizes, F, K, seed):
    """Oracle-quantized tokens [T, K], per-expert fused gate+up weights
    [G, 2F, K], offsets, and a routed row -> token index with repeats."""
    G = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(off[-1])
    xt = synth.normal_bf16((T, K), 1.0, synth.seed_of(31, seed, 0), outlier_frac=0.01)
    w = synth.normal_bf16((G, 2 * F, K), 0.06, synth.seed_of(31, seed, 1))
    aq, as_ = oracle.quant_act_1x128(synth.bf16_bits(xt))
    bqs, bss = zip(*[oracle.quant_weight_128x128(synth.bf16_bits(w[g])) for g in range(G)])
    idx = np.random.default_rng(synth.seed_of(31, seed, 2)).integers(0, T, M).astype(np.int32)
    return aq, as_, np.stack(bqs), np.stack(bss), off, idx


def _grouped(aq, as_, bq, bs, off, mode, idx=None):
    fp8q = lib()
    hq, hs = fp8q.fp8_grouped_gemm_swiglu_quant(_dev(aq), _dev(as_), _dev(bq), _dev(bs), _dev(off),
                                                row_index=None if idx is None else _dev(idx), mode=MODES[mode])
    torch.cuda.synchronize()
    return host_u8(hq), host_f32(hs)


def _dense(aq, as_, bq, bs, mode):
    fp8q = lib()
    hq, hs = fp8q.fp8_blockscaled_gemm_swiglu_quant(_dev(aq), _dev(as_), _dev(bq), _dev(bs), mode=MODES[mode])
    torch.cuda.synchronize()
    return host_u8(hq), host_f32(hs)


def _dequant(q, s):
    dec = torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    return dec * np.repeat(np.asarray(s, np.float64), 128, axis=1)


def _within_one_step(q, s, q_ref, s_ref, what, slack):
    """Dequantized values at most one E4M3 step apart (at the coarser of the
    two scales), plus `slack` for a difference in the values quantized."""
    a, b = _dequant(q, s), _dequant(q_ref, s_ref)
    srep = np.repeat(np.maximum(s, s_ref).astype(np.float64), 128, axis=1)
    tol = (2.0 ** -3 + 2.0 ** -7) * np.maximum(np.abs(a), np.abs(b)) + 2.0 ** -9 * srep + 1.125 * slack
    bad = np.flatnonzero(np.abs(a - b).reshape(-1) > tol.reshape(-1))
    if bad.size:
        i = bad[:4]
        raise AssertionError(f"{what}: {bad.size} elements more than one E4M3 step apart; idx {i.tolist()} "
                             f"got {a.reshape(-1)[i].tolist()} want {b.reshape(-1)[i].tolist()}")


def _slack(y):
    """How far h may move when gate and up each move within the GEMM tolerance
    (8e-3 of the value + 1e-3 of the rms of the rows' outputs): silu's slope
    is below 1.1.  y: the exact fused gate|up outputs [rows, 2F]."""
    rms = float(np.sqrt(np.mean(y ** 2)))
    g, u = oracle.swiglu_split(y)
    dg, du = 8e-3 * np.abs(g) + 1e-3 * rms, 8e-3 * np.abs(u) + 1e-3 * rms
    return 1.1 * dg * (np.abs(u) + du) + np.abs(g / (1.0 + np.exp(-g))) * du


def _check_against_oracle(q, s, y, mode, what):
    """q, s: the kernel's rows; y: the oracle's exact gate|up for those rows."""
    q_ref, s_ref = oracle.quant_act_1x128(oracle.round_bf16(_h_of(y)), mode)
    _within_one_step(q, s, q_ref, s_ref, what + " vs oracle", _slack(y))
    h = _h_of(y)
    e_gpu = np.linalg.norm(_dequant(q, s) - h)
    e_ref = np.linalg.norm(_dequant(q_ref, s_ref) - h)
    assert e_gpu <= 1.02 * e_ref + 2e-3 * np.linalg.norm(h), f"{what}: error {e_gpu:.4e} vs oracle's {e_ref:.4e}"


def _h_of(y):
    g, u = oracle.swiglu_split(oracle.bf16_to_f64(oracle.round_bf16(y)))
    return g / (1.0 + np.exp(-g)) * u


CASES = [
    (300, [3, 0, 130, 1, 0, 255, 128], 128, 256),          # 128-row tiles (M_total < 256 G)
    (1000, [129, 127, 128, 1, 256, 0, 64], 384, 512),
    (2000, [600, 0, 257, 1024, 1, 300, 256], 256, 384),    # 256-row tiles
    (1, [5], 128, 128),                                    # one token, one group
]


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T,sizes,F,K", CASES)
def test_equals_dense_per_group(T, sizes, F, K, mode):
    require_gpu()
    aq, as_, bq, bs, off, idx = _case(T, sizes, F, K, T + F + mode)
    ga, gs_ = aq[idx], as_[idx]
    say("grouped swiglu vs dense per group", T, sizes, F, K, MODES[mode])
    hq, hs = _grouped(ga, gs_, bq, bs, off, mode)
    assert hq.shape == (int(off[-1]), F) and hs.shape == (int(off[-1]), F // 128)
    for g in range(len(sizes)):
        a, b = int(off[g]), int(off[g + 1])
        if a == b:
            continue
        dq, ds = _dense(ga[a:b], gs_[a:b], bq[g], bs[g], mode)
        assert_bytes_equal(hq[a:b], dq, f"group {g} codes")
        assert_scales_equal(hs[a:b], ds, f"group {g} scales")


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T,sizes,F,K", CASES[:3])
def test_gather_equals_gathered_rows(T, sizes, F, K, mode):
    """Routed rows read by index give the rows of the non-gathering call on
    explicitly gathered operands; an index outside the tokens gives h = 0."""
    require_gpu()
    aq, as_, bq, bs, off, idx = _case(T, sizes, F, K, 3 * T + K + mode)
    bad = np.zeros(idx.size, bool)
    bad[np.random.default_rng(T).choice(idx.size, 7, replace=False)] = True
    idx = idx.copy()
    idx[bad] = np.array([-1, T, T + 9, 2 ** 31 - 1, -2 ** 31, -5, T], dtype=np.int64)[:int(bad.sum())].astype(np.int32)
    say("grouped swiglu gather", T, sizes, F, K, MODES[mode])
    hq, hs = _grouped(aq, as_, bq, bs, off, mode, idx)
    safe = np.where(bad, 0, idx)
    rq, rs = _grouped(aq[safe], as_[safe], bq, bs, off, mode)
    assert_bytes_equal(hq[~bad], rq[~bad], "gathered rows codes")
    assert_scales_equal(hs[~bad], rs[~bad], "gathered rows scales")
    assert not hq[bad].any() and (hs[bad] == 1.0).all(), "rows with an invalid index must quantize h = 0"


@pytest.mark.parametrize("mode", [0, 1])
@pytest.mark.parametrize("T,sizes,F,K", CASES[:3])
def test_against_oracle(T, sizes, F, K, mode):
    require_gpu()
    aq, as_, bq, bs, off, idx = _case(T, sizes, F, K, 5 * T + 3 * K + mode)
    say("grouped swiglu vs oracle", T, sizes, F, K, MODES[mode])
    hq, hs = _grouped(aq, as_, bq, bs, off, mode, idx)
    # end to end: the oracle's grouped fused product (fp64 GEMM and h)
    q_ref, s_ref = oracle.grouped_gemm_swiglu_quant(aq, as_, bq, bs, off, mode, row_index=idx)
    y = oracle.grouped_gemm_f64(aq[idx], as_[idx], bq, bs, off)
    _within_one_step(hq, hs, q_ref, s_ref, f"{sizes} vs oracle", _slack(y))
    h = _h_of(y)
    e_gpu = np.linalg.norm(_dequant(hq, hs) - h)
    e_ref = np.linalg.norm(_dequant(q_ref, s_ref) - h)
    assert e_gpu <= 1.02 * e_ref + 2e-3 * np.linalg.norm(h), f"error {e_gpu:.4e} vs oracle's {e_ref:.4e}"
    # the oracle's SwiGLU and row quantizer on the GPU's own bf16 gate and up
    y = lib().fp8_grouped_gemm_gather(_dev(aq), _dev(as_), _dev(bq), _dev(bs), _dev(off), _dev(idx))
    ybits = y.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    g, u = oracle.swiglu_split(oracle.bf16_to_f64(ybits))
    q_own, s_own = oracle.quant_act_1x128(oracle.round_bf16(g / (1.0 + np.exp(-g)) * u), mode)
    n_bytes = int(np.count_nonzero(hq != q_own))
    assert n_bytes <= max(4, 5e-4 * hq.size), f"{n_bytes} of {hq.size} bytes differ"
    _within_one_step(hq, hs, q_own, s_own, f"{sizes} vs own gate/up", 0.0)


@pytest.mark.parametrize("shape", [synth.QWEN3, synth.MOONLIGHT], ids=lambda s: s.name)
def test_moe_full_size(shape):
    """Full-size Qwen3-30B-A3B and Moonlight-16B gate+up, routed rows gathered
    from the quantized tokens: whole rows of every group against the oracle,
    and every row against the oracle's SwiGLU on the GPU's own bf16 gate and
    up (the gathering grouped GEMM, which shares the main loop)."""
    require_gpu()
    fp8q = lib()
    off, row_token, _ = oracle.moe_permute(synth.moe_routing(shape), shape.routed_experts, shape.shared_experts)
    xt = synth.moe_token_matrix(shape, "cuda")
    w = synth.moe_weights(shape, "gate_up", "cuda")
    G, N, K = w.shape
    say("grouped swiglu moe", shape.name, xt.shape, w.shape)
    bq = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for g in range(G):
        fp8q.fp8_quant_weight_128x128(w[g], out=(bq[g], bs[g]))
    del w
    offd = torch.from_numpy(off).to("cuda")
    idxd = torch.from_numpy(row_token.astype(np.int32)).to("cuda")
    aq, as_ = fp8q.fp8_quant_act_1x128(xt)
    hq, hs = fp8q.fp8_grouped_gemm_swiglu_quant(aq, as_, bq, bs, offd, row_index=idxd)
    y = fp8q.fp8_grouped_gemm_gather(aq, as_, bq, bs, offd, idxd)
    torch.cuda.synchronize()
    hq, hs = host_u8(hq), host_f32(hs)
    ybits = y.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    del y
    # every row against the oracle's SwiGLU of the GPU's own gate and up
    for lo in range(0, hq.shape[0], 8192):
        g, u = oracle.swiglu_split(oracle.bf16_to_f64(ybits[lo:lo + 8192]))
        q_ref, s_ref = oracle.quant_act_1x128(oracle.round_bf16(g / (1.0 + np.exp(-g)) * u))
        n_bytes = int(np.count_nonzero(hq[lo:lo + 8192] != q_ref))
        assert n_bytes <= 5e-4 * q_ref.size, f"rows {lo}..: {n_bytes} bytes differ"
        _within_one_step(hq[lo:lo + 8192], hs[lo:lo + 8192], q_ref, s_ref, f"rows {lo}..", 0.0)
    # whole rows of every group against the oracle end to end
    ms, gs = moe_rows(off, seed=9)
    tok = row_token[ms]
    haq, has = aq.cpu().numpy(), as_.cpu().numpy()
    R = ms.size
    yo = oracle.grouped_gemm_sampled_f64(haq, has, bq.cpu().numpy(), bs.cpu().numpy(), np.repeat(gs, N),
                                         np.repeat(tok, N), np.tile(np.arange(N), R)).reshape(R, N)
    _check_against_oracle(hq[ms], hs[ms], yo, 0, f"{shape.name} rows")
