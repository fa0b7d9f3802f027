"""GPU parity of the grouped (mixture-of-experts) block-scaled FP8 GEMM.

The recipe runs on MoE models too (Qwen3-30B and Moonlight 16B: page "NVIDIA
NeMo RL erreicht 48% Geschwindigkeitssteigerung ...", sections
"Leistungsgewinne in der Praxis" and "Warum dies fuer die KI-Oekonomie wichtig
ist"); every expert's linear layer is the dense block-scaled GEMM on its own
rows.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (gemm_tolerance_check, host_bf16_as_f64, lib, moe_layer_inputs, moe_rows,
                        moe_whole_rows_check, require_gpu, say)

pytestmark = pytest.mark.gpu


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _operands(sizes, N, K, seed):
    G = len(sizes)
    off = np.concatenate([[0], np.cumsum(sizes)]).astype(np.int32)
    M = int(off[-1])
    x = synth.normal_bf16((max(M, 1), K), 1.0, synth.seed_of(11, seed, 0))[:M]
    w = synth.normal_bf16((G, N, K), 0.02, synth.seed_of(11, seed, 1))
    aq, as_ = oracle.quant_act_1x128(synth.bf16_bits(x))
    bqs, bss = zip(*[oracle.quant_weight_128x128(synth.bf16_bits(w[g])) for g in range(G)])
    return aq, as_, np.stack(bqs), np.stack(bss), off


def _run(aq, as_, bq, bs, off):
    fp8q = lib()
    y = fp8q.fp8_grouped_gemm(_dev(aq), _dev(as_), _dev(bq), _dev(bs), _dev(off))
    torch.cuda.synchronize()
    return host_bf16_as_f64(y)


@pytest.mark.parametrize("sizes,N,K", [
    ([3, 0, 130, 1, 0, 255, 128], 256, 256),
    ([0, 0, 0, 17], 384, 384),
    ([500], 128, 128),
    ([129, 127, 128, 1, 256, 0, 64], 640, 512),
    ([600, 0, 257, 1024, 1, 300, 256], 384, 640),    # average >= 256 rows: 256-row tiles
    ([2048, 513], 2816, 1408),
])
def test_ragged_and_empty_groups(sizes, N, K):
    require_gpu()
    aq, as_, bq, bs, off = _operands(sizes, N, K, seed=sum(sizes) + N)
    say("grouped", sizes, N, K)
    y = _run(aq, as_, bq, bs, off)
    ref = oracle.grouped_gemm_f64(aq, as_, bq, bs, off)
    gemm_tolerance_check(y, ref, f"grouped {sizes}")


def test_single_group_equals_dense():
    require_gpu()
    fp8q = lib()
    aq, as_, bq, bs, off = _operands([300], 512, 384, seed=1)
    say("grouped vs dense")
    yg = _run(aq, as_, bq, bs, off)
    yd = fp8q.fp8_blockscaled_gemm(_dev(aq), _dev(as_), _dev(bq[0]), _dev(bs[0]))
    torch.cuda.synchronize()
    assert np.array_equal(yg, host_bf16_as_f64(yd))


@pytest.mark.parametrize("shape", [synth.QWEN3, synth.MOONLIGHT], ids=lambda s: s.name)
@pytest.mark.parametrize("layer", ["gate_up", "down"])
def test_moe_full_size_rows(shape, layer):
    """Full-size Qwen3-30B-A3B (128 experts, Zipf(1.1) load) and Moonlight-16B
    (64 routed + 2 shared experts) expert layers: quantize + grouped GEMM on the
    GPU; in every group its first, last and two random rows are checked whole
    (all N outputs) against the oracle."""
    require_gpu()
    fp8q = lib()
    x, w, off, _ = moe_layer_inputs(shape, layer)
    G, N, K = w.shape
    say("grouped moe", shape.name, layer, x.shape, w.shape)
    aq, as_ = fp8q.fp8_quant_act_1x128(x)
    bq = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for g in range(G):
        fp8q.fp8_quant_weight_128x128(w[g], out=(bq[g], bs[g]))
    y = fp8q.fp8_grouped_gemm(aq, as_, bq, bs, torch.from_numpy(off).to("cuda"))
    torch.cuda.synchronize()
    ms, gs = moe_rows(off, seed=3)
    haq, has = aq.cpu().numpy()[ms], as_.cpu().numpy()[ms]
    yr = y.float().cpu().numpy().astype(np.float64)[ms]
    moe_whole_rows_check(yr, haq, has, bq.cpu().numpy(), bs.cpu().numpy(), gs, f"{shape.name} {layer} rows")
