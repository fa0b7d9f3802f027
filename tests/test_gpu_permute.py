"""GPU parity of the MoE dispatch order (fp8_moe_permute): the group offsets,
the token of every row and the row of every entry must equal the oracle's
stable grouping bit for bit (index work), for the Qwen3-30B-A3B and
Moonlight-16B routings (page "NVIDIA NeMo RL erreicht 48% Geschwindigkeits-
steigerung ...", sections "Leistungsgewinne in der Praxis" and "Warum dies
fuer die KI-Oekonomie wichtig ist") and for edge cases: invalid expert ids,
repeated experts in one token, one expert, 1024 experts, no tokens, tables
that end inside a block."""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import assert_bytes_equal, lib, require_gpu, say

pytestmark = pytest.mark.gpu


def _check(ids, E, ns, what):
    fp8q = lib()
    say("moe permute", what, ids.shape, E, ns)
    off, rows, er = fp8q.fp8_moe_permute(torch.from_numpy(np.ascontiguousarray(ids, np.int32)).to("cuda"), E, ns)
    torch.cuda.synchronize()
    o_off, o_rows, o_er = oracle.moe_permute(ids, E, ns)
    assert_bytes_equal(off.cpu().numpy(), o_off, what + " offsets")
    assert_bytes_equal(rows.cpu().numpy(), o_rows, what + " row_index")
    assert_bytes_equal(er.cpu().numpy(), o_er, what + " entry_row")


@pytest.mark.parametrize("shape", [synth.QWEN3, synth.MOONLIGHT], ids=lambda s: s.name)
def test_model_routings(shape):
    _check(synth.moe_routing(shape), shape.routed_experts, shape.shared_experts, shape.name)


@pytest.mark.parametrize("T,k,E,ns,bad", [
    (0, 8, 128, 0, 0.0), (0, 2, 4, 2, 0.0), (1, 1, 1, 0, 0.0), (1, 8, 128, 1, 0.0),
    (127, 8, 128, 0, 0.0), (128, 8, 128, 0, 0.0), (129, 8, 128, 0, 0.0),
    (1000, 6, 64, 2, 0.0), (777, 3, 5, 1, 0.3), (3000, 4, 1024, 0, 0.0),
    (5000, 2, 1, 1, 0.0), (4096, 16, 256, 0, 0.1),
])
def test_edge_cases(T, k, E, ns, bad):
    rng = np.random.default_rng(T * 7 + k + E)
    ids = rng.integers(0, E, (T, k)).astype(np.int32)      # repeats inside a token allowed
    if bad > 0 and T:
        m = rng.random(ids.shape) < bad
        ids[m] = rng.choice(np.array([-1, E, E + 5, -(1 << 30), (1 << 31) - 1], np.int64), m.sum()).astype(np.int32)
    _check(ids, E, ns, f"T={T} k={k} E={E} ns={ns} bad={bad}")


def test_dispatch_chain_matches_oracle_order():
    """Routing -> device permute -> gathered GEMM gives the bits of the grouped
    GEMM on rows in the oracle's order (quantize before dispatch)."""
    require_gpu()
    fp8q = lib()
    shape = synth.MoEShape("small", tokens=900, hidden=512, routed_experts=16, top_k=4,
                           shared_experts=1, ffn=256, zipf_alpha=1.1)
    ids = synth.moe_routing(shape)
    xt = synth.moe_token_matrix(shape, "cuda")
    w = synth.moe_weights(shape, "gate_up", "cuda")
    G, N, K = w.shape
    bq = torch.empty((G, N, K), dtype=torch.uint8, device="cuda")
    bs = torch.empty((G, N // 128, K // 128), dtype=torch.float32, device="cuda")
    for g in range(G):
        fp8q.fp8_quant_weight_128x128(w[g], out=(bq[g], bs[g]))
    say("dispatch chain", xt.shape, w.shape)
    off, rows, _ = fp8q.fp8_moe_permute(torch.from_numpy(ids).to("cuda"), shape.routed_experts, 1)
    aq, as_ = fp8q.fp8_quant_act_1x128(xt)
    yg = fp8q.fp8_grouped_gemm_gather(aq, as_, bq, bs, off, rows)
    o_off, o_rows, _ = oracle.moe_permute(ids, shape.routed_experts, 1)
    idx = torch.from_numpy(o_rows.astype(np.int64)).to("cuda")
    yr = fp8q.fp8_grouped_gemm(aq[idx].contiguous(), as_[idx].contiguous(), bq, bs, torch.from_numpy(o_off).to("cuda"))
    torch.cuda.synchronize()
    assert torch.equal(yg.view(torch.int16), yr.view(torch.int16))
