"""GPU parity of FP8 attention for many query tokens (prefill, chunked
prefill, training forward) and of the multi-token cache append.

FP8 for the KV cache and for attention is what takes the recipe to about 48%
end to end (page "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung ...",
section "Leistungsgewinne in der Praxis").  Causal over the cache: query t of
sequence b at position start[b] + t sees cached tokens 0..start[b]+t.

The append must store the oracle's bytes and scales bit for bit.  The
attention output is checked element by element against the fp64 oracle with
the bound its arithmetic gives: each weight p_j * v_scale_j is rounded to bf16
(relative error <= 2^-8) before the value product, and the output is rounded
to bf16 once, so |out - exact| <= 2^-8 (A + |exact|) up to fp32 effects, where
A = sum_j p_j |v_j| / sum_j p_j (the oracle run on |v|).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import assert_bytes_equal, assert_scales_equal, lib, require_gpu, say

pytestmark = pytest.mark.gpu
D = 128


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _bits(shape, std, seed):
    return synth.bf16_bits(synth.normal_bf16(shape, std, synth.seed_of(31, *seed)))


def _cache(B, Hkv, S, seed, mode=0, kstd=1.0, vstd=1.0):
    kq, ks = oracle.quant_act_1x128(_bits((B * Hkv * S, D), kstd, (seed, 0)), mode)
    vq, vs = oracle.quant_act_1x128(_bits((B * Hkv * S, D), vstd, (seed, 1)), mode)
    return (kq.reshape(B, Hkv, S, D), ks.reshape(B, Hkv, S), vq.reshape(B, Hkv, S, D), vs.reshape(B, Hkv, S))


def _queries(B, T, Hq, seed, std=1.0, mode=0):
    qq, qs = oracle.quant_act_1x128(_bits((B * T * Hq, D), std, (seed, 2)), mode)
    return qq.reshape(B, T, Hq, D), qs.reshape(B, T, Hq)


def _run(qq, qs, cache, start):
    fp8q = lib()
    y = fp8q.fp8_attention_prefill(_dev(qq), _dev(qs), tuple(_dev(c) for c in cache),
                                   _dev(np.asarray(start, np.int32)))
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


def _check(y, qq, qs, cache, start, what):
    kq, ks, vq, vs = cache
    ref = oracle.attention_prefill_f64(qq, qs, kq, ks, vq, vs, start)
    absv = oracle.attention_prefill_f64(qq, qs, kq, ks, vq & np.uint8(0x7F), vs, start)   # sum p |v| / sum p
    tol = 2.0 ** -8 * (absv + np.abs(ref)) * (1 + 2.0 ** -6) + 1e-7 * absv
    bad = np.flatnonzero((np.abs(y - ref) > tol).reshape(-1))
    if bad.size:
        i = bad[:5]
        raise AssertionError(f"{what}: {bad.size} of {y.size} outside the bound; idx {i.tolist()} "
                             f"gpu {y.reshape(-1)[i].tolist()} ref {ref.reshape(-1)[i].tolist()}")
    n = float(np.linalg.norm(ref))
    if n > 0:
        assert float(np.linalg.norm(y - ref)) / n < 4e-3, what
    return ref


@pytest.mark.parametrize("grp", [1, 2, 3, 4, 8])
def test_prefill_ragged_tokens_and_group_sizes(grp):
    """T = 70 (one full 64-token query tile and a ragged one), two sequences
    starting at 0 and at 37 (chunked prefill), every group size including a
    non-power-of-two."""
    require_gpu()
    B, T, Hkv, S = 2, 70, 2, 200
    Hq = grp * Hkv
    cache = _cache(B, Hkv, S, seed=grp)
    qq, qs = _queries(B, T, Hq, seed=grp)
    start = np.array([0, 37], np.int32)
    say("attention prefill", grp, B, T, Hq, Hkv, S)
    y = _run(qq, qs, cache, start)
    _check(y, qq, qs, cache, start, f"prefill grp={grp}")


def test_prefill_positions_outside_the_cache():
    """Queries before position 0 give zeros; queries at or past S see all S
    tokens; S smaller than one key tile."""
    require_gpu()
    B, T, Hq, Hkv, S = 3, 50, 4, 1, 40
    cache = _cache(B, Hkv, S, seed=7)
    qq, qs = _queries(B, T, Hq, seed=7)
    start = np.array([-5, 20, 60], np.int32)
    say("attention prefill edges", start.tolist())
    y = _run(qq, qs, cache, start)
    assert not y[0, :5].any(), "positions below 0 see no token"
    _check(y, qq, qs, cache, start, "edges")


def test_prefill_peaked_and_flat_scores():
    """Large query and key scales (one key dominates each row) and all-zero
    keys (flat softmax, every value weighted equally)."""
    require_gpu()
    B, T, Hq, Hkv, S = 1, 64, 2, 1, 130
    qq, qs = _queries(B, T, Hq, seed=8, std=4.0)
    cache = _cache(B, Hkv, S, seed=8, kstd=4.0)
    say("attention prefill peaked")
    y = _run(qq, qs, cache, [66])
    _check(y, qq, qs, cache, np.array([66]), "peaked")
    kq0 = np.zeros_like(cache[0])
    flat = (kq0, cache[1], cache[2], cache[3])
    say("attention prefill flat")
    y = _run(qq, qs, flat, [66])
    _check(y, qq, qs, flat, np.array([66]), "flat")


@pytest.mark.parametrize("mode", [0, 1])
def test_append_tokens_then_prefill_end_to_end(mode):
    """bf16 K and V of a 100-token chunk appended after 30 cached tokens (bit
    for bit against the oracle's append), queries quantized by the library,
    then attention over the cache."""
    require_gpu()
    fp8q = lib()
    B, T, Hq, Hkv, S = 2, 100, 8, 2, 160
    rng = np.random.default_rng(40 + mode)
    kq0 = rng.integers(0, 0x7E, (B, Hkv, S, D)).astype(np.uint8)
    ks0 = rng.uniform(1e-3, 1e-2, (B, Hkv, S)).astype(np.float32)
    vq0, vs0 = kq0.copy(), ks0.copy()
    start = np.array([30, 70], np.int32)          # the second chunk runs past S
    kn = _bits((B, T, Hkv, D), 1.0, (mode, 3))
    vn = _bits((B, T, Hkv, D), 0.5, (mode, 4))
    cache = (_dev(kq0), _dev(ks0), _dev(vq0), _dev(vs0))
    say("append tokens", mode, B, T, Hkv, S)
    fp8q.fp8_kv_cache_append_tokens(_bf(kn), _bf(vn), _dev(start), cache, mode=mode)
    torch.cuda.synchronize()
    okq, oks = oracle.kv_cache_append_tokens(kn, start, kq0.copy(), ks0.copy(), mode)
    ovq, ovs = oracle.kv_cache_append_tokens(vn, start, vq0.copy(), vs0.copy(), mode)
    assert_bytes_equal(cache[0].cpu().numpy(), okq, "k cache")
    assert_scales_equal(cache[1].cpu().numpy(), oks, "k scales")
    assert_bytes_equal(cache[2].cpu().numpy(), ovq, "v cache")
    assert_scales_equal(cache[3].cpu().numpy(), ovs, "v scales")
    qb = _bits((B * T * Hq, D), 1.0, (mode, 5))
    q_q, q_s = fp8q.fp8_quant_act_1x128(_bf(qb), mode)
    say("prefill after append", mode)
    y = fp8q.fp8_attention_prefill(q_q.view(B, T, Hq, D), q_s.view(B, T, Hq), cache, _dev(start))
    torch.cuda.synchronize()
    oqq, oqs = oracle.quant_act_1x128(qb, mode)
    assert_bytes_equal(q_q.cpu().numpy(), oqq, "query codes")
    _check(y.float().cpu().numpy().astype(np.float64), oqq.reshape(B, T, Hq, D), oqs.reshape(B, T, Hq),
           (okq, oks, ovq, ovs), start, f"end to end mode {mode}")


def _bf(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


def test_llama_prefill_full_size_sampled():
    """Llama-3.1-8B attention at 4096 tokens (32 query / 8 key-value heads, one
    sequence prefilled from position 0); every head of a sample of query
    tokens, first and last included, against the oracle one token at a time."""
    require_gpu()
    fp8q = lib()
    B, T, Hq, Hkv = 1, 4096, 32, 8
    S = T
    g = torch.Generator(device="cuda").manual_seed(synth.seed_of(31, 4096, 0))
    kq = (torch.randn((B, Hkv, S, D), device="cuda", generator=g) * 32).clamp(-448, 448).to(torch.float8_e4m3fn)
    vq = (torch.randn((B, Hkv, S, D), device="cuda", generator=g) * 32).clamp(-448, 448).to(torch.float8_e4m3fn)
    ks = torch.rand((B, Hkv, S), device="cuda", generator=g) * 0.01 + 0.001
    vs = torch.rand((B, Hkv, S), device="cuda", generator=g) * 0.01 + 0.001
    qb = _bits((B * T * Hq, D), 1.0, (4096, 5))
    q_q, q_s = fp8q.fp8_quant_act_1x128(_bf(qb))
    q_q, q_s = q_q.view(B, T, Hq, D), q_s.view(B, T, Hq)
    cache = (kq.view(torch.uint8), ks, vq.view(torch.uint8), vs)
    say("attention llama prefill full size")
    y = fp8q.fp8_attention_prefill(q_q, q_s, cache, _dev(np.array([0], np.int32)))
    torch.cuda.synchronize()
    hc = tuple(c.cpu().numpy() for c in cache)
    hq, hs = q_q.cpu().numpy(), q_s.cpu().numpy()
    rng = np.random.default_rng(4096)
    picks = np.unique(np.concatenate([[0, 1, 63, 64, 2047, T - 1], rng.integers(0, T, 10)]))
    for t in picks:
        got = y[:, t:t + 1].float().cpu().numpy().astype(np.float64)
        _check(got, hq[:, t:t + 1], hs[:, t:t + 1], hc, np.array([t]), f"llama prefill token {t}")
