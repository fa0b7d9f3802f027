"""GPU parity of the FP8 KV cache and the FP8 decode attention.

FP8 for the KV cache and for attention is what takes the recipe to about 48%
end to end (page "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung ...",
section "Leistungsgewinne in der Praxis").  The cache append must store the
oracle's bytes and scales bit for bit; the attention output must meet the
GEMM tolerance against the fp64 oracle (element-wise 8e-3 relative + 1e-3 of
the rms, Frobenius 2e-3; bf16 output rounding alone costs ~1.7e-3 of the
latter).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import assert_bytes_equal, assert_scales_equal, gemm_tolerance_check, lib, require_gpu, say

pytestmark = pytest.mark.gpu
D = 128


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _bits(shape, std, seed):
    return synth.bf16_bits(synth.normal_bf16(shape, std, synth.seed_of(17, *seed)))


def _cache(B, Hkv, S, seed, mode=0, kstd=1.0, vstd=1.0):
    """Oracle-quantized K and V caches [B, Hkv, S, 128] and scales."""
    kb = _bits((B * Hkv * S, D), kstd, (seed, 0))
    vb = _bits((B * Hkv * S, D), vstd, (seed, 1))
    kq, ks = oracle.quant_act_1x128(kb, mode)
    vq, vs = oracle.quant_act_1x128(vb, mode)
    return (kq.reshape(B, Hkv, S, D), ks.reshape(B, Hkv, S), vq.reshape(B, Hkv, S, D), vs.reshape(B, Hkv, S))


def _query(B, Hq, seed, std=1.0, mode=0):
    qq, qs = oracle.quant_act_1x128(_bits((B * Hq, D), std, (seed, 2)), mode)
    return qq.reshape(B, Hq, D), qs.reshape(B, Hq)


def _run(qq, qs, cache, seq_len, workspace="auto"):
    fp8q = lib()
    dcache = tuple(_dev(c) for c in cache)
    y = fp8q.fp8_attention_decode(_dev(qq), _dev(qs), dcache, _dev(np.asarray(seq_len, np.int32)),
                                  workspace=workspace)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


@pytest.mark.parametrize("mode", [0, 1])
def test_kv_cache_append_bit_exact(mode):
    require_gpu()
    fp8q = lib()
    B, H, S = 5, 8, 40
    rng = np.random.default_rng(mode)
    kq = rng.integers(0, 256, (B, H, S, D)).astype(np.uint8)
    ks = rng.uniform(0, 1, (B, H, S)).astype(np.float32)
    vq, vs = kq.copy(), ks.copy()
    pos = np.array([0, 39, 17, -3, 40], dtype=np.int32)       # the last two are outside the cache
    kn = _bits((B, H, D), 2.0, (mode, 3))
    vn = _bits((B, H, D), 0.5, (mode, 4))
    say("kv append", mode)
    cache = (_dev(kq), _dev(ks), _dev(vq), _dev(vs))
    fp8q.fp8_kv_cache_append(synth_dev(kn), synth_dev(vn), _dev(pos), cache, mode=mode)
    torch.cuda.synchronize()
    okq, oks = oracle.kv_cache_append(kn, pos, kq.copy(), ks.copy(), mode)
    ovq, ovs = oracle.kv_cache_append(vn, pos, vq.copy(), vs.copy(), mode)
    assert_bytes_equal(cache[0].cpu().numpy(), okq, "k cache")
    assert_scales_equal(cache[1].cpu().numpy(), oks, "k scales")
    assert_bytes_equal(cache[2].cpu().numpy(), ovq, "v cache")
    assert_scales_equal(cache[3].cpu().numpy(), ovs, "v scales")


def synth_dev(bits):
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to("cuda:0")


@pytest.mark.parametrize("grp", [1, 2, 4, 8])
def test_decode_ragged_lengths(grp):
    """Lengths 0, 1, 63, 64, 65, 200 and the full cache (256), every group
    size; several tiles per wave and partial last tiles."""
    require_gpu()
    Hkv = 2
    Hq = grp * Hkv
    lens = np.array([0, 1, 63, 64, 65, 200, 256], dtype=np.int32)
    B, S = lens.size, 256
    cache = _cache(B, Hkv, S, seed=grp)
    qq, qs = _query(B, Hq, seed=grp)
    say("attention decode", grp, lens.tolist())
    y = _run(qq, qs, cache, lens)
    ref = oracle.attention_decode_f64(qq, qs, *cache, lens)
    assert not y[0].any(), "a sequence with no tokens gives zeros"
    gemm_tolerance_check(y, ref, f"decode grp={grp}")


@pytest.mark.parametrize("split", [True, False])
def test_decode_chunk_edges(split):
    """14 (sequence, head) pairs: with a workspace the 3000-token cache is cut
    into 12 chunks of 256 tokens; lengths at and around tile and chunk edges,
    with and without the split, against the oracle."""
    require_gpu()
    B, Hkv, Hq, S = 7, 2, 8, 3000
    lens = np.array([0, 1, 255, 256, 257, 2500, 3000], dtype=np.int32)
    cache = _cache(B, Hkv, S, seed=41)
    qq, qs = _query(B, Hq, seed=41)
    say("attention chunk edges", split)
    y = _run(qq, qs, cache, lens, workspace="auto" if split else None)
    gemm_tolerance_check(y, oracle.attention_decode_f64(qq, qs, *cache, lens), f"chunk edges split={split}")
    assert not y[0].any()


def test_decode_peaked_and_flat_scores():
    """Scores spread over a wide range (q and k with std 8: some weights near
    1, most near 0) and all-equal scores (zero keys: the mean of the values)."""
    require_gpu()
    B, Hkv, Hq, S = 3, 2, 8, 700
    lens = np.array([700, 513, 130], dtype=np.int32)
    cache = _cache(B, Hkv, S, seed=31, kstd=8.0)
    qq, qs = _query(B, Hq, seed=31, std=8.0)
    say("attention peaked")
    gemm_tolerance_check(_run(qq, qs, cache, lens), oracle.attention_decode_f64(qq, qs, *cache, lens), "peaked")
    kq, ks, vq, vs = cache
    flat = (np.zeros_like(kq), ks, vq, vs)
    say("attention flat")
    gemm_tolerance_check(_run(qq, qs, flat, lens), oracle.attention_decode_f64(qq, qs, *flat, lens), "flat")


@pytest.mark.parametrize("mode", [0, 1])
def test_decode_after_appends_end_to_end(mode):
    """The GPU quantizes the query and appends K/V step by step; the result
    equals the oracle's attention on the oracle's quantization of the same
    rows (the quantizers are bit-exact, so both see identical codes)."""
    require_gpu()
    fp8q = lib()
    B, Hkv, Hq, S, steps = 4, 8, 32, 96, 90
    kq = torch.zeros((B, Hkv, S, D), dtype=torch.uint8, device="cuda")
    vq = torch.zeros_like(kq)
    ks = torch.zeros((B, Hkv, S), dtype=torch.float32, device="cuda")
    vs = torch.zeros_like(ks)
    okq, ovq = np.zeros((B, Hkv, S, D), np.uint8), np.zeros((B, Hkv, S, D), np.uint8)
    oks, ovs = np.zeros((B, Hkv, S), np.float32), np.zeros((B, Hkv, S), np.float32)
    start = np.array([0, 5, 2, 6], dtype=np.int32)                 # ragged positions
    say("attention end to end", mode)
    for t in range(steps):
        kn = _bits((B, Hkv, D), 1.0, (mode, 10 + t))
        vn = _bits((B, Hkv, D), 1.0, (mode, 500 + t))
        pos = start + t
        fp8q.fp8_kv_cache_append(synth_dev(kn), synth_dev(vn), _dev(pos), (kq, ks, vq, vs), mode=mode)
        oracle.kv_cache_append(kn, pos, okq, oks, mode)
        oracle.kv_cache_append(vn, pos, ovq, ovs, mode)
    qb = _bits((B * Hq, D), 1.0, (mode, 999))
    q_q, q_s = fp8q.fp8_quant_act_1x128(synth_dev(qb), mode)
    lens = start + steps
    y = fp8q.fp8_attention_decode(q_q.view(B, Hq, D), q_s.view(B, Hq), (kq, ks, vq, vs), _dev(lens))
    torch.cuda.synchronize()
    oqq, oqs = oracle.quant_act_1x128(qb, mode)
    assert_bytes_equal(kq.cpu().numpy(), okq, "k cache")
    assert_bytes_equal(vq.cpu().numpy(), ovq, "v cache")
    ref = oracle.attention_decode_f64(oqq.reshape(B, Hq, D), oqs.reshape(B, Hq), okq, oks, ovq, ovs, lens)
    gemm_tolerance_check(y.float().cpu().numpy().astype(np.float64), ref, f"end to end mode {mode}")


def test_llama_decode_full_size_sampled():
    """Llama-3.1-8B decode shape: 64 sequences, 32 query / 8 key-value heads,
    8192-token cache, lengths drawn in [1, 8192]; every sequence's first and
    last groups and a few more checked against the oracle."""
    require_gpu()
    fp8q = lib()
    B, Hq, Hkv, S = 64, 32, 8, 8192
    g = torch.Generator(device="cuda").manual_seed(synth.seed_of(17, 64, 0))
    kq = (torch.randn((B, Hkv, S, D), device="cuda", generator=g) * 32).clamp(-448, 448).to(torch.float8_e4m3fn)
    vq = (torch.randn((B, Hkv, S, D), device="cuda", generator=g) * 32).clamp(-448, 448).to(torch.float8_e4m3fn)
    ks = torch.rand((B, Hkv, S), device="cuda", generator=g) * 0.01 + 0.001
    vs = torch.rand((B, Hkv, S), device="cuda", generator=g) * 0.01 + 0.001
    rng = np.random.default_rng(64)
    lens = rng.integers(1, S + 1, B).astype(np.int32)
    qb = _bits((B * Hq, D), 1.0, (64, 5))
    q_q, q_s = fp8q.fp8_quant_act_1x128(synth_dev(qb))
    say("attention llama decode full size")
    y = fp8q.fp8_attention_decode(q_q.view(B, Hq, D), q_s.view(B, Hq), (kq.view(torch.uint8), ks, vq.view(torch.uint8), vs),
                                  _dev(lens))
    torch.cuda.synchronize()
    hq, hs = q_q.view(B, Hq, D).cpu().numpy(), q_s.view(B, Hq).cpu().numpy()
    pick = np.unique(np.concatenate([[0, B - 1], rng.integers(0, B, 6)]))
    got, ref = [], []
    for b in pick:
        sl = slice(b, b + 1)
        c = (kq[sl].view(torch.uint8).cpu().numpy(), ks[sl].cpu().numpy(),
             vq[sl].view(torch.uint8).cpu().numpy(), vs[sl].cpu().numpy())
        ref.append(oracle.attention_decode_f64(hq[sl], hs[sl], *c, lens[sl])[0])
        got.append(y[b].float().cpu().numpy().astype(np.float64))
    gemm_tolerance_check(np.stack(got), np.stack(ref), "llama decode sampled")
