"""The allocation-free decode attention (fp8_attention_decode_noalloc), called
through the C ABI, gives the same output bits as fp8_attention_decode with a
workspace, on two calls in a row (the second with a smaller input), both on
the chunked path that uses the library's static scratch array."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import assert_bytes_equal, gemm_tolerance_check, lib, require_gpu, say

pytestmark = pytest.mark.gpu
D = 128


def _dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to("cuda:0")


def _case(B, Hq, Hkv, S, seed):
    rng = np.random.default_rng(seed)
    kb = synth.bf16_bits(synth.normal_bf16((B * Hkv * S, D), 1.0, synth.seed_of(23, seed, 0)))
    vb = synth.bf16_bits(synth.normal_bf16((B * Hkv * S, D), 1.0, synth.seed_of(23, seed, 1)))
    qb = synth.bf16_bits(synth.normal_bf16((B * Hq, D), 1.0, synth.seed_of(23, seed, 2)))
    kq, ks = oracle.quant_act_1x128(kb, 0)
    vq, vs = oracle.quant_act_1x128(vb, 0)
    qq, qs = oracle.quant_act_1x128(qb, 0)
    seq = rng.integers(0, S + 1, B).astype(np.int32)
    seq[0], seq[-1] = S, 0
    host = (qq.reshape(B, Hq, D), qs.reshape(B, Hq), kq.reshape(B, Hkv, S, D), ks.reshape(B, Hkv, S),
            vq.reshape(B, Hkv, S, D), vs.reshape(B, Hkv, S), seq)
    return host, tuple(_dev(a) for a in host)


def _ptr(t):
    return ctypes.c_void_p(int(t.data_ptr()))


def _one_call(B, Hq, Hkv, S, seed):
    fp8q = lib()
    from blockwise_scaled_fp8_quant_amd import _lib
    c = _lib.load()
    host, (qq, qs, kq, ks, vq, vs, seq) = _case(B, Hq, Hkv, S, seed)
    need = c.fp8_attention_decode_workspace_size(B, Hq, Hkv, S)
    assert need > 0, "the case must take the chunked path"
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda:0")
    y_ref = torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda:0")
    y = torch.full((B, Hq, D), float("nan"), dtype=torch.bfloat16, device="cuda:0")
    say("attention decode with workspace", B, Hq, Hkv, S)
    st = c.fp8_attention_decode(_ptr(qq), _ptr(qs), _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs), _ptr(seq), _ptr(y_ref),
                                B, Hq, Hkv, S, _ptr(ws), need, stream)
    assert st == 0, c.fp8q_last_error()
    say("attention decode noalloc", B, Hq, Hkv, S)
    st = c.fp8_attention_decode_noalloc(_ptr(qq), _ptr(qs), _ptr(kq), _ptr(ks), _ptr(vq), _ptr(vs), _ptr(seq),
                                        _ptr(y), B, Hq, Hkv, S, stream)
    assert st == 0, c.fp8q_last_error()
    torch.cuda.synchronize()
    got = y.cpu().view(torch.int16).numpy()
    want = y_ref.cpu().view(torch.int16).numpy()
    assert_bytes_equal(got, want, f"noalloc vs workspace {B}x{Hq}x{Hkv}x{S}")
    ref = oracle.attention_decode_f64(*host)
    gemm_tolerance_check(y.float().cpu().numpy().astype(np.float64), ref, "noalloc vs oracle")


def test_noalloc_matches_workspace_call_twice():
    require_gpu()
    _one_call(12, 32, 8, 3000, seed=1)   # 96 (sequence, head) pairs: chunked
    _one_call(3, 16, 4, 700, seed=2)     # smaller input, reusing the scratch
