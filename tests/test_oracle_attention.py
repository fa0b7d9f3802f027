"""Pins of the oracle's FP8 KV cache and FP8 decode attention.

Extending FP8 to the KV cache and to attention is what takes the recipe from
15-25% on the linear layers to about 48% end to end (page "NVIDIA NeMo RL
erreicht 48% Geschwindigkeitssteigerung ...", section "Leistungsgewinne in der
Praxis").  Pins, none of which uses the function under test:
  - torch's scaled_dot_product_attention in float64 on the dequantized
    operands, the grouped key/value heads expanded by repeat_interleave;
  - closed forms: one cached token gives its value row; equal scores give the
    mean of the value rows; two tokens give sigmoid weights;
  - tokens at or past seq_len, and other key/value heads, change nothing;
  - the cache append against the 1x128 row quantizer, placed by position.
Many query tokens (causal over the cache, query t at position start + t):
  - torch's scaled_dot_product_attention in float64 with an explicit boolean
    mask (key position <= query position);
  - closed forms: position 0 gives value row 0, equal scores give prefix means;
  - later cache rows and other heads change nothing; a query before position
    0 gives zeros; one query token at position p equals decode over p + 1;
  - the multi-token append against the row quantizer, placed at start + t.
"""
import math

import numpy as np
import pytest
import torch

from tests.test_oracle_quant import _bf16

D = 128


def _dec(q):
    return torch.from_numpy(np.ascontiguousarray(q)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _codes(rng, shape):
    finite = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    return rng.choice(finite, size=shape).astype(np.uint8)


def _inputs(rng, B, Hq, Hkv, S):
    qq = _codes(rng, (B, Hq, D))
    qs = rng.uniform(1e-3, 4e-3, size=(B, Hq)).astype(np.float32)
    kq, vq = _codes(rng, (B, Hkv, S, D)), _codes(rng, (B, Hkv, S, D))
    ks = rng.uniform(1e-3, 4e-3, size=(B, Hkv, S)).astype(np.float32)
    vs = rng.uniform(1e-3, 1e-2, size=(B, Hkv, S)).astype(np.float32)
    return qq, qs, kq, ks, vq, vs


def test_against_torch_sdpa(oracle_lib):
    rng = np.random.default_rng(1)
    B, Hq, Hkv, S = 3, 8, 2, 40
    qq, qs, kq, ks, vq, vs = _inputs(rng, B, Hq, Hkv, S)
    seq_len = np.array([40, 17, 1], dtype=np.int32)
    o = oracle_lib.attention_decode_f64(qq, qs, kq, ks, vq, vs, seq_len)
    for b in range(B):
        L = seq_len[b]
        q = torch.from_numpy(_dec(qq[b]) * qs[b][:, None].astype(np.float64))[:, None, :]       # [Hq, 1, D]
        k = torch.from_numpy(_dec(kq[b, :, :L]) * ks[b, :, :L, None].astype(np.float64))
        v = torch.from_numpy(_dec(vq[b, :, :L]) * vs[b, :, :L, None].astype(np.float64))
        k = k.repeat_interleave(Hq // Hkv, dim=0)
        v = v.repeat_interleave(Hq // Hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v)[:, 0, :].numpy()
        assert np.allclose(o[b], ref, rtol=1e-12, atol=1e-15), b


def test_single_token_returns_its_value_row(oracle_lib):
    rng = np.random.default_rng(2)
    qq, qs, kq, ks, vq, vs = _inputs(rng, 2, 4, 1, 5)
    o = oracle_lib.attention_decode_f64(qq, qs, kq, ks, vq, vs, np.array([1, 1]))
    for b in range(2):
        row = _dec(vq[b, 0, 0]) * float(vs[b, 0, 0])
        assert np.array_equal(o[b], np.broadcast_to(row, (4, D)))


def test_equal_scores_average_the_values(oracle_lib):
    rng = np.random.default_rng(3)
    qq, qs, kq, ks, vq, vs = _inputs(rng, 1, 4, 1, 9)
    kq[:] = 0                                   # every score is 0
    o = oracle_lib.attention_decode_f64(qq, qs, kq, ks, vq, vs, np.array([9]))
    mean = (_dec(vq[0, 0]) * vs[0, 0, :, None].astype(np.float64)).mean(axis=0)
    assert np.allclose(o[0], mean[None, :], rtol=1e-14, atol=0)


def test_two_tokens_sigmoid_weights(oracle_lib):
    """Scores d1 and d2 with q = e0 * 1, k_t = c_t e0: the weights are a
    sigmoid of (d1 - d2) / sqrt(D)."""
    qq = np.zeros((1, 1, D), np.uint8)
    qq[0, 0, 0] = 0x38                          # 1.0
    qs = np.ones((1, 1), np.float32)
    kq = np.zeros((1, 1, 2, D), np.uint8)
    kq[0, 0, 0, 0] = 0x58                       # 16.0
    kq[0, 0, 1, 0] = 0x48                       # 4.0
    ks = np.ones((1, 1, 2), np.float32)
    vq = np.zeros((1, 1, 2, D), np.uint8)
    vq[0, 0, 0, 1] = 0x38                       # v_0 = e1
    vq[0, 0, 1, 2] = 0x38                       # v_1 = e2
    vs = np.ones((1, 1, 2), np.float32)
    o = oracle_lib.attention_decode_f64(qq, qs, kq, ks, vq, vs, np.array([2]))
    w0 = 1.0 / (1.0 + math.exp(-(16.0 - 4.0) / math.sqrt(D)))
    assert math.isclose(o[0, 0, 1], w0, rel_tol=1e-14)
    assert math.isclose(o[0, 0, 2], 1.0 - w0, rel_tol=1e-13)
    assert o[0, 0, 0] == 0.0 and not o[0, 0, 3:].any()


def test_masking_and_head_groups(oracle_lib):
    """Tokens at or past seq_len and the other key/value heads do not enter an
    output; a sequence of length 0 gives zeros."""
    rng = np.random.default_rng(4)
    qq, qs, kq, ks, vq, vs = _inputs(rng, 2, 8, 2, 30)
    seq_len = np.array([20, 0])
    o = oracle_lib.attention_decode_f64(qq, qs, kq, ks, vq, vs, seq_len)
    kq2, vq2 = kq.copy(), vq.copy()
    kq2[0, :, 20:] = _codes(rng, kq2[0, :, 20:].shape)
    vq2[0, :, 20:] = _codes(rng, vq2[0, :, 20:].shape)
    kq2[0, 1] = _codes(rng, kq2[0, 1].shape)      # key/value head 1 serves query heads 4..7
    o2 = oracle_lib.attention_decode_f64(qq, qs, kq2, ks, vq2, vs, seq_len)
    assert np.array_equal(o[0, :4], o2[0, :4])
    assert not np.allclose(o[0, 4:], o2[0, 4:])
    assert not o[1].any()


@pytest.mark.parametrize("mode", [0, 1])
def test_cache_append_places_quantized_rows(oracle_lib, mode):
    rng = np.random.default_rng(5 + mode)
    B, H, S = 3, 2, 6
    new = _bf16(rng.standard_normal((B, H, D)).astype(np.float32))
    cq = np.full((B, H, S, D), 0x11, np.uint8)
    cs = np.full((B, H, S), 7.0, np.float32)
    pos = np.array([0, 5, 9])                    # the last is outside the cache
    cq, cs = oracle_lib.kv_cache_append(new, pos, cq, cs, mode)
    q, s = oracle_lib.quant_act_1x128(new.reshape(B * H, D), mode)
    q, s = q.reshape(B, H, D), s.reshape(B, H)
    assert np.array_equal(cq[0, :, 0], q[0]) and np.array_equal(cs[0, :, 0], s[0])
    assert np.array_equal(cq[1, :, 5], q[1]) and np.array_equal(cs[1, :, 5], s[1])
    untouched = np.ones((B, S), bool)
    untouched[0, 0] = untouched[1, 5] = False
    for b in range(B):
        for t in range(S):
            if untouched[b, t]:
                assert (cq[b, :, t] == 0x11).all() and (cs[b, :, t] == 7.0).all()


# ---------------------------------------------------------------------------
# Many query tokens (prefill / training forward): causal over the cache, query
# t of sequence b at position start[b] + t.
# ---------------------------------------------------------------------------

def _prefill_inputs(rng, B, T, Hq, Hkv, S):
    qq = _codes(rng, (B, T, Hq, D))
    qs = rng.uniform(1e-3, 4e-3, size=(B, T, Hq)).astype(np.float32)
    kq, vq = _codes(rng, (B, Hkv, S, D)), _codes(rng, (B, Hkv, S, D))
    ks = rng.uniform(1e-3, 4e-3, size=(B, Hkv, S)).astype(np.float32)
    vs = rng.uniform(1e-3, 1e-2, size=(B, Hkv, S)).astype(np.float32)
    return qq, qs, kq, ks, vq, vs


def test_prefill_against_torch_sdpa_causal_mask(oracle_lib):
    """torch's scaled_dot_product_attention in float64 with an explicit boolean
    mask (key position <= query position, below S), heads expanded."""
    rng = np.random.default_rng(11)
    B, T, Hq, Hkv, S = 3, 21, 8, 2, 40
    qq, qs, kq, ks, vq, vs = _prefill_inputs(rng, B, T, Hq, Hkv, S)
    start = np.array([0, 12, 30], dtype=np.int32)       # the last runs past S
    o = oracle_lib.attention_prefill_f64(qq, qs, kq, ks, vq, vs, start)
    for b in range(B):
        pos = start[b] + np.arange(T)
        mask = torch.from_numpy(np.arange(S)[None, :] <= pos[:, None])           # [T, S]
        q = torch.from_numpy((_dec(qq[b]) * qs[b][:, :, None].astype(np.float64)).transpose(1, 0, 2))  # [Hq, T, D]
        k = torch.from_numpy(_dec(kq[b]) * ks[b][:, :, None].astype(np.float64))
        v = torch.from_numpy(_dec(vq[b]) * vs[b][:, :, None].astype(np.float64))
        k = k.repeat_interleave(Hq // Hkv, dim=0)
        v = v.repeat_interleave(Hq // Hkv, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask).numpy()
        assert np.allclose(o[b].transpose(1, 0, 2), ref, rtol=1e-12, atol=1e-15), b


def test_prefill_position_zero_and_prefix_means(oracle_lib):
    """The query at position 0 returns value row 0; with every score equal the
    query at position p returns the mean of value rows 0..p."""
    rng = np.random.default_rng(12)
    B, T, Hq, Hkv, S = 1, 9, 4, 1, 9
    qq, qs, kq, ks, vq, vs = _prefill_inputs(rng, B, T, Hq, Hkv, S)
    o = oracle_lib.attention_prefill_f64(qq, qs, kq, ks, vq, vs, np.array([0]))
    v = _dec(vq[0, 0]) * vs[0, 0, :, None].astype(np.float64)
    assert np.array_equal(o[0, 0], np.broadcast_to(v[0], (Hq, D)))
    kq[:] = 0
    o = oracle_lib.attention_prefill_f64(qq, qs, kq, ks, vq, vs, np.array([0]))
    for t in range(T):
        assert np.allclose(o[0, t], v[:t + 1].mean(axis=0)[None, :], rtol=1e-14, atol=0), t


def test_prefill_future_tokens_and_other_heads_do_not_enter(oracle_lib):
    """Cache rows after a query's position, and the other key/value heads, do not
    change its output; a query before position 0 gives zeros."""
    rng = np.random.default_rng(13)
    B, T, Hq, Hkv, S = 2, 6, 4, 2, 20
    qq, qs, kq, ks, vq, vs = _prefill_inputs(rng, B, T, Hq, Hkv, S)
    start = np.array([4, -3])
    o = oracle_lib.attention_prefill_f64(qq, qs, kq, ks, vq, vs, start)
    kq2, vq2 = kq.copy(), vq.copy()
    kq2[0, :, 7:] = _codes(rng, kq2[0, :, 7:].shape)      # positions 7.. (queries 0..3 sit at 4..7)
    vq2[0, :, 7:] = _codes(rng, vq2[0, :, 7:].shape)
    kq2[0, 1] = _codes(rng, kq2[0, 1].shape)              # head 1 serves query heads 2, 3
    o2 = oracle_lib.attention_prefill_f64(qq, qs, kq2, ks, vq2, vs, start)
    assert np.array_equal(o[0, :3, :2], o2[0, :3, :2])
    assert not np.allclose(o[0, :3, 2:], o2[0, :3, 2:])
    assert not o[1, :3].any() and o[1, 3:].any()            # positions -3..-1 see nothing


def test_prefill_single_query_is_decode(oracle_lib):
    """One query token at position p is decode attention over p + 1 tokens."""
    rng = np.random.default_rng(14)
    B, Hq, Hkv, S = 3, 8, 2, 30
    qq, qs, kq, ks, vq, vs = _prefill_inputs(rng, B, 1, Hq, Hkv, S)
    start = np.array([0, 17, 40])
    o = oracle_lib.attention_prefill_f64(qq, qs, kq, ks, vq, vs, start)
    od = oracle_lib.attention_decode_f64(qq[:, 0], qs[:, 0], kq, ks, vq, vs, start + 1)
    assert np.allclose(o[:, 0], od, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("mode", [0, 1])
def test_cache_append_tokens_places_quantized_rows(oracle_lib, mode):
    """T rows per sequence land at start[b] + t as the 1x128 row quantizer
    codes them; positions outside the cache store nothing."""
    rng = np.random.default_rng(15 + mode)
    B, T, H, S = 3, 4, 2, 6
    new = _bf16(rng.standard_normal((B, T, H, D)).astype(np.float32))
    cq = np.full((B, H, S, D), 0x11, np.uint8)
    cs = np.full((B, H, S), 7.0, np.float32)
    start = np.array([0, 4, -2])
    cq, cs = oracle_lib.kv_cache_append_tokens(new, start, cq, cs, mode)
    q, s = oracle_lib.quant_act_1x128(new.reshape(B * T * H, D), mode)
    q, s = q.reshape(B, T, H, D), s.reshape(B, T, H)
    written = np.zeros((B, S), bool)
    for b in range(B):
        for t in range(T):
            p = start[b] + t
            if 0 <= p < S:
                written[b, p] = True
                assert np.array_equal(cq[b, :, p], q[b, t]) and np.array_equal(cs[b, :, p], s[b, t])
    assert written.sum() == 4 + 2 + 2
    for b in range(B):
        for p in range(S):
            if not written[b, p]:
                assert (cq[b, :, p] == 0x11).all() and (cs[b, :, p] == 7.0).all()
