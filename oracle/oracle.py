"""ctypes front end of the C oracle (fp8q_oracle.c).

TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Every function takes and returns numpy
arrays on the host.  bf16 tensors are passed as their raw uint16 bit patterns,
E4M3 tensors as raw uint8 codes, scales as float32.
"""
import ctypes
import os
import subprocess

import numpy as np

MODE_AMAX = 0
MODE_POW2 = 1

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fp8q_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

_CFLAGS = ["-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math"]


def build(force=True):
    """Compile the oracle library with gcc (no fast-math, no contraction)."""
    if not force and os.path.exists(_LIB):
        return _LIB
    tmp = _LIB + ".tmp"
    subprocess.run(["gcc", *_CFLAGS, "-o", tmp, _SRC, "-lm"], check=True)
    os.replace(tmp, _LIB)
    return _LIB


_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB):
        build()
    lib = ctypes.CDLL(_LIB)
    p = ctypes.c_void_p
    i64 = ctypes.c_int64
    i32 = ctypes.c_int32
    lib.oracle_e4m3_decode.restype = ctypes.c_double
    lib.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
    lib.oracle_e4m3_decode_table.argtypes = [p]
    lib.oracle_e4m3_encode.restype = ctypes.c_uint8
    lib.oracle_e4m3_encode.argtypes = [ctypes.c_float]
    lib.oracle_e4m3_encode_array.argtypes = [p, i64, p]
    lib.oracle_block_scale.restype = ctypes.c_float
    lib.oracle_block_scale.argtypes = [ctypes.c_float, ctypes.c_int]
    lib.oracle_quant_act_1x128.argtypes = [p, i64, i64, ctypes.c_int, p, p]
    lib.oracle_quant_weight_128x128.argtypes = [p, i64, i64, ctypes.c_int, p, p]
    lib.oracle_gemm_f64.argtypes = [p, p, p, p, i64, i64, i64, p]
    lib.oracle_gemm_sampled_f64.argtypes = [p, p, p, p, i64, i64, i64, p, p, i64, p]
    lib.oracle_grouped_gemm_f64.argtypes = [p, p, p, p, p, i32, i64, i64, i64, p]
    lib.oracle_grouped_gemm_sampled_f64.argtypes = [p, p, p, p, i64, i64, p, p, p, i64, p]
    lib.oracle_num_threads.restype = ctypes.c_int
    lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
    lib.oracle_set_num_threads.restype = None
    _lib = lib
    return lib


def _ptr(a):
    return ctypes.c_void_p(a.ctypes.data)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


def num_threads():
    return _load().oracle_num_threads()


def set_num_threads(n):
    """Threads of the following oracle calls (n < 1: the OpenMP default)."""
    _load().oracle_set_num_threads(int(n))


def e4m3_decode_table():
    out = np.empty(256, dtype=np.float64)
    _load().oracle_e4m3_decode_table(_ptr(out))
    return out


def e4m3_encode(r):
    """Encode float32 values (any shape) to E4M3 codes (RNE, saturating)."""
    r = _c(np.asarray(r, dtype=np.float32), np.float32)
    q = np.empty(r.shape, dtype=np.uint8)
    _load().oracle_e4m3_encode_array(_ptr(r), r.size, _ptr(q))
    return q


def block_scale(amax, mode):
    """Scale for one block of largest magnitude amax (vectorised loop)."""
    lib = _load()
    a = np.asarray(amax, dtype=np.float32)
    out = np.empty(a.shape, dtype=np.float32)
    flat_in, flat_out = a.reshape(-1), out.reshape(-1)
    for i in range(flat_in.size):
        flat_out[i] = lib.oracle_block_scale(float(flat_in[i]), mode)
    return out


def quant_act_1x128(x_bits, mode=MODE_AMAX):
    """x_bits: uint16 [M, K] bf16 bits.  Returns (q uint8 [M, K], s f32 [M, K/128])."""
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    if K % 128:
        raise ValueError("K must be a multiple of 128")
    q = np.empty((M, K), dtype=np.uint8)
    s = np.empty((M, K // 128), dtype=np.float32)
    _load().oracle_quant_act_1x128(_ptr(x), M, K, mode, _ptr(q), _ptr(s))
    return q, s


def quant_weight_128x128(w_bits, mode=MODE_AMAX):
    """w_bits: uint16 [N, K] bf16 bits.  Returns (q uint8 [N, K], s f32 [N/128, K/128])."""
    w = _c(w_bits, np.uint16)
    N, K = w.shape
    if K % 128 or N % 128:
        raise ValueError("N and K must be multiples of 128")
    q = np.empty((N, K), dtype=np.uint8)
    s = np.empty((N // 128, K // 128), dtype=np.float32)
    _load().oracle_quant_weight_128x128(_ptr(w), N, K, mode, _ptr(q), _ptr(s))
    return q, s


def gemm_f64(aq, as_, bq, bs):
    """Y[M, N] (fp64) = dequant(aq, as_) @ dequant(bq, bs)^T."""
    aq = _c(aq, np.uint8)
    bq = _c(bq, np.uint8)
    as_ = _c(as_, np.float32)
    bs = _c(bs, np.float32)
    M, K = aq.shape
    N = bq.shape[0]
    y = np.empty((M, N), dtype=np.float64)
    _load().oracle_gemm_f64(_ptr(aq), _ptr(as_), _ptr(bq), _ptr(bs), M, N, K, _ptr(y))
    return y


def round_bf16(y):
    """fp64 values -> bf16 bit patterns (uint16), rounded once to the nearest
    bf16 with ties to an even mantissa (IEEE-754 round-to-nearest-even at 8
    significant bits; below 2^-126 the bf16 spacing is 2^-133).  Finite
    inputs of magnitude below the bf16 overflow threshold."""
    y = np.asarray(y, dtype=np.float64)
    _, e = np.frexp(y)                        # |y| = m * 2^e, 0.5 <= m < 1
    step = np.ldexp(1.0, np.maximum(e - 8, -133))   # bf16 spacing at |y|
    r = np.round(y / step) * step             # exact quotient; round half to even
    r = np.where(y == 0.0, y, r)              # keeps -0.0
    return (r.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)


def gemm_quant_1x128(aq, as_, bq, bs, mode=MODE_AMAX):
    """The GEMM output Y = dequant(aq, as_) @ dequant(bq, bs)^T, rounded once to
    bf16, then quantized for the next layer in 1x128 blocks along N by the same
    rule as quant_act_1x128.  Returns (q uint8 [M, N], s f32 [M, N/128])."""
    return quant_act_1x128(round_bf16(gemm_f64(aq, as_, bq, bs)), mode)


def gemm_sampled_f64(aq, as_, bq, bs, ms, ns):
    aq = _c(aq, np.uint8)
    bq = _c(bq, np.uint8)
    as_ = _c(as_, np.float32)
    bs = _c(bs, np.float32)
    ms = _c(np.asarray(ms, dtype=np.int64), np.int64)
    ns = _c(np.asarray(ns, dtype=np.int64), np.int64)
    M, K = aq.shape
    N = bq.shape[0]
    y = np.empty(ms.shape, dtype=np.float64)
    _load().oracle_gemm_sampled_f64(_ptr(aq), _ptr(as_), _ptr(bq), _ptr(bs), M, N, K,
                                    _ptr(ms), _ptr(ns), ms.size, _ptr(y))
    return y


def grouped_gemm_f64(aq, as_, bq, bs, offsets):
    """aq [M_total, K], bq [G, N, K], bs [G, N/128, K/128], offsets int32 [G+1]."""
    aq = _c(aq, np.uint8)
    bq = _c(bq, np.uint8)
    as_ = _c(as_, np.float32)
    bs = _c(bs, np.float32)
    off = _c(np.asarray(offsets, dtype=np.int32), np.int32)
    M, K = aq.shape
    G, N, _ = bq.shape
    y = np.zeros((M, N), dtype=np.float64)
    _load().oracle_grouped_gemm_f64(_ptr(aq), _ptr(as_), _ptr(bq), _ptr(bs), _ptr(off),
                                    G, M, N, K, _ptr(y))
    return y


def grouped_gemm_sampled_f64(aq, as_, bq, bs, groups, ms, ns):
    aq = _c(aq, np.uint8)
    bq = _c(bq, np.uint8)
    as_ = _c(as_, np.float32)
    bs = _c(bs, np.float32)
    grp = _c(np.asarray(groups, dtype=np.int32), np.int32)
    ms = _c(np.asarray(ms, dtype=np.int64), np.int64)
    ns = _c(np.asarray(ns, dtype=np.int64), np.int64)
    K = aq.shape[1]
    N = bq.shape[1]
    y = np.empty(ms.shape, dtype=np.float64)
    _load().oracle_grouped_gemm_sampled_f64(_ptr(aq), _ptr(as_), _ptr(bq), _ptr(bs), N, K,
                                            _ptr(grp), _ptr(ms), _ptr(ns), ms.size, _ptr(y))
    return y


# ---------------------------------------------------------------------------
# Backward pass of the linear layer Y = X W^T.  Page 1 trains end to end in FP8
# ("Der technische Durchbruch": FP8 applied in generation and in training
# alike) with E4M3 blocks of 1x128 for activations and 128x128 for weights,
# and prints no other layout for the gradient GEMMs.  The reading taken here
# puts every scale block along the contraction dimension of its GEMM, as in
# the forward pass, so one scale pair factors out of each 128-long partial
# sum:
#   dX = dY W    dY in 1x128 blocks along N (its rows); W in its 128x128 tiles.
#   dW = dY^T X  dY and X in blocks of 128 tokens x 1 channel (128x1, along M),
#                stored transposed ([channels][Mp]) so that the contraction
#                runs along rows; Mp = M rounded up to a multiple of 128, the
#                padding holding zero codes.
# ---------------------------------------------------------------------------

def quant_act_colwise_t(x_bits, mode=MODE_AMAX):
    """Blocks of 128 rows x 1 column of x [M, K] (bf16 bits), stored transposed.

    Column k, rows 128*mb .. 128*mb+127 form one block, quantized by the same
    rule as a 1x128 activation block; rows past M count as +0.  Written out:
    the block is row k, block mb of the zero-padded transpose of x.
    Returns (q_t uint8 [K, Mp], s_t f32 [K, Mp/128]).
    """
    x = _c(x_bits, np.uint16)
    M, K = x.shape
    Mp = -(-M // 128) * 128
    xt = np.zeros((K, Mp), dtype=np.uint16)
    xt[:, :M] = x.T
    return quant_act_1x128(xt, mode)


def quant_weight_128x128_t(w_bits, mode=MODE_AMAX):
    """The 128x128-tile quantization of w [N, K] in the transposed layout the
    data-gradient GEMM reads: (q_t uint8 [K, N], s_t f32 [K/128, N/128]) with
    q_t = q^T and s_t = s^T (a tile and its transpose hold the same values)."""
    q, s = quant_weight_128x128(w_bits, mode)
    return np.ascontiguousarray(q.T), np.ascontiguousarray(s.T)


def gemm_dgrad_f64(gq, gs, wq, ws):
    """dX [M, K] (fp64) = dequant(gq, gs) @ dequant(wq, ws).

    gq [M, N] with scales gs [M, N/128] (1x128 along N); wq [N, K] with scales
    ws [N/128, K/128] (the forward weight tiles).  Written as the block-scaled
    GEMM with the weight operand transposed: operand row k of W^T is column k
    of W, and tile (kb, nb) of W^T has the scale of tile (nb, kb) of W.
    """
    return gemm_f64(gq, gs, np.ascontiguousarray(_c(wq, np.uint8).T),
                    np.ascontiguousarray(_c(ws, np.float32).T))


def gemm_dgrad_sampled_f64(gq, gs, wq, ws, ms, ks):
    """dX[ms[i], ks[i]] of gemm_dgrad_f64, for outputs chosen one by one."""
    return gemm_sampled_f64(gq, gs, np.ascontiguousarray(_c(wq, np.uint8).T),
                            np.ascontiguousarray(_c(ws, np.float32).T), ms, ks)


def _dequant_rows(q, s):
    """fp64 values of codes q [R, C] with one scale per 1x128 block of a row,
    s [R, C/128] (exact: 4-bit times 24-bit significands)."""
    table = e4m3_decode_table()
    return table[_c(q, np.uint8)] * np.repeat(_c(s, np.float32).astype(np.float64), 128, axis=1)


def gemm_wgrad_f64(gtq, gts, xtq, xts):
    """dW [N, K] (fp64) = dequant(gtq, gts) @ dequant(xtq, xts)^T.

    gtq [N, Mp], gts [N, Mp/128]: dY^T in 128-token blocks; xtq [K, Mp],
    xts [K, Mp/128]: X^T in 128-token blocks.  Every operand row has its own
    scale per block, on both sides:
        dW[n][k] = sum_mb gts[n][mb] * xts[k][mb] * sum_{m in mb} dec(gtq[n][m]) * dec(xtq[k][m]).
    Dequantization is exact in fp64; numpy's float64 matmul does the sums.
    """
    return _dequant_rows(gtq, gts) @ _dequant_rows(xtq, xts).T


def gemm_wgrad_sampled_f64(gtq, gts, xtq, xts, ns, ks):
    """dW[ns[i], ks[i]] of gemm_wgrad_f64, for outputs chosen one by one."""
    ns = np.asarray(ns, dtype=np.int64)
    ks = np.asarray(ks, dtype=np.int64)
    a = _dequant_rows(_c(gtq, np.uint8)[ns], _c(gts, np.float32)[ns])
    b = _dequant_rows(_c(xtq, np.uint8)[ks], _c(xts, np.float32)[ks])
    return np.einsum("ij,ij->i", a, b)


# ---------------------------------------------------------------------------
# FP8 KV cache and FP8 attention (page 1, "Leistungsgewinne in der Praxis":
# extending FP8 to the KV cache and to attention raises the end-to-end gain
# to about 48%).  The pages give no layout; the reading taken here applies
# the recipe's activation rule: every key and value row of one token and one
# key/value head (head dimension 128) is one 1x128 block with its own scale,
# and so is every query row of one query head.  Decode attention is the
# standard softmax(q k^T / sqrt(D)) v over the cached tokens, with grouped
# query heads (query head h reads key/value head h // (Hq / Hkv)).  With many
# query tokens (prefill, chunked prefill, a training forward pass) the plainest
# reading is causal attention over the cache: the query at position p sees the
# cached tokens 0..p, its own included.
# ---------------------------------------------------------------------------

def kv_cache_append(new_bits, pos, cache_q, cache_s, mode=MODE_AMAX):
    """Quantize one new row per sequence and key/value head and store it at
    token position pos[b]: new_bits uint16 [B, Hkv, D] (bf16), cache_q uint8
    [B, Hkv, S, D], cache_s f32 [B, Hkv, S] (updated in place and returned).
    A position outside [0, S) stores nothing."""
    new = _c(new_bits, np.uint16)
    B, H, D = new.shape
    q, s = quant_act_1x128(new.reshape(B * H, D), mode)
    q, s = q.reshape(B, H, D), s.reshape(B, H)
    for b in range(B):
        p = int(pos[b])
        if 0 <= p < cache_q.shape[2]:
            cache_q[b, :, p] = q[b]
            cache_s[b, :, p] = s[b]
    return cache_q, cache_s


def attention_decode_f64(qq, qs, kq, ks, vq, vs, seq_len):
    """One query token per sequence against its cached keys and values.

    qq uint8 [B, Hq, D], qs f32 [B, Hq]   query rows (1x128 blocks)
    kq, vq uint8 [B, Hkv, S, D], ks, vs f32 [B, Hkv, S]
    seq_len [B]: tokens 0 .. min(seq_len[b], S)-1 are attended; a sequence
    with none gives a zero output.
    Returns o [B, Hq, D] (fp64): every operand dequantized exactly, scores,
    softmax and the weighted sum of values in fp64.
    """
    table = e4m3_decode_table()
    qq, kq, vq = _c(qq, np.uint8), _c(kq, np.uint8), _c(vq, np.uint8)
    B, Hq, D = qq.shape
    Hkv, S = kq.shape[1], kq.shape[2]
    grp = Hq // Hkv
    o = np.zeros((B, Hq, D), dtype=np.float64)
    for b in range(B):
        L = min(int(seq_len[b]), S)
        if L <= 0:
            continue
        q = table[qq[b]] * np.asarray(qs[b], dtype=np.float64)[:, None]
        for g in range(Hkv):
            k = table[kq[b, g, :L]] * np.asarray(ks[b, g, :L], dtype=np.float64)[:, None]
            v = table[vq[b, g, :L]] * np.asarray(vs[b, g, :L], dtype=np.float64)[:, None]
            sc = q[g * grp:(g + 1) * grp] @ k.T / np.sqrt(D)
            sc -= sc.max(axis=1, keepdims=True)
            p = np.exp(sc)
            p /= p.sum(axis=1, keepdims=True)
            o[b, g * grp:(g + 1) * grp] = p @ v
    return o


def kv_cache_append_tokens(new_bits, start, cache_q, cache_s, mode=MODE_AMAX):
    """Quantize T new rows per sequence and key/value head and store token t of
    sequence b at position start[b] + t: new_bits uint16 [B, T, Hkv, D] (bf16,
    token-major as a projection writes its output), cache_q uint8
    [B, Hkv, S, D], cache_s f32 [B, Hkv, S] (updated in place and returned).
    A position outside [0, S) stores nothing."""
    new = _c(new_bits, np.uint16)
    B, T, H, D = new.shape
    q, s = quant_act_1x128(new.reshape(B * T * H, D), mode)
    q, s = q.reshape(B, T, H, D), s.reshape(B, T, H)
    S = cache_q.shape[2]
    for b in range(B):
        for t in range(T):
            p = int(start[b]) + t
            if 0 <= p < S:
                cache_q[b, :, p] = q[b, t]
                cache_s[b, :, p] = s[b, t]
    return cache_q, cache_s


def attention_prefill_f64(qq, qs, kq, ks, vq, vs, start):
    """Many query tokens per sequence (prefill, or a training forward pass)
    against the cached keys and values, causal.

    qq uint8 [B, T, Hq, D], qs f32 [B, T, Hq]   query rows (1x128 blocks),
        token-major as a projection writes them
    kq, vq uint8 [B, Hkv, S, D], ks, vs f32 [B, Hkv, S]
    start [B]: query t of sequence b sits at position start[b] + t and attends
    to the cached tokens 0 .. start[b] + t (itself included), those below S; a
    query with none gives a zero output.
    Returns o [B, T, Hq, D] (fp64): operands dequantized exactly, scores,
    softmax and the weighted sum of values in fp64.
    """
    table = e4m3_decode_table()
    qq, kq, vq = _c(qq, np.uint8), _c(kq, np.uint8), _c(vq, np.uint8)
    B, T, Hq, D = qq.shape
    Hkv, S = kq.shape[1], kq.shape[2]
    grp = Hq // Hkv
    o = np.zeros((B, T, Hq, D), dtype=np.float64)
    keys = np.arange(S)
    for b in range(B):
        pos = int(start[b]) + np.arange(T)
        allowed = keys[None, :] <= pos[:, None]                  # [T, S]
        live = allowed.any(axis=1)
        q = table[qq[b]] * np.asarray(qs[b], dtype=np.float64)[:, :, None]    # [T, Hq, D]
        for g in range(Hkv):
            k = table[kq[b, g]] * np.asarray(ks[b, g], dtype=np.float64)[:, None]
            v = table[vq[b, g]] * np.asarray(vs[b, g], dtype=np.float64)[:, None]
            for j in range(grp):
                h = g * grp + j
                sc = q[:, h, :] @ k.T / np.sqrt(D)                # [T, S]
                sc = np.where(allowed, sc, -np.inf)
                mx = np.where(live, sc.max(axis=1), 0.0)
                p = np.where(allowed, np.exp(sc - mx[:, None]), 0.0)
                den = p.sum(axis=1)
                p = p / np.where(live, den, 1.0)[:, None]
                o[b, :, h, :] = p @ v
    return o


# ---------------------------------------------------------------------------
# The gate+up projection of a SwiGLU MLP with its activation and the next
# layer's quantization fused (page 1, "Leistungsgewinne in der Praxis":
# quantization-kernel overhead is part of the gap to 2x; the Llama and Qwen3
# MLPs are SwiGLU).  Reading: the fused weight [2F][K] holds gate and up in
# alternating blocks of 128 rows (block 2p = gate rows 128p.., block 2p+1 =
# up rows 128p..), so one 256-row tile carries gate and up of the same 128
# output columns; gate and up are the GEMM's outputs rounded to bf16 (what a
# bf16-output GEMM would hand to a separate activation kernel); h = silu(g) * u
# = g / (1 + exp(-g)) * u, rounded to bf16, is quantized in 1x128 blocks by
# the activation rule.
# ---------------------------------------------------------------------------

def swiglu_split(y):
    """Columns of the fused gate+up output y [M, 2F] -> (gate [M, F], up [M, F])
    under the 128-block interleave."""
    y = np.asarray(y)
    M, N2 = y.shape
    blocks = y.reshape(M, N2 // 256, 2, 128)
    return blocks[:, :, 0, :].reshape(M, N2 // 2), blocks[:, :, 1, :].reshape(M, N2 // 2)


def bf16_to_f64(bits):
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def swiglu_h_f64(aq, as_, bq, bs):
    """h [M, F] in fp64 from the fused gate+up GEMM: silu(bf16(gate)) * bf16(up)
    before its final rounding."""
    y = bf16_to_f64(round_bf16(gemm_f64(aq, as_, bq, bs)))
    g, u = swiglu_split(y)
    return g / (1.0 + np.exp(-g)) * u


def gemm_swiglu_quant(aq, as_, bq, bs, mode=MODE_AMAX):
    """(h_q uint8 [M, F], h_s f32 [M, F/128]): h rounded to bf16 and quantized
    in 1x128 blocks, the input of the down projection."""
    return quant_act_1x128(round_bf16(swiglu_h_f64(aq, as_, bq, bs)), mode)


# The same fused gate+up projection for the experts of a SwiGLU
# mixture-of-experts layer (the recipe's MoE models, page 1, "Leistungsgewinne
# in der Praxis" and "Warum dies fuer die KI-Oekonomie wichtig ist"): routed
# row r of group g goes through expert g's fused gate+up weight, then the
# SwiGLU and row quantization above.  Reading: the grouping is that of the
# grouped GEMM (rows [offsets[g], offsets[g+1]) to expert g), and routed rows
# may be gathered from the token matrix by index, an index outside the tokens
# standing for a zero row (zero codes, zero scale), as for the gathering
# grouped GEMM.
# ---------------------------------------------------------------------------

def _gather_rows(aq, as_, row_index):
    """(a_q, a_s) of the routed rows: token row row_index[r], or a zero row."""
    aq = np.asarray(aq, dtype=np.uint8)
    as_ = np.asarray(as_, dtype=np.float32)
    idx = np.asarray(row_index, dtype=np.int64)
    ok = (idx >= 0) & (idx < aq.shape[0])
    gq = np.zeros((idx.size, aq.shape[1]), dtype=np.uint8)
    gs = np.zeros((idx.size, as_.shape[1]), dtype=np.float32)
    gq[ok] = aq[idx[ok]]
    gs[ok] = as_[idx[ok]]
    return gq, gs


def _swiglu_quant_of_y(y, mode):
    """Fused gate|up GEMM output y [rows, 2F] (fp64, before its bf16 rounding)
    -> the row quantization of bf16(silu(bf16(g)) * bf16(u))."""
    yb = bf16_to_f64(round_bf16(y))
    g, u = swiglu_split(yb)
    return quant_act_1x128(round_bf16(g / (1.0 + np.exp(-g)) * u), mode)


def grouped_gemm_swiglu_quant(aq, as_, bq, bs, offsets, mode=MODE_AMAX, row_index=None):
    """(h_q uint8 [M_total, F], h_s f32 [M_total, F/128]).  bq [G, 2F, K],
    bs [G, 2F/128, K/128] (gate/up interleaved per expert as for
    gemm_swiglu_quant), offsets int32 [G+1] covering all M_total rows.
    row_index None: aq [M_total, K] are the routed rows; else aq [T, K] the
    tokens and routed row r is token row_index[r]."""
    if row_index is not None:
        aq, as_ = _gather_rows(aq, as_, row_index)
    return _swiglu_quant_of_y(grouped_gemm_f64(aq, as_, bq, bs, offsets), mode)


def grouped_gemm_swiglu_quant_rows(aq, as_, bq, bs, groups, rows, mode=MODE_AMAX):
    """The rows `rows` of grouped_gemm_swiglu_quant's output, row rows[i] of aq
    (already gathered, or the token row it reads) going through the expert
    groups[i]: (h_q uint8 [len(rows), F], h_s f32 [len(rows), F/128])."""
    rows = np.asarray(rows, dtype=np.int64)
    N = np.asarray(bq).shape[1]
    ms = np.repeat(rows, N)
    ns = np.tile(np.arange(N, dtype=np.int64), rows.size)
    grp = np.repeat(np.asarray(groups, dtype=np.int32), N)
    y = grouped_gemm_sampled_f64(aq, as_, bq, bs, grp, ms, ns).reshape(rows.size, N)
    return _swiglu_quant_of_y(y, mode)


# ---------------------------------------------------------------------------
# RMS normalization with the next layer's quantization fused: the third
# producer of FP8 activations in a Llama/Qwen3 block (its norms feed the QKV
# and gate+up projections; page 1, "Leistungsgewinne in der Praxis": the
# quantization kernels are overhead).  Reading: y = gamma * x / sqrt(mean(x^2)
# + eps) over each row of K values, computed exactly (fp64) from the bf16 x
# and gamma and the fp32 eps, rounded once to bf16, then quantized in 1x128
# blocks by the activation rule.
# ---------------------------------------------------------------------------

def rmsnorm_f64(x_bits, gamma_bits, eps):
    """y [M, K] in fp64 before its bf16 rounding; x_bits [M, K] and gamma_bits
    [K] are bf16 bit patterns, eps a float32 value."""
    x = bf16_to_f64(np.asarray(x_bits, dtype=np.uint16))
    g = bf16_to_f64(np.asarray(gamma_bits, dtype=np.uint16))
    if x.ndim != 2 or g.shape != (x.shape[1],):
        raise ValueError("x must be [M, K] and gamma [K]")
    ms = np.mean(x * x, axis=1, keepdims=True)
    e = float(np.float32(eps))
    return x / np.sqrt(ms + e) * g[None, :]


def rmsnorm_quant_1x128(x_bits, gamma_bits, eps, mode=MODE_AMAX):
    """(q uint8 [M, K], s f32 [M, K/128]): bf16(rmsnorm(x)) quantized in 1x128
    blocks, the input of the projection that follows the norm."""
    return quant_act_1x128(round_bf16(rmsnorm_f64(x_bits, gamma_bits, eps)), mode)


# ---------------------------------------------------------------------------
# MoE dispatch order (page "NVIDIA NeMo RL erreicht 48% Geschwindigkeits-
# steigerung ...", section "Leistungsgewinne in der Praxis": the recipe trains
# the Qwen3-30B mixture-of-experts model; section "Warum dies fuer die KI-
# Oekonomie wichtig ist": Moonlight 16B).  The grouped GEMM wants the routed
# rows grouped by expert.  The pages give no order inside a group; the reading
# taken here is the plainest one: rows sorted by expert, and within an expert
# in the order of the routing table read row by row (token t, slot j: entry
# t*k + j).  Shared experts (every token goes to each of them) follow as
# groups of all tokens in token order.  An expert id outside [0, E) places its
# entry in no group; such entries leave rows at the end, after the last group,
# with token -1.
# ---------------------------------------------------------------------------

def moe_permute(expert_ids, E, n_shared=0):
    """expert_ids int [T, k] -> (offsets int32 [E+n_shared+1], row_index int32
    [T*(k+n_shared)], entry_row int32 [T*k]).

    offsets[g] is the first row of group g (experts 0..E-1, then the shared
    groups); row_index[r] is the token of row r (-1 for the trailing rows of
    invalid entries); entry_row[t*k + j] is the row of entry (t, j), -1 for an
    invalid expert id.  The grouping is one stable sort of the entries by
    expert (a library sort, stable by position)."""
    ids = np.asarray(expert_ids).astype(np.int64)
    T, k = ids.shape
    flat = ids.reshape(-1)
    n = flat.size
    valid = (flat >= 0) & (flat < E)
    key = np.where(valid, flat, E)                   # invalid entries sort last
    order = np.argsort(key, kind="stable")           # entries by expert, stable by position
    counts = np.bincount(flat[valid], minlength=E)[:E]
    nv = int(counts.sum())
    G = E + n_shared
    offsets = np.zeros(G + 1, dtype=np.int64)
    offsets[1:E + 1] = np.cumsum(counts)
    for s in range(n_shared):
        offsets[E + 1 + s] = nv + (s + 1) * T
    rows = T * (k + n_shared)
    row_index = np.full(rows, -1, dtype=np.int64)
    row_index[:nv] = order[:nv] // k                 # the token of each routed entry
    for s in range(n_shared):
        row_index[nv + s * T: nv + (s + 1) * T] = np.arange(T)
    entry_row = np.full(n, -1, dtype=np.int64)
    entry_row[order[:nv]] = np.arange(nv)
    return offsets.astype(np.int32), row_index.astype(np.int32), entry_row.astype(np.int32)
