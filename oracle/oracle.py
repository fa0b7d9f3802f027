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
