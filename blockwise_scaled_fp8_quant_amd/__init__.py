"""Blockwise-scaled FP8 linear layer for AMD MI355X (gfx950).

Python face of the C ABI in include/fp8q.h.  These functions only check and
marshal arguments (torch tensors in device memory, the current HIP stream);
every step of the computation runs in the library's HIP kernels.  PyTorch is
used for device memory and streams only.

The layer is the one of the end-to-end FP8 RL recipe (page "NVIDIA NeMo RL
erreicht 48% Geschwindigkeitssteigerung mit End-to-End FP8-Praezisionstraining",
section "Der technische Durchbruch"): E4M3 codes, one fp32 scale per 1x128
activation block and per 128x128 weight block, and a block-scaled GEMM with
fp32 accumulation and bf16 output; weights are requantized after every policy
update (section "Leistungsgewinne in der Praxis"), optionally with
power-of-two scales (section "Warum dies fuer die KI-Oekonomie wichtig ist").
"""
import ctypes

import torch

from . import _lib

SCALE_AMAX = 0
SCALE_POW2 = 1
_MODES = {"amax": SCALE_AMAX, "pow2": SCALE_POW2, SCALE_AMAX: SCALE_AMAX, SCALE_POW2: SCALE_POW2}

__all__ = ["SCALE_AMAX", "SCALE_POW2", "fp8_quant_act_1x128", "fp8_rmsnorm_quant_1x128",
           "fp8_quant_weight_128x128", "WeightBatch", "fp8_quant_weight_128x128_batched",
           "fp8_blockscaled_gemm", "fp8_grouped_gemm", "fp8_blockscaled_gemm_pow2",
           "fp8_grouped_gemm_pow2", "fp8_blockscaled_gemm_quant", "fp8_blockscaled_gemm_swiglu_quant",
           "fp8_grouped_gemm_gather", "fp8_grouped_gemm_swiglu_quant",
           "fp8_quant_act_dual", "fp8_quant_weight_128x128_dual", "fp8_blockscaled_gemm_wgrad",
           "fp8_blockscaled_gemm_wgrad_pow2",
           "fp8_kv_cache_append", "fp8_attention_decode", "fp8_attention_decode_workspace_size",
           "abi_version", "library_path"]


def library_path():
    return _lib.LIB_PATH


def abi_version():
    return _lib.load().fp8q_abi_version()


def _mode(mode):
    try:
        return _MODES[mode]
    except KeyError:
        raise ValueError(f"unknown scale mode {mode!r} (use 'amax' or 'pow2')") from None


def _stream(t):
    return ctypes.c_void_p(int(torch.cuda.current_stream(t.device).cuda_stream))


def _dev(t, name, dtype, ndim):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be in device memory (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return ctypes.c_void_p(int(t.data_ptr()))


def _as_bytes(t, name, ndim):
    if isinstance(t, torch.Tensor) and t.dtype == torch.float8_e4m3fn:
        t = t.view(torch.uint8)
    return t, _dev(t, name, torch.uint8, ndim)


def fp8_quant_act_1x128(x, mode="amax", out=None):
    """x: bf16 [M, K] (K % 128 == 0) -> (q uint8 [M, K] E4M3 codes, s fp32 [M, K/128])."""
    px = _dev(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if out is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        s = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    else:
        q, s = out
    _, pq = _as_bytes(q, "q", 2)
    ps = _dev(s, "scales", torch.float32, 2)
    if tuple(q.shape) != (M, K) or tuple(s.shape) != (M, K // 128):
        raise ValueError("output shapes do not match x")
    _lib.check("fp8_quant_act_1x128",
               _lib.load().fp8_quant_act_1x128(px, M, K, pq, ps, _mode(mode), _stream(x)))
    return q, s


def fp8_rmsnorm_quant_1x128(x, gamma, eps=1e-5, mode="amax", out=None):
    """RMS normalization fused with the 1x128 quantization of its output:
    x bf16 [M, K], gamma bf16 [K] (K % 128 == 0, K <= 8192) ->
    (q uint8 [M, K], s fp32 [M, K/128]) of bf16(x / sqrt(mean(x^2) + eps) * gamma)."""
    px = _dev(x, "x", torch.bfloat16, 2)
    pg = _dev(gamma, "gamma", torch.bfloat16, 1)
    M, K = x.shape
    if tuple(gamma.shape) != (K,):
        raise ValueError("gamma must have K elements")
    if out is None:
        q = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        s = torch.empty((M, K // 128), dtype=torch.float32, device=x.device)
    else:
        q, s = out
    _, pq = _as_bytes(q, "q", 2)
    ps = _dev(s, "scales", torch.float32, 2)
    if tuple(q.shape) != (M, K) or tuple(s.shape) != (M, K // 128):
        raise ValueError("output shapes do not match x")
    _lib.check("fp8_rmsnorm_quant_1x128",
               _lib.load().fp8_rmsnorm_quant_1x128(px, pg, M, K, float(eps), pq, ps, _mode(mode), _stream(x)))
    return q, s


def fp8_quant_weight_128x128(w, mode="amax", out=None):
    """w: bf16 [N, K] (N, K % 128 == 0) -> (q uint8 [N, K], s fp32 [N/128, K/128])."""
    pw = _dev(w, "w", torch.bfloat16, 2)
    N, K = w.shape
    if out is None:
        q = torch.empty((N, K), dtype=torch.uint8, device=w.device)
        s = torch.empty((N // 128, K // 128), dtype=torch.float32, device=w.device)
    else:
        q, s = out
    _, pq = _as_bytes(q, "q", 2)
    ps = _dev(s, "scales", torch.float32, 2)
    if tuple(q.shape) != (N, K) or tuple(s.shape) != (N // 128, K // 128):
        raise ValueError("output shapes do not match w")
    _lib.check("fp8_quant_weight_128x128",
               _lib.load().fp8_quant_weight_128x128(pw, N, K, pq, ps, _mode(mode), _stream(w)))
    return q, s


class WeightBatch:
    """A fixed set of weight matrices that are requantized together, e.g. every
    linear weight of a model after each policy update.

    weights: bf16 [N_i, K_i] tensors on one device (N_i, K_i % 128 == 0).
    outs:    optional (q uint8 [N_i, K_i], s fp32 [N_i/128, K_i/128]) per weight.
    The job table of the C ABI (fp8q_weight_job: w, q, scales, N, K,
    tile_begin; 48 bytes each) is built once, here, in device memory; the
    tensors stay referenced so that the addresses in it remain valid.
    """

    def __init__(self, weights, outs=None):
        weights = list(weights)
        if not weights:
            raise ValueError("WeightBatch needs at least one weight")
        device = weights[0].device
        if outs is None:
            outs = [(torch.empty(tuple(w.shape), dtype=torch.uint8, device=device),
                     torch.empty((w.shape[0] // 128, w.shape[1] // 128), dtype=torch.float32, device=device))
                    for w in weights]
        outs = list(outs)
        if len(outs) != len(weights):
            raise ValueError("one (q, s) pair per weight")
        rows, tiles = [], 0
        for i, (w, (q, s)) in enumerate(zip(weights, outs)):
            pw = _dev(w, f"weights[{i}]", torch.bfloat16, 2)
            _, pq = _as_bytes(q, f"q[{i}]", 2)
            ps = _dev(s, f"scales[{i}]", torch.float32, 2)
            if w.device != device or q.device != device or s.device != device:
                raise ValueError("all tensors of a WeightBatch must be on one device")
            N, K = w.shape
            if N % 128 or K % 128 or K == 0:
                raise ValueError(f"weights[{i}]: N and K must be multiples of 128 and K > 0 (got {N}x{K})")
            if tuple(q.shape) != (N, K) or tuple(s.shape) != (N // 128, K // 128):
                raise ValueError(f"outs[{i}]: shapes do not match weights[{i}]")
            rows.append([pw.value, pq.value, ps.value, N, K, tiles])
            tiles += (N // 128) * (K // 128)
        self.weights, self.outs = weights, outs
        self.total_tiles = tiles
        self.jobs = torch.tensor(rows, dtype=torch.int64).to(device)
        torch.cuda.synchronize(device)

    def __len__(self):
        return len(self.weights)


def fp8_quant_weight_128x128_batched(batch, mode="amax"):
    """Quantize every weight of a WeightBatch in one launch, each exactly as
    fp8_quant_weight_128x128 would; returns the batch's list of (q, s)."""
    if not isinstance(batch, WeightBatch):
        raise TypeError("batch must be a WeightBatch")
    _lib.check("fp8_quant_weight_128x128_batched",
               _lib.load().fp8_quant_weight_128x128_batched(
                   ctypes.c_void_p(int(batch.jobs.data_ptr())), len(batch), batch.total_tiles, _mode(mode),
                   _stream(batch.jobs)))
    return batch.outs


def _gemm(fn, a_q, a_s, b_q, b_s, out):
    a_q, pa = _as_bytes(a_q, "a_q", 2)
    b_q, pb = _as_bytes(b_q, "b_q", 2)
    pas = _dev(a_s, "a_s", torch.float32, 2)
    pbs = _dev(b_s, "b_s", torch.float32, 2)
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K or tuple(a_s.shape) != (M, K // 128) or tuple(b_s.shape) != (N // 128, K // 128):
        raise ValueError("operand shapes do not match")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device) if out is None else out
    py = _dev(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("output shape does not match")
    _lib.check(fn, getattr(_lib.load(), fn)(pa, pas, pb, pbs, py, M, N, K, _stream(a_q)))
    return y


def fp8_blockscaled_gemm(a_q, a_s, b_q, b_s, out=None):
    """Y[M, N] bf16 = dequant(a_q, a_s) @ dequant(b_q, b_s)^T (fp32 accumulation)."""
    return _gemm("fp8_blockscaled_gemm", a_q, a_s, b_q, b_s, out)


def fp8_blockscaled_gemm_pow2(a_q, a_s, b_q, b_s, out=None):
    """As fp8_blockscaled_gemm, for scales that are all powers of two (the
    matrix cores apply them); an output that depends on any other scale is NaN."""
    return _gemm("fp8_blockscaled_gemm_pow2", a_q, a_s, b_q, b_s, out)


def fp8_blockscaled_gemm_quant(a_q, a_s, b_q, b_s, mode="amax", out=None):
    """The GEMM with its output quantized for the next FP8 layer:
    (y_q uint8 [M, N] E4M3 codes, y_s fp32 [M, N/128]), equal to
    fp8_quant_act_1x128(fp8_blockscaled_gemm(...), mode)."""
    a_q, pa = _as_bytes(a_q, "a_q", 2)
    b_q, pb = _as_bytes(b_q, "b_q", 2)
    pas = _dev(a_s, "a_s", torch.float32, 2)
    pbs = _dev(b_s, "b_s", torch.float32, 2)
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K or tuple(a_s.shape) != (M, K // 128) or tuple(b_s.shape) != (N // 128, K // 128):
        raise ValueError("operand shapes do not match")
    if out is None:
        yq = torch.empty((M, N), dtype=torch.uint8, device=a_q.device)
        ys = torch.empty((M, N // 128), dtype=torch.float32, device=a_q.device)
    else:
        yq, ys = out
    yq, pyq = _as_bytes(yq, "y_q", 2)
    pys = _dev(ys, "y_s", torch.float32, 2)
    if tuple(yq.shape) != (M, N) or tuple(ys.shape) != (M, N // 128):
        raise ValueError("output shapes do not match")
    _lib.check("fp8_blockscaled_gemm_quant",
               _lib.load().fp8_blockscaled_gemm_quant(pa, pas, pb, pbs, pyq, pys, M, N, K, _mode(mode),
                                                      _stream(a_q)))
    return yq, ys


def fp8_blockscaled_gemm_swiglu_quant(a_q, a_s, b_q, b_s, mode="amax", out=None):
    """Fused gate+up projection of a SwiGLU MLP with its activation quantized:
    b_q [2F, K] holds gate and up rows in alternating 128-row blocks; returns
    (h_q uint8 [M, F], h_s fp32 [M, F/128]), the 1x128 quantization of the
    bf16 h = silu(gate) * up."""
    a_q, pa = _as_bytes(a_q, "a_q", 2)
    b_q, pb = _as_bytes(b_q, "b_q", 2)
    pas = _dev(a_s, "a_s", torch.float32, 2)
    pbs = _dev(b_s, "b_s", torch.float32, 2)
    M, K = a_q.shape
    N = b_q.shape[0]
    if N % 256 != 0:
        raise ValueError("b_q must have 2F rows, F a multiple of 128")
    F = N // 2
    if b_q.shape[1] != K or tuple(a_s.shape) != (M, K // 128) or tuple(b_s.shape) != (N // 128, K // 128):
        raise ValueError("operand shapes do not match")
    if out is None:
        hq = torch.empty((M, F), dtype=torch.uint8, device=a_q.device)
        hs = torch.empty((M, F // 128), dtype=torch.float32, device=a_q.device)
    else:
        hq, hs = out
    hq, phq = _as_bytes(hq, "h_q", 2)
    phs = _dev(hs, "h_s", torch.float32, 2)
    if tuple(hq.shape) != (M, F) or tuple(hs.shape) != (M, F // 128):
        raise ValueError("output shapes do not match")
    _lib.check("fp8_blockscaled_gemm_swiglu_quant",
               _lib.load().fp8_blockscaled_gemm_swiglu_quant(pa, pas, pb, pbs, phq, phs, M, F, K, _mode(mode),
                                                             _stream(a_q)))
    return hq, hs


def _grouped(fn, a_q, a_s, b_q, b_s, group_offsets, out):
    a_q, pa = _as_bytes(a_q, "a_q", 2)
    b_q, pb = _as_bytes(b_q, "b_q", 3)
    pas = _dev(a_s, "a_s", torch.float32, 2)
    pbs = _dev(b_s, "b_s", torch.float32, 3)
    poff = _dev(group_offsets, "group_offsets", torch.int32, 1)
    M, K = a_q.shape
    G, N, Kb = b_q.shape
    if Kb != K or tuple(a_s.shape) != (M, K // 128) or tuple(b_s.shape) != (G, N // 128, K // 128):
        raise ValueError("operand shapes do not match")
    if group_offsets.numel() != G + 1:
        raise ValueError("group_offsets must have G+1 entries")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device) if out is None else out
    py = _dev(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("output shape does not match")
    _lib.check(fn, getattr(_lib.load(), fn)(pa, pas, pb, pbs, poff, G, M, N, K, py, _stream(a_q)))
    return y


def fp8_grouped_gemm(a_q, a_s, b_q, b_s, group_offsets, out=None):
    """Grouped (mixture-of-experts) GEMM.

    a_q [M_total, K], a_s [M_total, K/128], b_q [G, N, K], b_s [G, N/128, K/128],
    group_offsets int32 [G+1] in device memory (rows of group g are
    [offsets[g], offsets[g+1])).  Returns Y bf16 [M_total, N].
    """
    return _grouped("fp8_grouped_gemm", a_q, a_s, b_q, b_s, group_offsets, out)


def fp8_grouped_gemm_pow2(a_q, a_s, b_q, b_s, group_offsets, out=None):
    """As fp8_grouped_gemm, for scales that are all powers of two."""
    return _grouped("fp8_grouped_gemm_pow2", a_q, a_s, b_q, b_s, group_offsets, out)


def fp8_grouped_gemm_gather(a_q, a_s, b_q, b_s, group_offsets, row_index, mode="amax", out=None):
    """Grouped GEMM over routed rows gathered from a quantized token matrix.

    a_q [T, K], a_s [T, K/128] (the tokens, quantized once before dispatch),
    b_q [G, N, K], b_s [G, N/128, K/128], group_offsets int32 [G+1] and
    row_index int32 [M_total] in device memory: routed row r reads token
    row_index[r] (rows with an index outside [0, T) come out as zeros).
    mode 'amax' for any scales, 'pow2' for power-of-two scales.
    Returns Y bf16 [M_total, N], equal to fp8_grouped_gemm on a_q[row_index].
    """
    a_q, pa = _as_bytes(a_q, "a_q", 2)
    b_q, pb = _as_bytes(b_q, "b_q", 3)
    pas = _dev(a_s, "a_s", torch.float32, 2)
    pbs = _dev(b_s, "b_s", torch.float32, 3)
    poff = _dev(group_offsets, "group_offsets", torch.int32, 1)
    pidx = _dev(row_index, "row_index", torch.int32, 1)
    T, K = a_q.shape
    G, N, Kb = b_q.shape
    M = row_index.numel()
    if Kb != K or tuple(a_s.shape) != (T, K // 128) or tuple(b_s.shape) != (G, N // 128, K // 128):
        raise ValueError("operand shapes do not match")
    if group_offsets.numel() != G + 1:
        raise ValueError("group_offsets must have G+1 entries")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device) if out is None else out
    py = _dev(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("output shape does not match")
    _lib.check("fp8_grouped_gemm_gather",
               _lib.load().fp8_grouped_gemm_gather(pa, pas, T, pb, pbs, poff, pidx, G, M, N, K, py,
                                                   _mode(mode), _stream(a_q)))
    return y


def fp8_grouped_gemm_swiglu_quant(a_q, a_s, b_q, b_s, group_offsets, row_index=None, mode="amax", out=None):
    """Experts' fused gate+up projection with SwiGLU and the down projection's
    quantization in the epilogue.

    b_q [G, 2F, K], b_s [G, 2F/128, K/128] (gate and up rows in alternating
    128-row blocks per expert), group_offsets int32 [G+1] in device memory.
    row_index None: a_q [M_total, K], a_s [M_total, K/128], routed row r is row
    r; else int32 [M_total] in device memory and a_q [T, K] the tokens, routed
    row r reading token row_index[r].  Returns (h_q uint8 [M_total, F],
    h_s fp32 [M_total, F/128]): per row, fp8_blockscaled_gemm_swiglu_quant
    with the row's expert weight.
    """
    a_q, pa = _as_bytes(a_q, "a_q", 2)
    b_q, pb = _as_bytes(b_q, "b_q", 3)
    pas = _dev(a_s, "a_s", torch.float32, 2)
    pbs = _dev(b_s, "b_s", torch.float32, 3)
    poff = _dev(group_offsets, "group_offsets", torch.int32, 1)
    T, K = a_q.shape
    G, N, Kb = b_q.shape
    if N % 256 != 0:
        raise ValueError("b_q must have 2F rows per expert, F a multiple of 128")
    F = N // 2
    if Kb != K or tuple(a_s.shape) != (T, K // 128) or tuple(b_s.shape) != (G, N // 128, K // 128):
        raise ValueError("operand shapes do not match")
    if group_offsets.numel() != G + 1:
        raise ValueError("group_offsets must have G+1 entries")
    if row_index is None:
        M, pidx = T, None
    else:
        pidx = _dev(row_index, "row_index", torch.int32, 1)
        M = row_index.numel()
    if out is None:
        hq = torch.empty((M, F), dtype=torch.uint8, device=a_q.device)
        hs = torch.empty((M, F // 128), dtype=torch.float32, device=a_q.device)
    else:
        hq, hs = out
    hq, phq = _as_bytes(hq, "h_q", 2)
    phs = _dev(hs, "h_s", torch.float32, 2)
    if tuple(hq.shape) != (M, F) or tuple(hs.shape) != (M, F // 128):
        raise ValueError("output shapes do not match")
    _lib.check("fp8_grouped_gemm_swiglu_quant",
               _lib.load().fp8_grouped_gemm_swiglu_quant(pa, pas, T, pb, pbs, poff, pidx, G, M, F, K, phq, phs,
                                                         _mode(mode), _stream(a_q)))
    return hq, hs


def _dual(fn, x, rows_mult, mode, rowwise, out):
    px = _dev(x, "x", torch.bfloat16, 2)
    M, K = x.shape
    if rows_mult and M % 128:
        raise ValueError("N must be a multiple of 128")
    Mp = (M + 127) // 128 * 128
    tile = fn == "fp8_quant_weight_128x128_dual"
    s_shape = (M // 128, K // 128) if tile else (M, K // 128)
    st_shape = (K // 128, Mp // 128) if tile else (K, Mp // 128)
    if out is None:
        dev = x.device
        q = torch.empty((M, K), dtype=torch.uint8, device=dev) if rowwise else None
        s = torch.empty(s_shape, dtype=torch.float32, device=dev) if rowwise else None
        qt = torch.empty((K, Mp), dtype=torch.uint8, device=dev)
        st = torch.empty(st_shape, dtype=torch.float32, device=dev)
    else:
        q, s, qt, st = out
    pq = ps = None
    if q is not None:
        q, pq = _as_bytes(q, "q", 2)
        ps = _dev(s, "scales", torch.float32, 2)
        if tuple(q.shape) != (M, K) or tuple(s.shape) != s_shape:
            raise ValueError("row-major output shapes do not match the input")
    qt, pqt = _as_bytes(qt, "q_t", 2)
    pst = _dev(st, "scales_t", torch.float32, 2)
    if tuple(qt.shape) != (K, Mp) or tuple(st.shape) != st_shape:
        raise ValueError("transposed output shapes do not match the input")
    _lib.check(fn, getattr(_lib.load(), fn)(px, M, K, pq, ps, pqt, pst, _mode(mode), _stream(x)))
    return q, s, qt, st


def fp8_quant_act_dual(x, mode="amax", rowwise=True, out=None):
    """x bf16 [M, K] -> (q [M, K], s [M, K/128], q_t [K, Mp], s_t [K, Mp/128]).

    q, s: the 1x128 row blocks (as fp8_quant_act_1x128; None with
    rowwise=False).  q_t, s_t: blocks of 128 rows x 1 column, transposed, for
    the weight-gradient GEMM; Mp = M rounded up to 128, padding codes 0.
    """
    return _dual("fp8_quant_act_dual", x, False, mode, rowwise, out)


def fp8_quant_weight_128x128_dual(w, mode="amax", rowwise=True, out=None):
    """w bf16 [N, K] -> (q [N, K], s [N/128, K/128], q_t [K, N], s_t [K/128, N/128]):
    the 128x128-tile quantization and its transpose (for the data gradient)."""
    return _dual("fp8_quant_weight_128x128_dual", w, True, mode, rowwise, out)


def fp8_blockscaled_gemm_wgrad_pow2(a_q, a_s, b_q, b_s, out=None):
    """As fp8_blockscaled_gemm_wgrad, for scales that are all powers of two
    (the matrix cores apply them); an output that depends on any other scale
    is NaN."""
    return fp8_blockscaled_gemm_wgrad(a_q, a_s, b_q, b_s, out, _fn="fp8_blockscaled_gemm_wgrad_pow2")


def fp8_blockscaled_gemm_wgrad(a_q, a_s, b_q, b_s, out=None, _fn="fp8_blockscaled_gemm_wgrad"):
    """Y [M, N] bf16 = dequant(a_q, a_s) @ dequant(b_q, b_s)^T with 1x128 scale
    blocks on both operands: a_s [M, K/128], b_s [N, K/128].  The weight
    gradient dW = dY^T X from the transposed outputs of fp8_quant_act_dual."""
    a_q, pa = _as_bytes(a_q, "a_q", 2)
    b_q, pb = _as_bytes(b_q, "b_q", 2)
    pas = _dev(a_s, "a_s", torch.float32, 2)
    pbs = _dev(b_s, "b_s", torch.float32, 2)
    M, K = a_q.shape
    N = b_q.shape[0]
    if b_q.shape[1] != K or tuple(a_s.shape) != (M, K // 128) or tuple(b_s.shape) != (N, K // 128):
        raise ValueError("operand shapes do not match")
    y = torch.empty((M, N), dtype=torch.bfloat16, device=a_q.device) if out is None else out
    py = _dev(y, "y", torch.bfloat16, 2)
    if tuple(y.shape) != (M, N):
        raise ValueError("output shape does not match")
    _lib.check(_fn, getattr(_lib.load(), _fn)(pa, pas, pb, pbs, py, M, N, K, _stream(a_q)))
    return y


def fp8_kv_cache_append(k_new, v_new, pos, cache, mode="amax"):
    """Quantize one new key and value row per sequence and head (bf16
    [B, Hkv, 128] each) into the FP8 cache at token positions pos (int32 [B],
    device).  cache = (k_q uint8 [B, Hkv, S, 128], k_s f32 [B, Hkv, S],
    v_q, v_s), updated in place."""
    kq, ks, vq, vs = cache
    pk = _dev(k_new, "k_new", torch.bfloat16, 3)
    pv = _dev(v_new, "v_new", torch.bfloat16, 3)
    ppos = _dev(pos, "pos", torch.int32, 1)
    kq, pkq = _as_bytes(kq, "k_cache", 4)
    vq, pvq = _as_bytes(vq, "v_cache", 4)
    pks = _dev(ks, "k_scale", torch.float32, 3)
    pvs = _dev(vs, "v_scale", torch.float32, 3)
    B, H, S, Dh = kq.shape
    if Dh != 128 or tuple(k_new.shape) != (B, H, 128) or tuple(v_new.shape) != (B, H, 128):
        raise ValueError("new rows must be [B, Hkv, 128] matching the cache")
    if tuple(vq.shape) != (B, H, S, 128) or tuple(ks.shape) != (B, H, S) or tuple(vs.shape) != (B, H, S):
        raise ValueError("cache shapes do not match")
    if pos.numel() != B:
        raise ValueError("pos must have B entries")
    _lib.check("fp8_kv_cache_append",
               _lib.load().fp8_kv_cache_append(pk, pv, ppos, pkq, pks, pvq, pvs, B, H, S, _mode(mode),
                                               _stream(k_new)))
    return cache


def fp8_kv_cache_append_tokens(k_new, v_new, start, cache, mode="amax"):
    """Quantize T new key and value rows per sequence and head (bf16
    [B, T, Hkv, 128] each, token-major) into the FP8 cache: token t of sequence
    b at position start[b] + t (start int32 [B], device).  cache as for
    fp8_kv_cache_append, updated in place."""
    kq, ks, vq, vs = cache
    pk = _dev(k_new, "k_new", torch.bfloat16, 4)
    pv = _dev(v_new, "v_new", torch.bfloat16, 4)
    pst = _dev(start, "start", torch.int32, 1)
    kq, pkq = _as_bytes(kq, "k_cache", 4)
    vq, pvq = _as_bytes(vq, "v_cache", 4)
    pks = _dev(ks, "k_scale", torch.float32, 3)
    pvs = _dev(vs, "v_scale", torch.float32, 3)
    B, H, S, Dh = kq.shape
    T = k_new.shape[1]
    if Dh != 128 or tuple(k_new.shape) != (B, T, H, 128) or tuple(v_new.shape) != (B, T, H, 128):
        raise ValueError("new rows must be [B, T, Hkv, 128] matching the cache")
    if tuple(vq.shape) != (B, H, S, 128) or tuple(ks.shape) != (B, H, S) or tuple(vs.shape) != (B, H, S):
        raise ValueError("cache shapes do not match")
    if start.numel() != B:
        raise ValueError("start must have B entries")
    _lib.check("fp8_kv_cache_append_tokens",
               _lib.load().fp8_kv_cache_append_tokens(pk, pv, pst, pkq, pks, pvq, pvs, B, T, H, S, _mode(mode),
                                                      _stream(k_new)))
    return cache


def fp8_attention_prefill(q_q, q_s, cache, start, out=None):
    """Causal attention of T query tokens per sequence over the FP8 cache:
    query t of sequence b at position start[b] + t sees cached tokens
    0 .. start[b] + t.  q_q uint8 [B, T, Hq, 128] and q_s f32 [B, T, Hq] (query
    rows in 1x128 blocks), cache as for fp8_kv_cache_append, start int32 [B]
    (device).  Returns bf16 [B, T, Hq, 128]."""
    kq, ks, vq, vs = cache
    q_q, pq = _as_bytes(q_q, "q_q", 4)
    pqs = _dev(q_s, "q_s", torch.float32, 3)
    kq, pkq = _as_bytes(kq, "k_cache", 4)
    vq, pvq = _as_bytes(vq, "v_cache", 4)
    pks = _dev(ks, "k_scale", torch.float32, 3)
    pvs = _dev(vs, "v_scale", torch.float32, 3)
    pst = _dev(start, "start", torch.int32, 1)
    B, T, Hq, Dh = q_q.shape
    Bk, Hkv, S, Dk = kq.shape
    if Dh != 128 or Dk != 128 or Bk != B or tuple(q_s.shape) != (B, T, Hq):
        raise ValueError("query and cache shapes do not match")
    if tuple(vq.shape) != (B, Hkv, S, 128) or tuple(ks.shape) != (B, Hkv, S) or tuple(vs.shape) != (B, Hkv, S):
        raise ValueError("cache shapes do not match")
    if start.numel() != B:
        raise ValueError("start must have B entries")
    y = torch.empty((B, T, Hq, 128), dtype=torch.bfloat16, device=q_q.device) if out is None else out
    py = _dev(y, "out", torch.bfloat16, 4)
    if tuple(y.shape) != (B, T, Hq, 128):
        raise ValueError("output shape does not match")
    _lib.check("fp8_attention_prefill",
               _lib.load().fp8_attention_prefill(pq, pqs, pkq, pks, pvq, pvs, pst, py, B, T, Hq, Hkv, S,
                                                 _stream(q_q)))
    return y


def fp8_attention_decode_workspace_size(B, Hq, Hkv, S):
    return _lib.load().fp8_attention_decode_workspace_size(B, Hq, Hkv, S)


def fp8_attention_decode(q_q, q_s, cache, seq_len, out=None, workspace="auto"):
    """Decode attention of one query token per sequence over the FP8 cache.
    q_q uint8 [B, Hq, 128] and q_s f32 [B, Hq] (the query rows in 1x128
    blocks), cache as for fp8_kv_cache_append, seq_len int32 [B] (device).
    workspace: a device tensor of at least fp8_attention_decode_workspace_size
    bytes, "auto" (allocated here), or None (no splitting of sequences).
    Returns bf16 [B, Hq, 128]."""
    kq, ks, vq, vs = cache
    q_q, pq = _as_bytes(q_q, "q_q", 3)
    pqs = _dev(q_s, "q_s", torch.float32, 2)
    kq, pkq = _as_bytes(kq, "k_cache", 4)
    vq, pvq = _as_bytes(vq, "v_cache", 4)
    pks = _dev(ks, "k_scale", torch.float32, 3)
    pvs = _dev(vs, "v_scale", torch.float32, 3)
    plen = _dev(seq_len, "seq_len", torch.int32, 1)
    B, Hq, Dh = q_q.shape
    Bk, Hkv, S, Dk = kq.shape
    if Dh != 128 or Dk != 128 or Bk != B or tuple(q_s.shape) != (B, Hq):
        raise ValueError("query and cache shapes do not match")
    if tuple(vq.shape) != (B, Hkv, S, 128) or tuple(ks.shape) != (B, Hkv, S) or tuple(vs.shape) != (B, Hkv, S):
        raise ValueError("cache shapes do not match")
    if seq_len.numel() != B:
        raise ValueError("seq_len must have B entries")
    y = torch.empty((B, Hq, 128), dtype=torch.bfloat16, device=q_q.device) if out is None else out
    py = _dev(y, "out", torch.bfloat16, 3)
    if tuple(y.shape) != (B, Hq, 128):
        raise ValueError("output shape does not match")
    need = fp8_attention_decode_workspace_size(B, Hq, Hkv, S)
    if isinstance(workspace, str) and workspace == "auto":
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=q_q.device) if need else None
    if workspace is None:
        pws, nws = None, 0
    else:
        if workspace.device.type != "cuda" or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous device tensor")
        pws, nws = ctypes.c_void_p(int(workspace.data_ptr())), workspace.numel() * workspace.element_size()
    _lib.check("fp8_attention_decode",
               _lib.load().fp8_attention_decode(pq, pqs, pkq, pks, pvq, pvs, plen, py, B, Hq, Hkv, S, pws, nws,
                                                _stream(q_q)))
    return y


def fp8_attention_decode_noalloc(q_q, q_s, cache, seq_len, out):
    """fp8_attention_decode without a workspace, for callers that cannot
    allocate: the library's static per-GPU scratch array takes the chunked
    path's partial results.  `out` (bf16 [B, Hq, 128], device) is required, so
    the call allocates nothing.  Calls that overlap on one GPU race."""
    kq, ks, vq, vs = cache
    q_q, pq = _as_bytes(q_q, "q_q", 3)
    pqs = _dev(q_s, "q_s", torch.float32, 2)
    kq, pkq = _as_bytes(kq, "k_cache", 4)
    vq, pvq = _as_bytes(vq, "v_cache", 4)
    pks = _dev(ks, "k_scale", torch.float32, 3)
    pvs = _dev(vs, "v_scale", torch.float32, 3)
    plen = _dev(seq_len, "seq_len", torch.int32, 1)
    B, Hq, Dh = q_q.shape
    Bk, Hkv, S, Dk = kq.shape
    if Dh != 128 or Dk != 128 or Bk != B or tuple(q_s.shape) != (B, Hq):
        raise ValueError("query and cache shapes do not match")
    if tuple(vq.shape) != (B, Hkv, S, 128) or tuple(ks.shape) != (B, Hkv, S) or tuple(vs.shape) != (B, Hkv, S):
        raise ValueError("cache shapes do not match")
    if seq_len.numel() != B:
        raise ValueError("seq_len must have B entries")
    py = _dev(out, "out", torch.bfloat16, 3)
    if tuple(out.shape) != (B, Hq, 128):
        raise ValueError("output shape does not match")
    _lib.check("fp8_attention_decode_noalloc",
               _lib.load().fp8_attention_decode_noalloc(pq, pqs, pkq, pks, pvq, pvs, plen, py, B, Hq, Hkv, S,
                                                        _stream(q_q)))
    return out


def fp8_moe_permute_workspace_size(T, k, E):
    return _lib.load().fp8_moe_permute_workspace_size(T, k, E)


def fp8_moe_permute(expert_ids, E, n_shared=0, out=None, workspace=None):
    """Routing table int32 [T, k] (device) -> (group_offsets int32 [E+n_shared+1],
    row_index int32 [T*(k+n_shared)], entry_row int32 [T*k]): rows sorted by
    expert, stable in table order, shared experts last -- the offsets and
    row map of fp8_grouped_gemm / fp8_grouped_gemm_gather.  out: optional
    (offsets, row_index, entry_row) tensors (entry_row may be None);
    workspace: optional device tensor of fp8_moe_permute_workspace_size
    bytes (allocated here if None)."""
    ids = _dev(expert_ids, "expert_ids", torch.int32, 2)
    T, k = expert_ids.shape
    dev = expert_ids.device
    rows = T * (k + n_shared)
    if out is None:
        off = torch.empty(E + n_shared + 1, dtype=torch.int32, device=dev)
        row_index = torch.empty(rows, dtype=torch.int32, device=dev)
        entry_row = torch.empty(T * k, dtype=torch.int32, device=dev)
    else:
        off, row_index, entry_row = out
    poff = _dev(off, "group_offsets", torch.int32, 1)
    prow = _dev(row_index, "row_index", torch.int32, 1)
    pent = None if entry_row is None else _dev(entry_row, "entry_row", torch.int32, 1)
    if off.numel() != E + n_shared + 1 or row_index.numel() != rows or (
            entry_row is not None and entry_row.numel() != T * k):
        raise ValueError("output sizes do not match the routing table")
    need = fp8_moe_permute_workspace_size(T, k, E)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=dev)
    if workspace.device.type != "cuda" or not workspace.is_contiguous():
        raise ValueError("workspace must be a contiguous device tensor")
    pws = ctypes.c_void_p(int(workspace.data_ptr()))
    nws = workspace.numel() * workspace.element_size()
    _lib.check("fp8_moe_permute", _lib.load().fp8_moe_permute(ids, T, k, E, n_shared, poff, prow, pent, pws, nws,
                                                              _stream(expert_ids)))
    return off, row_index, entry_row


def fp8_blockscaled_gemm_tile_plan(M, N, swiglu=False):
    """(R, P): the tiles of token rows [0, R) and 256-row weight panels [0, P)
    of a dense M x N GEMM run as 256-token tiles, all others as 128-token tiles
    (swiglu: for fp8_blockscaled_gemm_swiglu_quant, else for the other dense
    GEMMs)."""
    rows = ctypes.c_int64(0)
    n1 = _lib.load().fp8_blockscaled_gemm_tile_plan(M, N, 1 if swiglu else 0, ctypes.byref(rows))
    if n1 < 0:
        raise ValueError("invalid GEMM size")
    return rows.value, n1
