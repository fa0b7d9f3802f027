"""Helpers shared by the GPU parity tests (test code only)."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_bits


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def lib():
    """The HIP library's Python face; fails loudly if it cannot be loaded."""
    import blockwise_scaled_fp8_quant_amd as fp8q
    fp8q.abi_version()  # loads libfp8q.so or raises
    return fp8q


def say(*a):
    """Name the case before a GPU step (flushed, so a crash still shows it)."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def dev_bf16(bits):
    """uint16 numpy bits -> bf16 tensor on cuda:0."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to("cuda:0")


def host_u8(t):
    return t.detach().to("cpu").contiguous().view(torch.uint8).numpy()


def host_f32(t):
    return t.detach().to("cpu").contiguous().numpy()


def host_bf16_as_f64(t):
    return t.detach().to("cpu").float().numpy().astype(np.float64)


def assert_bytes_equal(got, want, what):
    got = np.asarray(got)
    want = np.asarray(want)
    assert got.shape == want.shape, (what, got.shape, want.shape)
    bad = np.flatnonzero(got.reshape(-1) != want.reshape(-1))
    if bad.size:
        i = bad[:8]
        raise AssertionError(f"{what}: {bad.size} of {got.size} differ; first idx {i.tolist()} "
                             f"got {got.reshape(-1)[i].tolist()} want {want.reshape(-1)[i].tolist()}")


def assert_scales_equal(got, want, what):
    got = np.asarray(got, dtype=np.float32)
    want = np.asarray(want, dtype=np.float32)
    assert_bytes_equal(got.view(np.uint32), want.view(np.uint32), what + " (scale bits)")


def gemm_tolerance_check(y_gpu, y_ref, what, elem_rel=8e-3, elem_rms=1e-3, frob=2e-3):
    """|dY| <= elem_rel*|Y_ref| + elem_rms*rms(Y_ref) element-wise and
    ||dY||_F / ||Y_ref||_F <= frob."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    d = np.abs(y_gpu - y_ref)
    rms = float(np.sqrt(np.mean(y_ref ** 2))) if y_ref.size else 0.0
    bound = elem_rel * np.abs(y_ref) + elem_rms * rms
    bad = np.flatnonzero(d.reshape(-1) > bound.reshape(-1))
    if bad.size:
        i = bad[:5]
        raise AssertionError(f"{what}: {bad.size} elements out of tolerance; e.g. idx {i.tolist()} "
                             f"gpu {y_gpu.reshape(-1)[i].tolist()} ref {y_ref.reshape(-1)[i].tolist()}")
    nref = float(np.linalg.norm(y_ref))
    if nref > 0:
        rel = float(np.linalg.norm(y_gpu - y_ref)) / nref
        assert rel <= frob, f"{what}: relative Frobenius error {rel:.3e} > {frob}"
        return rel
    return 0.0


def quantize_pair_oracle(x_bf16, w_bf16, mode=0):
    """Oracle quantization of host copies of x and w (bf16 tensors)."""
    xq, xs = oracle.quant_act_1x128(bf16_bits(x_bf16), mode)
    wq, ws = oracle.quant_weight_128x128(bf16_bits(w_bf16), mode)
    return xq, xs, wq, ws


def moe_layer_inputs(shape, layer, device="cuda"):
    """One expert layer of a synthetic MoE workload: (X bf16 [rows, K], W bf16
    [G, N, K], offsets int32 [G+1], row_index int32 [rows]).  The rows are in
    the oracle's dispatch order (sorted by expert, stable by table position,
    shared experts last); the gate+up input row r is the hidden state of token
    row_index[r], the down input an independent matrix."""
    import synth
    ids = synth.moe_routing(shape)
    off, rows, _ = oracle.moe_permute(ids, shape.routed_experts, shape.shared_experts)
    w = synth.moe_weights(shape, layer, device)
    if layer == "gate_up":
        xt = synth.moe_token_matrix(shape, device)
        x = xt[torch.from_numpy(rows.astype(np.int64)).to(xt.device)].contiguous()
    else:
        x = synth.moe_down_input(shape, device)
    return x, w, off, rows


def moe_rows(off, seed, per_group=2):
    """Whole rows to check in every non-empty group: its first and last row and
    `per_group` random ones (group of each row returned alongside)."""
    rng = np.random.default_rng(seed)
    ms, gs = [], []
    for g in range(len(off) - 1):
        r0, r1 = int(off[g]), int(off[g + 1])
        if r1 > r0:
            pick = np.unique(np.concatenate([[r0, r1 - 1], rng.integers(r0, r1, per_group)]))
            ms.append(pick)
            gs.append(np.full(pick.size, g))
    return np.concatenate(ms), np.concatenate(gs)


def moe_whole_rows_check(y_rows, aq_rows, as_rows, bq, bs, gs, what):
    """GEMM tolerance on whole output rows of a grouped GEMM: y_rows [R, N]
    (f64) against the oracle for the operand rows aq_rows/as_rows of groups gs,
    rms taken over those rows."""
    R, N = y_rows.shape
    ms = np.repeat(np.arange(R), N)
    ns = np.tile(np.arange(N), R)
    ref = oracle.grouped_gemm_sampled_f64(aq_rows, as_rows, bq, bs, np.repeat(gs, N), ms, ns)
    return gemm_tolerance_check(y_rows.reshape(-1), ref, what)
