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
