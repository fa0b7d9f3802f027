"""GPU parity of the batched weight recalibration (fp8_quant_weight_128x128_batched).

Every matrix of a batch must get exactly the bytes and scales that the oracle's
128x128 quantizer gives it (page "NVIDIA NeMo RL erreicht 48%
Geschwindigkeitssteigerung ...", sections "Der technische Durchbruch" and
"Leistungsgewinne in der Praxis"), and exactly what the single-matrix entry
point writes; tiles of inconsistent jobs are skipped without touching memory.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from tests._gpu import (assert_bytes_equal, assert_scales_equal, dev_bf16, host_f32, host_u8,
                        lib, require_gpu, say)

pytestmark = pytest.mark.gpu
MODES = (0, 1)

# shapes of different tile counts, so that tiles of neighbouring jobs interleave
# in the flat tile sequence at every offset
SHAPES = [(128, 128), (256, 640), (384, 128), (128, 1024), (640, 384), (128, 256)]


def _special_matrix():
    """A 256x384 weight whose tiles are: all zero, bf16 subnormals, one huge
    value among tiny ones, exact E4M3 values x 2^-20 (round trip), negative
    zeros, and ordinary N(0, 0.02)."""
    w = synth.bf16_bits(synth.normal_bf16((256, 384), 0.02, synth.seed_of(21, 0, 1)))
    w[0:128, 0:128] = 0
    rng = np.random.default_rng(5)
    w[0:128, 128:256] = rng.integers(1, 0x80, size=(128, 128), dtype=np.uint16) | \
        (rng.integers(0, 2, size=(128, 128), dtype=np.uint16) << 15)
    w[0:128, 256:384] = 0x0001
    w[5, 300] = 0x7F7F  # largest finite bf16
    codes = np.arange(128 * 128, dtype=np.int64) % 254
    codes = np.where(codes >= 0x7F, codes + 1, codes).astype(np.uint8)  # skip NaN encodings
    vals = oracle.e4m3_decode_table()[codes].reshape(128, 128) * 2.0 ** -20
    vals[0, 0] = 448.0 * 2.0 ** -20
    w[128:256, 0:128] = synth.bf16_bits(torch.from_numpy(vals.astype(np.float32)).to(torch.bfloat16))
    w[128:256, 128:256] = 0x8000
    return w


def _batch_inputs(seed):
    mats = [synth.bf16_bits(synth.normal_bf16(s, 0.02, synth.seed_of(21, seed, i))) for i, s in enumerate(SHAPES)]
    mats.insert(2, _special_matrix())
    return mats


@pytest.mark.parametrize("mode", MODES)
def test_batch_matches_oracle(mode):
    require_gpu()
    fp8q = lib()
    mats = _batch_inputs(1)
    say("quant_weight_batched", [m.shape for m in mats], "mode", mode)
    batch = fp8q.WeightBatch([dev_bf16(m) for m in mats])
    outs = fp8q.fp8_quant_weight_128x128_batched(batch, mode)
    torch.cuda.synchronize()
    for i, (m, (q, s)) in enumerate(zip(mats, outs)):
        oq, os_ = oracle.quant_weight_128x128(m, mode)
        assert_scales_equal(host_f32(s), os_, f"job {i} {m.shape} scales")
        assert_bytes_equal(host_u8(q), oq, f"job {i} {m.shape} bytes")


@pytest.mark.parametrize("mode", MODES)
def test_batch_equals_single_matrix_calls_full_size(mode):
    """One layer of the 32-layer Llama-3.1-8B shape (QKV, O, gate+up, down) at
    full size: the batched launch writes the same bits as four single calls."""
    require_gpu()
    fp8q = lib()
    ws = [synth.llama_weight(31, kind, device="cuda") for kind in range(4)]
    say("quant_weight_batched llama layer 31", [tuple(w.shape) for w in ws], "mode", mode)
    batch = fp8q.WeightBatch(ws)
    outs = fp8q.fp8_quant_weight_128x128_batched(batch, mode)
    for w, (q, s) in zip(ws, outs):
        q1, s1 = fp8q.fp8_quant_weight_128x128(w, mode)
        torch.cuda.synchronize()
        assert torch.equal(q.view(torch.uint8), q1.view(torch.uint8))
        assert torch.equal(s.view(torch.int32), s1.view(torch.int32))


def test_repeated_passes_and_guards():
    """Two passes (amax, then pow2) over one batch each leave exactly their own
    result; bytes past each output stay untouched."""
    require_gpu()
    fp8q = lib()
    mats = _batch_inputs(2)
    outs, guards = [], []
    for m in mats:
        N, K = m.shape
        qb = torch.full((N * K + 2048,), 0xA5, dtype=torch.uint8, device="cuda")
        sb = torch.full((N * K // 16384 + 256,), -7.0, dtype=torch.float32, device="cuda")
        outs.append((qb[: N * K].view(N, K), sb[: N * K // 16384].view(N // 128, K // 128)))
        guards.append((qb, sb, N * K, N * K // 16384))
    batch = fp8q.WeightBatch([dev_bf16(m) for m in mats], outs)
    for mode in (0, 1):
        say("quant_weight_batched repeated pass, mode", mode)
        fp8q.fp8_quant_weight_128x128_batched(batch, mode)
        torch.cuda.synchronize()
        for i, (m, (q, s)) in enumerate(zip(mats, outs)):
            oq, os_ = oracle.quant_weight_128x128(m, mode)
            assert_scales_equal(host_f32(s), os_, f"pass {mode} job {i} scales")
            assert_bytes_equal(host_u8(q), oq, f"pass {mode} job {i} bytes")
    for qb, sb, nq, ns in guards:
        assert torch.all(qb[nq:] == 0xA5) and torch.all(sb[ns:] == -7.0)


def _fresh(mats):
    return [(torch.full(tuple(m.shape), 0x5A, dtype=torch.uint8, device="cuda"),
             torch.full((m.shape[0] // 128, m.shape[1] // 128), -3.0, dtype=torch.float32, device="cuda"))
            for m in mats]


def _exact(m, out, what):
    oq, os_ = oracle.quant_weight_128x128(m, 0)
    assert_bytes_equal(host_u8(out[0]), oq, what + " bytes")
    assert_scales_equal(host_f32(out[1]), os_, what + " scales")


def _untouched(out):
    return bool(torch.all(out[0] == 0x5A)) and bool(torch.all(out[1] == -3.0))


def test_inconsistent_jobs_are_skipped():
    """Tiles in a gap left by tile_begin values past the running sum, and every
    tile of a job whose shape is not a multiple of 128, are skipped: those
    outputs keep their contents and the consistent jobs are still exact."""
    require_gpu()
    fp8q = lib()
    mats = [synth.bf16_bits(synth.normal_bf16(s, 0.02, synth.seed_of(21, 3, i)))
            for i, s in enumerate([(256, 256), (128, 384), (256, 128)])]
    ws = [dev_bf16(m) for m in mats]

    # jobs 1 and 2 start 5 tiles late: tiles 4..8 fall past job 0's 4 tiles
    outs = _fresh(mats)
    batch = fp8q.WeightBatch(ws, outs)
    jobs = batch.jobs.cpu()
    jobs[1:, 5] += 5
    batch.jobs, batch.total_tiles = jobs.to("cuda"), batch.total_tiles + 5
    say("quant_weight_batched tile gap")
    fp8q.fp8_quant_weight_128x128_batched(batch, 0)
    torch.cuda.synchronize()
    for i in range(3):
        _exact(mats[i], outs[i], f"gap: job {i}")

    # job 1 claims N = 100: all its tiles are skipped
    outs = _fresh(mats)
    batch = fp8q.WeightBatch(ws, outs)
    jobs = batch.jobs.cpu()
    jobs[1, 3] = 100
    batch.jobs = jobs.to("cuda")
    say("quant_weight_batched bad shape")
    fp8q.fp8_quant_weight_128x128_batched(batch, 0)
    torch.cuda.synchronize()
    _exact(mats[0], outs[0], "bad shape: job 0")
    assert _untouched(outs[1])
    _exact(mats[2], outs[2], "bad shape: job 2")


def test_host_job_table_is_rejected():
    """A job table in host memory is refused on the host (FP8Q_EINVAL), before
    any launch: the kernel would have to read it from the device."""
    require_gpu()
    fp8q = lib()
    from blockwise_scaled_fp8_quant_amd import _lib
    import ctypes
    w = dev_bf16(synth.bf16_bits(synth.normal_bf16((128, 128), 0.02, synth.seed_of(21, 4, 0))))
    batch = fp8q.WeightBatch([w])
    host_table = batch.jobs.cpu()
    st = _lib.load().fp8_quant_weight_128x128_batched(ctypes.c_void_p(int(host_table.data_ptr())), 1, 1, 0, None)
    assert st == 1 and "device memory" in _lib.load().fp8q_last_error().decode()
    # the library still works afterwards (no error left behind)
    outs = fp8q.fp8_quant_weight_128x128_batched(batch, 0)
    torch.cuda.synchronize()
    oq, os_ = oracle.quant_weight_128x128(synth.bf16_bits(w.cpu()), 0)
    assert_bytes_equal(host_u8(outs[0][0]), oq, "after a rejected call")
