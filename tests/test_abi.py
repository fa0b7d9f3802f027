"""The C ABI library loads, exports every entry point that include/fp8q.h
declares, and rejects bad arguments on the host before touching any device
(these calls never reach a kernel, so they run without a GPU)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8q.h")


@pytest.fixture(scope="module")
def lib():
    from blockwise_scaled_fp8_quant_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from blockwise_scaled_fp8_quant_amd import build
        build.build()
    return _lib.load()


def _declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fp8\w*)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = _declared_functions()
    for n in ("fp8_quant_act_1x128", "fp8_rmsnorm_quant_1x128", "fp8_quant_weight_128x128",
              "fp8_quant_weight_128x128_batched", "fp8_blockscaled_gemm",
              "fp8_grouped_gemm", "fp8_blockscaled_gemm_pow2", "fp8_grouped_gemm_pow2",
              "fp8_blockscaled_gemm_quant", "fp8_blockscaled_gemm_swiglu_quant", "fp8_grouped_gemm_gather",
              "fp8_grouped_gemm_swiglu_quant", "fp8_quant_act_dual", "fp8_quant_weight_128x128_dual", "fp8_blockscaled_gemm_wgrad", "fp8_blockscaled_gemm_wgrad_pow2",
              "fp8_kv_cache_append", "fp8_kv_cache_append_tokens", "fp8_attention_prefill",
              "fp8_moe_permute", "fp8_blockscaled_gemm_tile_plan",
              "fp8_attention_decode", "fp8_attention_decode_workspace_size", "fp8q_status_string", "fp8q_last_error", "fp8q_abi_version"):
        assert n in names


def test_every_declared_symbol_is_exported(lib):
    for n in _declared_functions():
        assert hasattr(lib, n), n


def test_version_and_status_strings(lib):
    assert lib.fp8q_abi_version() == 1
    for st in range(6):
        assert lib.fp8q_status_string(st)
    assert lib.fp8q_status_string(99) == b"unknown status"


P = ctypes.c_void_p
GOOD = P(0x10000)      # a 16-byte-aligned address that is never dereferenced
ODD = P(0x10008)


def _err(lib):
    return lib.fp8q_last_error().decode()


@pytest.mark.parametrize("fn", ["fp8_quant_act_1x128", "fp8_quant_weight_128x128"])
def test_quantizer_argument_errors(lib, fn):
    f = getattr(lib, fn)
    assert f(GOOD, 128, 100, GOOD, GOOD, 0, None) == 2          # K % 128
    assert f(GOOD, 128, 0, GOOD, GOOD, 0, None) == 2            # K == 0
    assert f(GOOD, -1, 128, GOOD, GOOD, 0, None) == 1           # negative size
    assert f(GOOD, 128, 128, GOOD, GOOD, 7, None) == 1          # unknown mode
    assert "mode" in _err(lib)
    assert f(None, 128, 128, GOOD, GOOD, 0, None) == 1          # null pointer
    assert f(GOOD, 128, 128, None, GOOD, 1, None) == 1
    assert f(ODD, 128, 128, GOOD, GOOD, 0, None) == 3           # misaligned
    assert f(GOOD, 0, 128, None, None, 0, None) == 0            # empty: no-op
    if fn == "fp8_quant_weight_128x128":
        assert f(GOOD, 100, 128, GOOD, GOOD, 0, None) == 2      # N % 128


def test_batched_weight_quant_argument_errors(lib):
    f = lib.fp8_quant_weight_128x128_batched
    assert f(GOOD, -1, 4, 0, None) == 1                # negative count
    assert f(GOOD, 2, -4, 0, None) == 1                # negative tile total
    assert f(GOOD, 2, 4, 5, None) == 1                 # unknown mode
    assert "mode" in _err(lib)
    assert f(GOOD, 2, 1 << 31, 0, None) == 2           # more tiles than one grid holds
    assert f(None, 2, 4, 0, None) == 1                 # null table
    assert f(P(0x10004), 2, 4, 1, None) == 3           # table not 8-byte aligned
    assert f(None, 0, 0, 0, None) == 0                 # empty batch: no-op
    assert f(None, 3, 0, 1, None) == 0                 # no tiles: no-op


@pytest.mark.parametrize("fn", ["fp8_blockscaled_gemm", "fp8_blockscaled_gemm_pow2"])
def test_gemm_argument_errors(lib, fn):
    f = getattr(lib, fn)
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, 130, None) == 2
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 64, 100, 128, None) == 2
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, -1, 128, 128, None) == 1
    assert f(GOOD, None, GOOD, GOOD, GOOD, 64, 128, 128, None) == 1
    assert f(GOOD, GOOD, GOOD, GOOD, ODD, 64, 128, 128, None) == 3
    assert f(None, None, None, None, None, 0, 128, 128, None) == 0
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, (1 << 22) + 128, None) == 2   # K too large
    assert "K" in _err(lib)


def test_gemm_quant_argument_errors(lib):
    f = lib.fp8_blockscaled_gemm_quant
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, 128, 7, None) == 1      # unknown mode
    assert "mode" in _err(lib)
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, 130, 0, None) == 2      # K not a multiple of 128
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 100, 128, 1, None) == 2      # N not a multiple of 128
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, -1, 128, 128, 0, None) == 1
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, None, 64, 128, 128, 0, None) == 1      # null scales out
    assert f(GOOD, GOOD, GOOD, GOOD, ODD, GOOD, 64, 128, 128, 0, None) == 3       # misaligned y_q
    assert f(None, None, None, None, None, None, 0, 128, 128, 0, None) == 0       # empty call
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, (1 << 22) + 128, 0, None) == 2


def test_rmsnorm_quant_argument_errors(lib):
    import ctypes
    f = lib.fp8_rmsnorm_quant_1x128
    e = ctypes.c_float(1e-5)
    assert f(GOOD, GOOD, 4, 256, e, GOOD, GOOD, 3, None) == 1                     # unknown mode
    assert f(GOOD, GOOD, 4, 200, e, GOOD, GOOD, 0, None) == 2                     # K not a multiple of 128
    assert f(GOOD, GOOD, 4, 8192 + 128, e, GOOD, GOOD, 0, None) == 2              # K above 8192
    assert "8192" in _err(lib)
    assert f(GOOD, GOOD, 4, 256, ctypes.c_float(-1.0), GOOD, GOOD, 0, None) == 1  # negative eps
    assert f(GOOD, GOOD, 4, 256, ctypes.c_float(float("nan")), GOOD, GOOD, 0, None) == 1
    assert f(GOOD, GOOD, 4, 256, ctypes.c_float(float("inf")), GOOD, GOOD, 0, None) == 1
    assert f(GOOD, None, 4, 256, e, GOOD, GOOD, 0, None) == 1                     # null gamma
    assert f(GOOD, ODD, 4, 256, e, GOOD, GOOD, 0, None) == 3                      # misaligned gamma
    assert f(GOOD, GOOD, -1, 256, e, GOOD, GOOD, 0, None) == 1
    assert f(None, None, 0, 256, e, None, None, 0, None) == 0                     # empty call
    assert f(GOOD, GOOD, 1 << 26, 256, e, GOOD, GOOD, 0, None) == 2               # 64*M work-items >= 2^32
    assert "2^26" in _err(lib)


def test_launch_size_bounds(lib):
    """Sizes whose launch would exceed a dispatch's 2^32 work-items are refused
    on the host with FP8Q_ESHAPE (checked before any pointer or device)."""
    f = lib.fp8_quant_act_1x128
    assert f(GOOD, 1 << 22, 1 << 14, GOOD, GOOD, 0, None) == 2                     # M*K/128 = 2^29
    assert "2^29" in _err(lib)
    a = lib.fp8_attention_decode
    assert a(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1 << 21, 64, 8, 1, None, 0, None) == 2   # B*Hkv = 2^24
    assert "2^24" in _err(lib)


def test_gemm_swiglu_quant_argument_errors(lib):
    f = lib.fp8_blockscaled_gemm_swiglu_quant
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, 128, 2, None) == 1      # unknown mode
    assert "mode" in _err(lib)
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, 130, 0, None) == 2      # K not a multiple of 128
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 64, 128, 1, None) == 2       # F not a multiple of 128
    assert "F" in _err(lib)
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, -128, 128, 0, None) == 1
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, (1 << 30) + 128, 128, 0, None) == 1
    assert f(GOOD, GOOD, None, GOOD, GOOD, GOOD, 64, 128, 128, 0, None) == 1      # null weight
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, ODD, 64, 128, 128, 0, None) == 3       # misaligned h_s
    assert f(None, None, None, None, None, None, 64, 0, 128, 0, None) == 0        # F = 0: nothing to do
    assert f(None, None, None, None, None, None, 0, 128, 128, 0, None) == 0
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, (1 << 22) + 128, 0, None) == 2


@pytest.mark.parametrize("fn", ["fp8_grouped_gemm", "fp8_grouped_gemm_pow2"])
def test_grouped_argument_errors(lib, fn):
    f = getattr(lib, fn)
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 0, 64, 128, 128, GOOD, None) == 1   # G < 1
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 2, 64, 128, 100, GOOD, None) == 2
    assert f(GOOD, GOOD, GOOD, GOOD, None, 2, 64, 128, 128, GOOD, None) == 1   # null offsets
    assert f(GOOD, GOOD, GOOD, GOOD, ODD, 2, 64, 128, 128, GOOD, None) == 3
    assert f(None, None, None, None, None, 3, 0, 128, 128, None, None) == 0
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 2, 64, 128, (1 << 22) + 128, GOOD, None) == 2


def test_grouped_swiglu_quant_argument_errors(lib):
    f = lib.fp8_grouped_gemm_swiglu_quant
    #        aq    as    T   bq    bs    off   idx   G  M    F    K    hq    hs    mode
    assert f(GOOD, GOOD, 64, GOOD, GOOD, GOOD, GOOD, 2, 100, 128, 128, GOOD, GOOD, 2, None) == 1   # unknown mode
    assert "mode" in _err(lib)
    assert f(GOOD, GOOD, 64, GOOD, GOOD, GOOD, GOOD, 0, 100, 128, 128, GOOD, GOOD, 0, None) == 1   # G < 1
    assert f(GOOD, GOOD, 64, GOOD, GOOD, GOOD, GOOD, 2, 100, 64, 128, GOOD, GOOD, 0, None) == 2    # F % 128
    assert "F" in _err(lib)
    assert f(GOOD, GOOD, 64, GOOD, GOOD, GOOD, GOOD, 2, 100, 128, 200, GOOD, GOOD, 0, None) == 2   # K % 128
    assert f(GOOD, GOOD, 64, GOOD, GOOD, GOOD, GOOD, 2, -1, 128, 128, GOOD, GOOD, 0, None) == 1    # negative size
    assert f(GOOD, GOOD, 64, GOOD, GOOD, None, GOOD, 2, 100, 128, 128, GOOD, GOOD, 0, None) == 1   # null offsets
    assert f(GOOD, GOOD, 64, GOOD, GOOD, GOOD, GOOD, 2, 100, 128, 128, None, GOOD, 0, None) == 1   # null h_q
    assert f(GOOD, GOOD, 64, GOOD, GOOD, GOOD, ODD, 2, 100, 128, 128, GOOD, GOOD, 0, None) == 3    # misaligned index
    assert f(GOOD, GOOD, 0, GOOD, GOOD, GOOD, GOOD, 2, 100, 128, 128, GOOD, GOOD, 0, None) == 1    # T = 0, rows routed
    assert f(GOOD, GOOD, 1 << 20, GOOD, GOOD, GOOD, GOOD, 2, 100, 128, 4096, GOOD, GOOD, 0, None) == 2  # T*K = 2^32
    assert "2^31" in _err(lib)
    assert f(None, None, 0, None, None, None, None, 2, 0, 128, 128, None, None, 0, None) == 0      # no routed rows
    assert f(GOOD, GOOD, 64, GOOD, GOOD, GOOD, GOOD, 2, 100, 128, (1 << 22) + 128, GOOD, GOOD, 0, None) == 2


@pytest.mark.parametrize("fn", ["fp8_quant_act_dual", "fp8_quant_weight_128x128_dual"])
def test_dual_quantizer_argument_errors(lib, fn):
    f = getattr(lib, fn)
    #        x     M    K    q     s     q_t   s_t   mode
    assert f(GOOD, 128, 100, GOOD, GOOD, GOOD, GOOD, 0, None) == 2       # K % 128
    assert f(GOOD, -1, 128, GOOD, GOOD, GOOD, GOOD, 0, None) == 1        # negative size
    assert f(GOOD, 128, 128, GOOD, GOOD, GOOD, GOOD, 3, None) == 1       # unknown mode
    assert f(GOOD, 128, 128, GOOD, None, GOOD, GOOD, 0, None) == 1       # q without scales
    assert "both" in _err(lib)
    assert f(GOOD, 128, 128, None, None, None, GOOD, 0, None) == 1       # no transposed output
    assert f(GOOD, 128, 128, None, None, GOOD, ODD, 0, None) == 3        # misaligned scales_t
    assert f(GOOD, 128, 128, ODD, GOOD, GOOD, GOOD, 0, None) == 3        # misaligned q
    assert f(None, 0, 128, None, None, None, None, 0, None) == 0         # empty call
    if fn == "fp8_quant_weight_128x128_dual":
        assert f(GOOD, 100, 128, GOOD, GOOD, GOOD, GOOD, 0, None) == 2   # N % 128


@pytest.mark.parametrize("fn", ["fp8_blockscaled_gemm_wgrad", "fp8_blockscaled_gemm_wgrad_pow2"])
def test_wgrad_argument_errors(lib, fn):
    f = getattr(lib, fn)
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, 130, None) == 2      # K % 128
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 64, 100, 128, None) == 2      # N % 128
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, -1, 128, 128, None) == 1
    assert f(GOOD, GOOD, GOOD, None, GOOD, 64, 128, 128, None) == 1      # null pointer
    assert f(GOOD, GOOD, ODD, GOOD, GOOD, 64, 128, 128, None) == 3
    assert f(None, None, None, None, None, 0, 128, 128, None) == 0       # empty call
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, 64, 128, (1 << 22) + 128, None) == 2


def test_kv_cache_append_argument_errors(lib):
    f = lib.fp8_kv_cache_append
    #        k_new v_new pos   kc    ks    vc    vs    B  H  S   mode
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 8, 64, 3, None) == 1     # unknown mode
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, -1, 8, 64, 0, None) == 1    # negative size
    assert f(GOOD, GOOD, None, GOOD, GOOD, GOOD, GOOD, 2, 8, 64, 0, None) == 1     # null positions
    assert f(GOOD, GOOD, GOOD, GOOD, ODD, GOOD, GOOD, 2, 8, 64, 1, None) == 3      # misaligned
    assert f(None, None, None, None, None, None, None, 0, 8, 64, 0, None) == 0     # empty call


def test_kv_cache_append_tokens_argument_errors(lib):
    f = lib.fp8_kv_cache_append_tokens
    #        k_new v_new start kc    ks    vc    vs    B  T   H  S   mode
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 16, 8, 64, 3, None) == 1     # unknown mode
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, -1, 8, 64, 0, None) == 1     # negative T
    assert f(GOOD, GOOD, None, GOOD, GOOD, GOOD, GOOD, 2, 16, 8, 64, 0, None) == 1     # null start
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, ODD, GOOD, 2, 16, 8, 64, 1, None) == 3      # misaligned
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1 << 20, 1 << 12, 8, 64, 0, None) == 2   # B*T*H = 2^35
    assert f(None, None, None, None, None, None, None, 2, 0, 8, 64, 0, None) == 0     # no tokens


def test_attention_prefill_argument_errors(lib):
    f = lib.fp8_attention_prefill
    #        qq    qs    kc    ks    vc    vs    start out   B  T   Hq  Hkv S
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 64, 32, 6, 128, None) == 2     # Hq % Hkv
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 64, 32, 0, 128, None) == 2     # Hkv = 0
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, -1, 32, 8, 128, None) == 1     # negative T
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 64, 32, 8, 1 << 31, None) == 2  # S = 2^31
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1 << 20, 1 << 16, 32, 8, 128, None) == 2  # grid
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, 2, 64, 32, 8, 128, None) == 1     # null start
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, ODD, 2, 64, 32, 8, 128, None) == 3      # misaligned out
    assert f(None, None, None, None, None, None, None, None, 2, 0, 32, 8, 128, None) == 0      # no queries


def test_attention_decode_argument_errors(lib):
    f = lib.fp8_attention_decode
    #        qq    qs    kc    ks    vc    vs    len   out   B  Hq  Hkv S   ws  bytes
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 32, 6, 64, None, 0, None) == 2    # Hq % Hkv
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 48, 3, 64, None, 0, None) == 2    # 16 per group
    assert "1, 2, 4 or 8" in _err(lib)
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 32, 0, 64, None, 0, None) == 2    # Hkv = 0
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, -1, 32, 8, 64, None, 0, None) == 1   # negative size
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, 2, 32, 8, 64, None, 0, None) == 1    # null seq_len
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, ODD, 2, 32, 8, 64, None, 0, None) == 3     # misaligned out
    # 16 (sequence, head) pairs: 32 chunks of two tiles would be wanted, at
    # least four tiles each -> 16 chunks of 4 tiles for 4096 tokens
    need = lib.fp8_attention_decode_workspace_size(2, 32, 8, 4096)
    assert need == 2 * 32 * 16 * 130 * 4
    assert lib.fp8_attention_decode_workspace_size(64, 32, 8, 8192) == 0    # 512 pairs fill the GPU
    assert lib.fp8_attention_decode_workspace_size(2, 32, 8, 256) == 0      # four tiles: one chunk
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 32, 8, 4096, GOOD, need - 4, None) == 1
    assert "workspace" in _err(lib)
    assert f(None, None, None, None, None, None, None, None, 0, 32, 8, 64, None, 0, None) == 0    # empty call


def test_attention_decode_noalloc_argument_errors(lib):
    f = lib.fp8_attention_decode_noalloc
    #        qq    qs    kc    ks    vc    vs    len   out   B  Hq  Hkv S
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 32, 6, 64, None) == 2      # Hq % Hkv
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 2, 48, 3, 64, None) == 2      # 16 per group
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, -1, 32, 8, 64, None) == 1     # negative size
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, None, GOOD, 2, 32, 8, 64, None) == 1      # null seq_len
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, ODD, 2, 32, 8, 64, None) == 3       # misaligned out
    assert f(GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, GOOD, 1 << 21, 64, 8, 1, None) == 2  # B*Hkv = 2^24
    assert f(None, None, None, None, None, None, None, None, 0, 32, 8, 64, None) == 0      # empty call


def test_noalloc_scratch_covers_every_split():
    """The static scratch of fp8_attention_decode_noalloc (the header's
    FP8Q_NOALLOC_SCRATCH_BYTES) is at least the workspace any accepted size
    asks for: the worst case of the split rule is 511 pairs in two chunks
    with 8 query heads per key/value head."""
    from blockwise_scaled_fp8_quant_amd import _lib
    lib = _lib.load()
    text = open(HEADER).read()
    cap = int(re.search(r"#define FP8Q_NOALLOC_SCRATCH_BYTES (\d+)", text).group(1))
    worst = 0
    for B, Hkv in [(511, 1), (1, 511), (73, 7), (255, 2), (64, 8), (1, 1), (2, 8), (16, 8), (3, 4)]:
        for grp in (1, 2, 4, 8):
            for S in (1, 256, 257, 260, 4096, 65536, 1 << 20, (1 << 31) - 1):
                worst = max(worst, lib.fp8_attention_decode_workspace_size(B, grp * Hkv, Hkv, S))
    assert worst == cap == 8 * 1022 * 130 * 4


def test_gemm_tile_plan(lib):
    """Tile plans: all 256-token tiles for gate+up and down at 4096 tokens; QKV
    split by weight panels (16 of 24 large, one round on each shape); the
    weight gradient of QKV (dW 6144 x 4096) split by rows (4096 large); all
    small tiles for O at 2048 tokens; the SwiGLU GEMM's output is not split."""
    import ctypes
    f = lib.fp8_blockscaled_gemm_tile_plan

    def plan(M, N, swiglu=0):
        r = ctypes.c_int64(-7)
        p = f(M, N, swiglu, ctypes.byref(r))
        return r.value, p
    assert plan(4096, 28672) == (4096, 112) and plan(4096, 4096) == (4096, 16)
    assert plan(4096, 6144) == (4096, 16)
    assert plan(4096, 6144, 1) in ((0, 0), (4096, 24))
    assert plan(6144, 4096) == (4096, 16)
    assert plan(2048, 4096) == (0, 0)
    assert f(4096, 6144, 0, None) == 16
    assert f(0, 128, 0, None) == -1 and f(64, 100, 0, None) == -1


def test_moe_permute_argument_errors(lib):
    f = lib.fp8_moe_permute
    ws = lib.fp8_moe_permute_workspace_size(100, 8, 128)
    assert ws == (100 * 8 * 4 + 255) // 256 * 256 + 128 * 4     # ranks, then 128 experts x 1 block of counts
    assert lib.fp8_moe_permute_workspace_size(100, 8, 2048) == 0     # too many experts
    assert lib.fp8_moe_permute_workspace_size(-1, 8, 128) == 0
    #        ids   T    k  E    ns off   rows  entry ws    bytes
    assert f(GOOD, -1, 8, 128, 0, GOOD, GOOD, None, GOOD, ws, None) == 1           # negative T
    assert f(GOOD, 100, 0, 128, 0, GOOD, GOOD, None, GOOD, ws, None) == 1          # k = 0
    assert f(GOOD, 100, 8, 0, 0, GOOD, GOOD, None, GOOD, ws, None) == 2            # E = 0
    assert f(GOOD, 100, 8, 1025, 0, GOOD, GOOD, None, GOOD, ws, None) == 2         # E > 1024
    assert f(GOOD, 1 << 28, 8, 128, 0, GOOD, GOOD, None, GOOD, ws, None) == 2      # rows >= 2^31
    assert f(GOOD, 100, 8, 128, 0, None, GOOD, None, GOOD, ws, None) == 1          # null offsets
    assert f(GOOD, 100, 8, 128, 0, GOOD, GOOD, ODD, GOOD, ws, None) == 3           # misaligned entry_row
    assert f(GOOD, 100, 8, 128, 0, GOOD, GOOD, None, GOOD, ws - 4, None) == 1      # workspace too small
    assert "workspace" in _err(lib)


def test_gather_argument_errors(lib):
    f = lib.fp8_grouped_gemm_gather
    #      a_q   a_s   T    b_q   b_s   off   idx   G  M   N    K    y     mode
    assert f(GOOD, GOOD, 10, GOOD, GOOD, GOOD, GOOD, 2, 64, 128, 128, GOOD, 5, None) == 1    # unknown mode
    assert "mode" in _err(lib)
    assert f(GOOD, GOOD, 10, GOOD, GOOD, GOOD, GOOD, 0, 64, 128, 128, GOOD, 0, None) == 1    # G < 1
    assert f(GOOD, GOOD, -1, GOOD, GOOD, GOOD, GOOD, 2, 64, 128, 128, GOOD, 0, None) == 1    # T < 0
    assert f(GOOD, GOOD, 10, GOOD, GOOD, GOOD, GOOD, 2, 64, 128, 100, GOOD, 0, None) == 2    # K % 128
    assert f(GOOD, GOOD, 10, GOOD, GOOD, GOOD, GOOD, 2, 64, 100, 128, GOOD, 1, None) == 2    # N % 128
    assert f(GOOD, GOOD, 1 << 24, GOOD, GOOD, GOOD, GOOD, 2, 64, 128, 128, GOOD, 0, None) == 2   # T*K = 2^31
    assert "2^31" in _err(lib)
    assert f(GOOD, GOOD, (1 << 24) - 1, GOOD, GOOD, GOOD, None, 2, 64, 128, 128, GOOD, 0, None) == 1  # null idx
    assert f(GOOD, GOOD, 0, GOOD, GOOD, GOOD, GOOD, 2, 64, 128, 128, GOOD, 0, None) == 1     # no tokens
    assert f(GOOD, GOOD, 10, GOOD, GOOD, GOOD, ODD, 2, 64, 128, 128, GOOD, 0, None) == 3     # misaligned idx
    assert f(None, None, 0, None, None, None, None, 3, 0, 128, 128, None, 0, None) == 0      # empty call
    assert f(GOOD, GOOD, 10, GOOD, GOOD, GOOD, GOOD, 2, 64, 128, (1 << 22) + 128, GOOD, 0, None) == 2


def test_valid_call_without_gpu_reports_device_error(lib):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present")
    assert lib.fp8_quant_act_1x128(GOOD, 1, 128, GOOD, GOOD, 0, None) == 4
    assert "device" in _err(lib) or "HIP" in _err(lib) or _err(lib)


def test_python_binding_rejects_host_tensors():
    import torch
    import blockwise_scaled_fp8_quant_amd as fp8q
    with pytest.raises(ValueError):
        fp8q.fp8_quant_act_1x128(torch.zeros((4, 128), dtype=torch.bfloat16))
    with pytest.raises(ValueError):
        fp8q.fp8_quant_act_1x128(torch.zeros((4, 128), dtype=torch.bfloat16), mode="nope")
