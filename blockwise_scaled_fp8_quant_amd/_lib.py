"""ctypes loader of libfp8q.so (the HIP kernels behind the C ABI in include/fp8q.h).

There is no fallback: if the library is missing or fails to load, every entry
point raises.
"""
import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libfp8q.so")

FP8Q_OK = 0
STATUS_NAMES = {0: "FP8Q_OK", 1: "FP8Q_EINVAL", 2: "FP8Q_ESHAPE", 3: "FP8Q_EALIGN",
                4: "FP8Q_EDEVICE", 5: "FP8Q_EHIP"}
ENTRY_POINTS = ("fp8_quant_act_1x128", "fp8_rmsnorm_quant_1x128", "fp8_quant_weight_128x128",
                "fp8_quant_weight_128x128_batched",
                "fp8_blockscaled_gemm",
                "fp8_grouped_gemm", "fp8_blockscaled_gemm_pow2", "fp8_grouped_gemm_pow2",
                "fp8_blockscaled_gemm_quant", "fp8_blockscaled_gemm_swiglu_quant", "fp8_grouped_gemm_gather",
                "fp8_grouped_gemm_swiglu_quant", "fp8_quant_act_dual",
                "fp8_quant_weight_128x128_dual", "fp8_blockscaled_gemm_wgrad", "fp8_blockscaled_gemm_wgrad_pow2",
                "fp8_kv_cache_append", "fp8_kv_cache_append_tokens", "fp8_attention_prefill",
                "fp8_attention_decode", "fp8_attention_decode_workspace_size", "fp8_attention_decode_noalloc",
                "fp8_moe_permute", "fp8_moe_permute_workspace_size", "fp8_blockscaled_gemm_tile_plan",
                "fp8q_status_string", "fp8q_last_error", "fp8q_abi_version")

_lib = None


class Fp8qError(RuntimeError):
    def __init__(self, fn, status, message):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({message})")


def load():
    """Load (once) and return the library; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} not found: build the HIP library first "
            "(python -m blockwise_scaled_fp8_quant_amd.build)")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32, ci = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_int
    lib.fp8_quant_act_1x128.argtypes = [p, i64, i64, p, p, ci, p]
    lib.fp8_quant_act_1x128.restype = ci
    lib.fp8_rmsnorm_quant_1x128.argtypes = [p, p, i64, i64, ctypes.c_float, p, p, ci, p]
    lib.fp8_rmsnorm_quant_1x128.restype = ci
    lib.fp8_quant_weight_128x128.argtypes = [p, i64, i64, p, p, ci, p]
    lib.fp8_quant_weight_128x128.restype = ci
    lib.fp8_quant_weight_128x128_batched.argtypes = [p, i32, i64, ci, p]
    lib.fp8_quant_weight_128x128_batched.restype = ci
    for name in ("fp8_quant_act_dual", "fp8_quant_weight_128x128_dual"):
        getattr(lib, name).argtypes = [p, i64, i64, p, p, p, p, ci, p]
        getattr(lib, name).restype = ci
    for name in ("fp8_blockscaled_gemm", "fp8_blockscaled_gemm_pow2", "fp8_blockscaled_gemm_wgrad",
                 "fp8_blockscaled_gemm_wgrad_pow2"):
        getattr(lib, name).argtypes = [p, p, p, p, p, i64, i64, i64, p]
        getattr(lib, name).restype = ci
    lib.fp8_blockscaled_gemm_quant.argtypes = [p, p, p, p, p, p, i64, i64, i64, ci, p]
    lib.fp8_blockscaled_gemm_quant.restype = ci
    lib.fp8_blockscaled_gemm_swiglu_quant.argtypes = [p, p, p, p, p, p, i64, i64, i64, ci, p]
    lib.fp8_blockscaled_gemm_swiglu_quant.restype = ci
    for name in ("fp8_grouped_gemm", "fp8_grouped_gemm_pow2"):
        getattr(lib, name).argtypes = [p, p, p, p, p, i32, i64, i64, i64, p, p]
        getattr(lib, name).restype = ci
    lib.fp8_grouped_gemm_gather.argtypes = [p, p, i64, p, p, p, p, i32, i64, i64, i64, p, ci, p]
    lib.fp8_grouped_gemm_gather.restype = ci
    lib.fp8_grouped_gemm_swiglu_quant.argtypes = [p, p, i64, p, p, p, p, i32, i64, i64, i64, p, p, ci, p]
    lib.fp8_grouped_gemm_swiglu_quant.restype = ci
    lib.fp8_kv_cache_append.argtypes = [p, p, p, p, p, p, p, i32, i32, i64, ci, p]
    lib.fp8_kv_cache_append.restype = ci
    lib.fp8_kv_cache_append_tokens.argtypes = [p, p, p, p, p, p, p, i32, i32, i32, i64, ci, p]
    lib.fp8_kv_cache_append_tokens.restype = ci
    lib.fp8_attention_prefill.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, i32, i64, p]
    lib.fp8_attention_prefill.restype = ci
    lib.fp8_attention_decode.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, i64, p, i64, p]
    lib.fp8_attention_decode.restype = ci
    lib.fp8_blockscaled_gemm_tile_plan.argtypes = [i64, i64, ci, ctypes.POINTER(ctypes.c_int64)]
    lib.fp8_blockscaled_gemm_tile_plan.restype = i32
    lib.fp8_moe_permute.argtypes = [p, i64, i32, i32, i32, p, p, p, p, i64, p]
    lib.fp8_moe_permute.restype = ci
    lib.fp8_moe_permute_workspace_size.argtypes = [i64, i32, i32]
    lib.fp8_moe_permute_workspace_size.restype = i64
    lib.fp8_attention_decode_noalloc.argtypes = [p, p, p, p, p, p, p, p, i32, i32, i32, i64, p]
    lib.fp8_attention_decode_noalloc.restype = ci
    lib.fp8_attention_decode_workspace_size.argtypes = [i32, i32, i32, i64]
    lib.fp8_attention_decode_workspace_size.restype = i64
    lib.fp8q_status_string.argtypes = [ci]
    lib.fp8q_status_string.restype = ctypes.c_char_p
    lib.fp8q_last_error.argtypes = []
    lib.fp8q_last_error.restype = ctypes.c_char_p
    lib.fp8q_abi_version.argtypes = []
    lib.fp8q_abi_version.restype = ci
    _lib = lib
    return lib


def check(fn, status):
    if status != FP8Q_OK:
        msg = load().fp8q_last_error().decode(errors="replace")
        raise Fp8qError(fn, status, msg)
