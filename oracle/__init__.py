"""CPU oracle for the blockwise-scaled FP8 linear layer.

TEST INFRASTRUCTURE, NOT PRODUCT CODE: only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import this package.  It shares
no code with the HIP path.
"""
from .oracle import (  # noqa: F401
    MODE_AMAX,
    MODE_POW2,
    build,
    e4m3_decode_table,
    e4m3_encode,
    block_scale,
    quant_act_1x128,
    quant_weight_128x128,
    gemm_f64,
    round_bf16,
    gemm_quant_1x128,
    gemm_sampled_f64,
    grouped_gemm_f64,
    grouped_gemm_sampled_f64,
    quant_act_colwise_t,
    quant_weight_128x128_t,
    gemm_dgrad_f64,
    gemm_dgrad_sampled_f64,
    gemm_wgrad_f64,
    gemm_wgrad_sampled_f64,
    kv_cache_append,
    attention_decode_f64,
    kv_cache_append_tokens,
    attention_prefill_f64,
    swiglu_split,
    bf16_to_f64,
    swiglu_h_f64,
    gemm_swiglu_quant,
    grouped_gemm_swiglu_quant,
    grouped_gemm_swiglu_quant_rows,
    rmsnorm_f64,
    rmsnorm_quant_1x128,
    moe_permute,
    num_threads,
    set_num_threads,
)
