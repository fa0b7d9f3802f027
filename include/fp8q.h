/*
 * fp8q.h -- C ABI of the blockwise-scaled FP8 linear layer for AMD MI355X
 * (CDNA4, gfx950).
 *
 * The layer is the one of the end-to-end FP8 reinforcement-learning recipe
 * described on the page "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung
 * mit End-to-End FP8-Praezisionstraining":
 *   - section "Der technische Durchbruch": linear layers compute in FP8 E4M3,
 *     with one scale per 1x128 block of activations and one per 128x128 block
 *     of weights;
 *   - section "Leistungsgewinne in der Praxis": the weight scales are
 *     recalibrated (and the weights requantized) after every policy update;
 *   - section "Warum dies fuer die KI-Oekonomie wichtig ist": the scales may be
 *     restricted to powers of two.
 * The +-448 range of E4M3 is from the page "FP8 Trainingsinfrastructuur:
 * Numerieke Precisie van de Volgende Generatie", section "Het landschap van
 * numerieke precisie".
 *
 * Conventions shared by every entry point
 *  - Memory: every tensor pointer is DEVICE memory, allocated and owned by the
 *    caller.  The library allocates nothing and keeps no per-call state; it is
 *    reentrant and may be called from several host threads.
 *  - Layout: all tensors are dense and row-major, no strides.  bf16 values are
 *    passed as their raw 16-bit patterns, E4M3 values as raw bytes (OCP
 *    "E4M3FN": bias 7, largest finite 448, NaN only 0x7F/0xFF), scales as fp32.
 *  - Scales are dequantisation multipliers: x ~= decode(q) * s.
 *  - Alignment: every pointer must be 16-byte aligned (torch allocations are).
 *  - Shapes: K is a positive multiple of 128; N is a multiple of 128; M (and
 *    every group size) is any value >= 0 -- ragged tails are masked.  M == 0 or
 *    N == 0 is a valid empty call that enqueues nothing.  The GEMMs accept
 *    K <= 4194304 (FP8Q_ESHAPE otherwise).
 *  - Execution: each call enqueues its kernels on `stream` (a hipStream_t; NULL
 *    is the null stream) and returns without synchronising.  The outputs are
 *    valid once the stream reaches that point.
 *  - Errors: arguments are checked on the host before anything is enqueued; on
 *    any error nothing is enqueued and the outputs are untouched.  A HIP launch
 *    failure returns FP8Q_EHIP.  fp8q_last_error() gives a message for the last
 *    failing call of the calling thread.
 *  - Inputs must be finite (no NaN or Inf); the results for other inputs are
 *    unspecified but every access stays inside the given tensors.
 *  - Determinism: the same inputs give the same output bits on every call.
 */
#ifndef FP8Q_H
#define FP8Q_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP8Q_ABI_VERSION 1

typedef enum fp8q_status {
    FP8Q_OK = 0,
    FP8Q_EINVAL = 1,  /* null pointer, negative size, unknown mode, G < 1 */
    FP8Q_ESHAPE = 2,  /* K not a positive multiple of 128 (or, for a GEMM, above 4194304), or N not a multiple of 128 */
    FP8Q_EALIGN = 3,  /* a pointer not 16-byte aligned (a batched job table: not 8-byte aligned) */
    FP8Q_EDEVICE = 4, /* no HIP device, or the current device is not gfx950 */
    FP8Q_EHIP = 5     /* the HIP runtime reported an error while enqueueing */
} fp8q_status;

/* Scale rule of one block whose largest magnitude is amax.  An all-zero block
 * (amax == 0) always gets s = 1. */
typedef enum fp8q_scale_mode {
    FP8Q_SCALE_AMAX = 0, /* s = amax / 448, rounded to the nearest fp32 */
    FP8Q_SCALE_POW2 = 1  /* s = 2^e, e the smallest integer >= -127 with 448 * 2^e >= amax */
} fp8q_scale_mode;

/*
 * Dynamic activation quantization, 1x128 blocks (page 1, "Der technische
 * Durchbruch").
 *   x       [M][K] bf16 bits (in)
 *   q       [M][K] E4M3 bytes (out)
 *   scales  [M][K/128] fp32 (out): block (m, kb) covers x[m][128*kb .. 128*kb+127]
 *   mode    fp8q_scale_mode
 * Every element: q = E4M3(RN_fp32(x / s)), rounded to nearest with ties to an
 * even mantissa and saturated to +-448; a zero keeps its sign.
 * The result is bit-identical to that rule for every finite input.
 * Sizes: M*K/128 < 2^29 (FP8Q_ESHAPE otherwise; the launch's work-items stay
 * below 2^32).
 */
fp8q_status fp8_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K,
                                uint8_t *q, float *scales, int mode,
                                void *stream);

/*
 * RMS normalization with its output quantized in 1x128 blocks, in one pass:
 * the norms ahead of a block's QKV and gate+up projections produce those
 * layers' FP8 inputs directly (page 1, "Leistungsgewinne in der Praxis":
 * separate quantization kernels are part of the gap to 2x).
 *   x       [M][K] bf16 bits (in), K a multiple of 128, 128 <= K <= 8192
 *   gamma   [K] bf16 bits (in): the norm's weight
 *   eps     finite, >= 0
 *   q       [M][K] E4M3 bytes (out), scales [M][K/128] fp32 (out), laid out
 *           as by fp8_quant_act_1x128
 *   mode    fp8q_scale_mode
 * y = bf16_RNE((x * r) * gamma) with r = 1 / sqrt(sum(x^2) / K + eps), each
 * step in fp32 (the sum of squares in a fixed but unspecified order), and y
 * is then quantized exactly as fp8_quant_act_1x128 quantizes a bf16 input.
 * Against y computed exactly, the fp32 steps cost a few fp32 ulp, which can
 * move the bf16 rounding (and then a code) where y sits on a rounding
 * midpoint.  Precondition, as for the quantizer: finite x and gamma; with
 * eps = 0 also no row whose mean square is 0 in fp32 (an all-zero row, or
 * values below about 1e-19, whose squares underflow); the outputs of such a
 * row are unspecified.
 * Sizes: M < 2^26 (one 64-lane wave per row; FP8Q_ESHAPE otherwise).
 */
fp8q_status fp8_rmsnorm_quant_1x128(const uint16_t *x, const uint16_t *gamma,
                                    int64_t M, int64_t K, float eps,
                                    uint8_t *q, float *scales, int mode,
                                    void *stream);

/*
 * Weight recalibration and requantization, 128x128 blocks (page 1, "Der
 * technische Durchbruch" and "Leistungsgewinne in der Praxis"; power-of-two
 * mode: "Warum dies fuer die KI-Oekonomie wichtig ist").
 *   w       [N][K] bf16 bits (in), N and K multiples of 128
 *   q       [N][K] E4M3 bytes (out)
 *   scales  [N/128][K/128] fp32 (out): tile (nb, kb) covers rows 128*nb.. and
 *           columns 128*kb.. (127 more each)
 *   mode    fp8q_scale_mode
 * Element rule as in fp8_quant_act_1x128, with the tile's scale.
 */
fp8q_status fp8_quant_weight_128x128(const uint16_t *w, int64_t N, int64_t K,
                                     uint8_t *q, float *scales, int mode,
                                     void *stream);

/*
 * One matrix of a batched weight recalibration (fp8_quant_weight_128x128_batched).
 *   w, q, scales  as the arguments of fp8_quant_weight_128x128 (device memory,
 *                 16-byte aligned)
 *   N, K          the matrix shape: N >= 0 and K > 0, both multiples of 128
 *   tile_begin    the sum of (N/128)*(K/128) over the jobs before this one
 */
typedef struct fp8q_weight_job {
    const uint16_t *w;
    uint8_t *q;
    float *scales;
    int64_t N;
    int64_t K;
    int64_t tile_begin;
} fp8q_weight_job;

/*
 * Recalibration of a whole set of weights in one launch (page 1,
 * "Leistungsgewinne in der Praxis": every weight's scales are recomputed after
 * each policy update).  Each job is quantized exactly as
 * fp8_quant_weight_128x128 quantizes it, with the same bytes and scales; one
 * launch for all of them pays a launch's start-up and drain once instead of
 * once per matrix.
 *   jobs         [count] fp8q_weight_job in DEVICE memory, read by the kernel
 *                when it runs: it must stay valid and unchanged until the
 *                call's work on the stream has completed (build it once per
 *                set of weights and keep it)
 *   count        number of jobs, >= 0
 *   total_tiles  sum of (N/128)*(K/128) over the jobs, < 2^31
 *   mode         fp8q_scale_mode, for every job
 * The host checks count, total_tiles, mode, the table's alignment (8 bytes)
 * and that the table is device (or managed) memory (else FP8Q_EINVAL); it
 * cannot read the table's contents.  On the device a tile whose job
 * has a shape that is not a positive multiple of 128, or which falls outside
 * its job's range of tiles (tile_begin not the running sum), is skipped: its
 * outputs are left as they were, and no access leaves a job's tensors.  Jobs
 * must not write to one another's inputs.  Every workgroup finds its job by
 * reading the table's tile_begin fields in rounds of 64 jobs, so the lookup
 * cost grows with count: meant for weight sets of up to a few thousand
 * matrices (a whole model's linear layers is a few hundred).
 */
fp8q_status fp8_quant_weight_128x128_batched(const fp8q_weight_job *jobs, int32_t count,
                                             int64_t total_tiles, int mode, void *stream);

/*
 * Both quantized layouts of an activation (or activation gradient) in one
 * pass, for training end to end in FP8 (page 1, title and "Der technische
 * Durchbruch": FP8 in training as well as in generation).  Each GEMM takes its
 * scale blocks along its contraction dimension: the forward product and the
 * data gradient read 1x128 blocks along a row; the weight gradient
 * dW = dY^T X contracts over the tokens and reads blocks of 128 tokens x 1
 * channel, stored transposed so that they too are contiguous rows.
 *   x         [M][K] bf16 bits (in), M >= 0 any, K a multiple of 128
 *   q         [M][K] E4M3 (out) and scales [M][K/128] (out): exactly the
 *             outputs of fp8_quant_act_1x128.  Both may be NULL (then only the
 *             transposed layout is written).
 *   q_t       [K][Mp] E4M3 (out), Mp = M rounded up to a multiple of 128:
 *             q_t[k][m] is x[m][k] quantized with the scale of its block of
 *             rows 128*(m/128) .. +127 of column k; for m >= M it is 0x00.
 *   scales_t  [K][Mp/128] fp32 (out): block (k, mb) covers x[128*mb ..][k]
 *             (the rows below M only; rows past M count as zeros).
 *   mode      fp8q_scale_mode, for both layouts
 * Each 128x1 block follows exactly the rule of a 1x128 block of
 * fp8_quant_act_1x128 (amax, scale, element rule).
 */
fp8q_status fp8_quant_act_dual(const uint16_t *x, int64_t M, int64_t K,
                               uint8_t *q, float *scales,
                               uint8_t *q_t, float *scales_t, int mode,
                               void *stream);

/*
 * Both layouts of a quantized weight in one pass (the data gradient
 * dX = dY W reads W's 128x128 tiles with N as its contraction dimension,
 * i.e. W^T row-major; a tile of W^T holds the values of one tile of W).
 *   w         [N][K] bf16 bits (in), N and K multiples of 128
 *   q, scales exactly the outputs of fp8_quant_weight_128x128 (both may be NULL)
 *   q_t       [K][N] E4M3 (out): q_t[k][n] = q[n][k]
 *   scales_t  [K/128][N/128] fp32 (out): scales_t[kb][nb] = scales[nb][kb]
 *   mode      fp8q_scale_mode
 * With q_t and scales_t, dX = fp8_blockscaled_gemm(dY_q, dY_s, q_t, scales_t)
 * with M = tokens, N = K of the layer, K = N of the layer.
 */
fp8q_status fp8_quant_weight_128x128_dual(const uint16_t *w, int64_t N, int64_t K,
                                          uint8_t *q, float *scales,
                                          uint8_t *q_t, float *scales_t, int mode,
                                          void *stream);

/*
 * Block-scaled FP8 GEMM of a linear layer, Y = X * W^T (page 1, "Der
 * technische Durchbruch"; the GEMM outputs feed bf16 operators):
 *   Y[m][n] = sum_kb a_s[m][kb] * b_s[n/128][kb] *
 *                    sum_{k in block kb} dec(a_q[m][k]) * dec(b_q[n][k])
 * with fp32 accumulation; Y is rounded once to bf16 (nearest, ties to even).
 *   a_q [M][K] E4M3, a_s [M][K/128] fp32   (from fp8_quant_act_1x128)
 *   b_q [N][K] E4M3, b_s [N/128][K/128]     (from fp8_quant_weight_128x128)
 *   y   [M][N] bf16 bits (out)
 * The summation order inside the GPU is fixed but unspecified; results agree
 * with the exact value to within fp32 accumulation and the final bf16 rounding.
 */
fp8q_status fp8_blockscaled_gemm(const uint8_t *a_q, const float *a_s,
                                 const uint8_t *b_q, const float *b_s,
                                 uint16_t *y, int64_t M, int64_t N, int64_t K,
                                 void *stream);

/*
 * The same GEMM with its output quantized for the next FP8 layer: Y is
 * computed and rounded to bf16 exactly as by fp8_blockscaled_gemm, and then
 * quantized in 1x128 blocks along N exactly as fp8_quant_act_1x128 quantizes
 * a bf16 input -- in the GEMM's epilogue, so the bf16 Y never goes to memory
 * and no separate quantization pass reads it back (page 1, "Leistungsgewinne
 * in der Praxis": quantization-kernel overhead is part of the gap between the
 * FP8 linear layers' gain and the ideal 2x).
 *   a_q, a_s, b_q, b_s as for fp8_blockscaled_gemm
 *   y_q [M][N] E4M3 bytes (out)
 *   y_s [M][N/128] fp32 (out): block (m, nb) covers Y[m][128*nb .. 128*nb+127]
 *   mode fp8q_scale_mode of the output blocks
 * y_q and y_s are bit-identical to fp8_quant_act_1x128(mode) applied to the
 * y of fp8_blockscaled_gemm on the same inputs.
 */
fp8q_status fp8_blockscaled_gemm_quant(const uint8_t *a_q, const float *a_s,
                                       const uint8_t *b_q, const float *b_s,
                                       uint8_t *y_q, float *y_s,
                                       int64_t M, int64_t N, int64_t K, int mode,
                                       void *stream);

/*
 * The fused gate and up projections of a SwiGLU MLP with the activation of
 * the down projection quantized in the epilogue: the 1x128 quantization of
 *   h = silu(gate) * up,  silu(g) = g / (1 + e^-g),
 * where gate and up are the two halves of one block-scaled FP8 GEMM against
 * the concatenated weight, each rounded to bf16 as fp8_blockscaled_gemm rounds
 * its output.  The bf16 gate, up and h never go to memory (page 1,
 * "Leistungsgewinne in der Praxis": quantization-kernel overhead is part of
 * the gap between the FP8 linear layers' gain and the ideal 2x).
 *   a_q [M][K], a_s [M][K/128]    as for fp8_blockscaled_gemm
 *   b_q [2F][K], b_s [2F/128][K/128]  the weight with gate and up rows in
 *                                 alternating 128-row blocks: rows
 *                                 256p .. 256p+127 are gate rows 128p .., rows
 *                                 256p+128 .. 256p+255 the up rows of the same
 *                                 output features; each block is one 128x128
 *                                 tile row of the quantized weight
 *   h_q [M][F] E4M3 bytes (out), h_s [M][F/128] fp32 (out): block (m, fb)
 *                                 covers h[m][128*fb .. 128*fb+127]
 *   F  output features, a positive multiple of 128 (0 returns at once)
 *   mode fp8q_scale_mode of the output blocks (the weight's own scales are
 *        read as fp8_blockscaled_gemm reads them, either mode)
 * h is formed in fp32 from the bf16 gate and up (the exponential is the
 * hardware's base-2 one, a few ulp from exact) and rounded to bf16 (nearest
 * even) before the 1x128 quantization, whose rule is fp8_quant_act_1x128's.
 * Errors as for fp8_blockscaled_gemm_quant.
 */
fp8q_status fp8_blockscaled_gemm_swiglu_quant(const uint8_t *a_q, const float *a_s,
                                              const uint8_t *b_q, const float *b_s,
                                              uint8_t *h_q, float *h_s,
                                              int64_t M, int64_t F, int64_t K, int mode,
                                              void *stream);

/*
 * Block-scaled FP8 GEMM with 1x128 blocks on both operands: the weight
 * gradient of a linear layer (training end to end in FP8, page 1, title and
 * "Der technische Durchbruch"), dW = dY^T X, contracted over the tokens:
 *   Y[m][n] = sum_kb a_s[m][kb] * b_s[n][kb] *
 *                    sum_{k in block kb} dec(a_q[m][k]) * dec(b_q[n][k])
 *   a_q [M][K], a_s [M][K/128]   (dY^T: q_t and scales_t of fp8_quant_act_dual
 *                                 of dY; M = output features)
 *   b_q [N][K], b_s [N][K/128]   (X^T: the same of X; N = input features, a
 *                                 multiple of 128)
 *   y   [M][N] bf16 bits (out)   (dW, in the layout of W)
 *   K   tokens rounded up to a multiple of 128 (Mp of fp8_quant_act_dual)
 * fp32 accumulation, one bf16 rounding (nearest even) at the end; the
 * summation order is fixed but unspecified.  The only difference from
 * fp8_blockscaled_gemm is b_s: one scale per row of b and block of K.
 */
fp8q_status fp8_blockscaled_gemm_wgrad(const uint8_t *a_q, const float *a_s,
                                       const uint8_t *b_q, const float *b_s,
                                       uint16_t *y, int64_t M, int64_t N, int64_t K,
                                       void *stream);

/*
 * The same product for scales that are all powers of two (FP8Q_SCALE_POW2
 * quantization; page 1, "Warum dies fuer die KI-Oekonomie wichtig ist"): the
 * matrix cores apply both operands' per-row scales themselves (E8M0), so no
 * per-block rescaling runs on the vector ALUs.  Same precondition and NaN rule
 * as fp8_blockscaled_gemm_pow2: an output that depends on a scale other than
 * 2^e, -127 <= e <= 127, is NaN.
 */
fp8q_status fp8_blockscaled_gemm_wgrad_pow2(const uint8_t *a_q, const float *a_s,
                                            const uint8_t *b_q, const float *b_s,
                                            uint16_t *y, int64_t M, int64_t N, int64_t K,
                                            void *stream);

/*
 * Grouped block-scaled FP8 GEMM for mixture-of-experts layers (the recipe's
 * MoE models on page 1, "Leistungsgewinne in der Praxis" and "Warum dies fuer
 * die KI-Oekonomie wichtig ist"): group g owns rows
 * [group_offsets[g], group_offsets[g+1]) of a_q, a_s and y and multiplies them
 * by its own weight matrix.
 *   a_q [M_total][K], a_s [M_total][K/128]
 *   b_q [G][N][K],    b_s [G][N/128][K/128]
 *   group_offsets [G+1] int32, DEVICE memory: non-decreasing, offsets[0] = 0,
 *                 offsets[G] = M_total.  Empty groups are allowed.  The offsets
 *                 are read on the device (no host synchronisation); values
 *                 outside [0, M_total] are clamped and a decrease is treated as
 *                 an empty group, so a malformed array cannot cause an access
 *                 outside the tensors (rows no group covers are left unwritten).
 *   y   [M_total][N] bf16 bits (out)
 * Per group the arithmetic is that of fp8_blockscaled_gemm.
 */
fp8q_status fp8_grouped_gemm(const uint8_t *a_q, const float *a_s,
                             const uint8_t *b_q, const float *b_s,
                             const int32_t *group_offsets, int32_t G,
                             int64_t M_total, int64_t N, int64_t K,
                             uint16_t *y, void *stream);

/*
 * The same two products for operands whose scales are all powers of two --
 * what fp8_quant_act_1x128 and fp8_quant_weight_128x128 produce in
 * FP8Q_SCALE_POW2 mode (page 1, "Warum dies fuer die KI-Oekonomie wichtig
 * ist": power-of-two scale factors as an option "for additional
 * optimization").  On gfx950 the matrix cores then apply the scales
 * themselves (E8M0 block-scale operands), so no per-block rescaling runs on
 * the vector ALUs.  Arguments, layouts, errors and the result (up to the fp32
 * summation order) are those of fp8_blockscaled_gemm / fp8_grouped_gemm.
 * Precondition: every scale an output depends on is 2^e with -127 <= e <= 127
 * (an E8M0 value); an output that depends on any other scale value is written
 * as NaN instead of a silently different product.  POW2-mode quantization
 * always gives such scales: its exponent is at least -127.
 */
fp8q_status fp8_blockscaled_gemm_pow2(const uint8_t *a_q, const float *a_s,
                                      const uint8_t *b_q, const float *b_s,
                                      uint16_t *y, int64_t M, int64_t N, int64_t K,
                                      void *stream);

fp8q_status fp8_grouped_gemm_pow2(const uint8_t *a_q, const float *a_s,
                                  const uint8_t *b_q, const float *b_s,
                                  const int32_t *group_offsets, int32_t G,
                                  int64_t M_total, int64_t N, int64_t K,
                                  uint16_t *y, void *stream);

/*
 * Grouped GEMM of a mixture-of-experts layer whose activations were quantized
 * before dispatch (page 1, "Leistungsgewinne in der Praxis": the recipe's MoE
 * models; quantizing each token once, ahead of routing, means the FP8 bytes,
 * half the size of bf16, are what gets dispatched).  Routed row r of group g
 * (group_offsets[g] <= r < group_offsets[g+1]) is token row row_index[r] of
 * the quantized token matrix, read directly by the GEMM's loads; no gathered
 * copy of the activations is made:
 *   y[r][n] = sum_kb a_s[i][kb] * b_s[g][n/128][kb] *
 *             sum_{k in block kb} dec(a_q[i][k]) * dec(b_q[g][n][k]),  i = row_index[r]
 *   a_q [T][K] E4M3, a_s [T][K/128] fp32  (fp8_quant_act_1x128 of the T tokens)
 *   b_q, b_s, group_offsets, G, M_total, N, K, y as for fp8_grouped_gemm
 *   row_index [M_total] int32, DEVICE memory.  A row whose index lies outside
 *             [0, T) is written as zeros (no memory outside a_q/a_s is read).
 *   mode  FP8Q_SCALE_AMAX: any finite scales (the arithmetic of
 *         fp8_grouped_gemm); FP8Q_SCALE_POW2: power-of-two scales (that of
 *         fp8_grouped_gemm_pow2, with its NaN rule for other scale values).
 * The result equals fp8_grouped_gemm(_pow2) on the gathered rows a_q[row_index],
 * a_s[row_index] bit for bit.  Requires T*K < 2^31 (byte offsets into a_q are
 * 32-bit); larger token matrices return FP8Q_ESHAPE.  T = 0 with routed rows
 * (M_total > 0, N > 0) returns FP8Q_EINVAL.
 */
fp8q_status fp8_grouped_gemm_gather(const uint8_t *a_q, const float *a_s, int64_t T,
                                    const uint8_t *b_q, const float *b_s,
                                    const int32_t *group_offsets, const int32_t *row_index,
                                    int32_t G, int64_t M_total, int64_t N, int64_t K,
                                    uint16_t *y, int mode, void *stream);

/*
 * The gate+up projection of the experts of a SwiGLU mixture-of-experts layer
 * with the activation and the down projection's 1x128 quantization in its
 * epilogue: fp8_blockscaled_gemm_swiglu_quant per group (the recipe's MoE
 * models, page 1, "Leistungsgewinne in der Praxis" and "Warum dies fuer die
 * KI-Oekonomie wichtig ist"; the separate activation and quantization passes
 * it replaces are the quantization-kernel overhead named in "Leistungsgewinne
 * in der Praxis").  Routed row r of group g (group_offsets[g] <= r <
 * group_offsets[g+1]) is multiplied by expert g's fused gate+up weight, and
 * row r of h is written:
 *   a_q, a_s   row_index != NULL: [T][K], [T][K/128], the tokens quantized
 *              once before dispatch; routed row r reads token row_index[r]
 *              (an index outside [0, T) reads zeros), as in
 *              fp8_grouped_gemm_gather.  row_index == NULL: [M_total][K],
 *              [M_total][K/128], routed row r is row r (T is ignored).
 *   b_q [G][2F][K], b_s [G][2F/128][K/128]  each expert's weight with gate and
 *              up rows in alternating 128-row blocks, the layout of
 *              fp8_blockscaled_gemm_swiglu_quant
 *   group_offsets [G+1] int32, DEVICE memory, as for fp8_grouped_gemm (rows
 *              no group covers are left unwritten)
 *   row_index  [M_total] int32, DEVICE memory, or NULL
 *   h_q [M_total][F] E4M3 bytes (out), h_s [M_total][F/128] fp32 (out)
 *   F  output features per expert, a multiple of 128
 *   mode fp8q_scale_mode of h's blocks; the GEMM applies the operands' scales
 *        as fp8_grouped_gemm does (any finite values)
 * Each row of h equals, bit for bit, what fp8_blockscaled_gemm_swiglu_quant
 * gives for that row with its group's weight.  Errors as for
 * fp8_grouped_gemm_gather (T*K below 2^31 bytes when row_index is given).
 */
fp8q_status fp8_grouped_gemm_swiglu_quant(const uint8_t *a_q, const float *a_s, int64_t T,
                                          const uint8_t *b_q, const float *b_s,
                                          const int32_t *group_offsets, const int32_t *row_index,
                                          int32_t G, int64_t M_total, int64_t F, int64_t K,
                                          uint8_t *h_q, float *h_s, int mode, void *stream);

/*
 * FP8 KV cache (page 1, "Leistungsgewinne in der Praxis": FP8 for the KV cache
 * and attention takes the end-to-end gain to about 48%).  The cache holds
 * every key and value row of one token and one key/value head (head
 * dimension 128) as one 1x128 block: E4M3 bytes plus one fp32 scale, the
 * activation rule of fp8_quant_act_1x128.
 *   k_new, v_new  [B][Hkv][128] bf16 bits (in): the new token's rows
 *   pos           [B] int32, DEVICE memory: token position of each sequence;
 *                 a position outside [0, S) stores nothing
 *   k_cache, v_cache  [B][Hkv][S][128] E4M3 (in/out)
 *   k_scale, v_scale  [B][Hkv][S] fp32 (in/out)
 *   mode          fp8q_scale_mode
 * The stored bytes and scales are exactly fp8_quant_act_1x128 of the rows.
 */
fp8q_status fp8_kv_cache_append(const uint16_t *k_new, const uint16_t *v_new,
                                const int32_t *pos,
                                uint8_t *k_cache, float *k_scale,
                                uint8_t *v_cache, float *v_scale,
                                int32_t B, int32_t Hkv, int64_t S, int mode,
                                void *stream);

/*
 * Append T tokens per sequence to the FP8 KV cache (prefill, chunked prefill;
 * same passage and layout as fp8_kv_cache_append).
 *   k_new, v_new  [B][T][Hkv][128] bf16 bits (in), token-major as the QKV
 *                 projection writes them
 *   start         [B] int32, DEVICE memory: token t of sequence b goes to
 *                 position start[b] + t; positions outside [0, S) store
 *                 nothing
 *   k_cache .. v_scale, mode  as for fp8_kv_cache_append
 * With T = 1 this is fp8_kv_cache_append.  Sizes: B*T*Hkv < 2^34.
 */
fp8q_status fp8_kv_cache_append_tokens(const uint16_t *k_new, const uint16_t *v_new,
                                       const int32_t *start,
                                       uint8_t *k_cache, float *k_scale,
                                       uint8_t *v_cache, float *v_scale,
                                       int32_t B, int32_t T, int32_t Hkv, int64_t S, int mode,
                                       void *stream);

/*
 * FP8 attention for many query tokens (prefill, chunked prefill, a training
 * forward pass) over the FP8 KV cache (same passage), causal: query t of
 * sequence b sits at position p = start[b] + t and
 *   out[b][t][h] = sum_j softmax_j(q[b][t][h] . k[b][g][j] / sqrt(128)) v[b][g][j]
 * over the cached tokens j <= p, j < S, with g = h / (Hq / Hkv); a query with
 * no such token gives zeros.  The queries' own keys and values are in the
 * cache already (fp8_kv_cache_append_tokens first).
 *   q_q [B][T][Hq][128] E4M3, q_s [B][T][Hq] fp32: query rows in 1x128 blocks
 *       (fp8_quant_act_1x128 of the projection's [B*T][Hq*128] output); the
 *       query scales must be positive and finite, as the quantizer makes them
 *   k_cache, k_scale, v_cache, v_scale as for fp8_kv_cache_append
 *   start [B] int32, DEVICE memory
 *   out [B][T][Hq][128] bf16 bits (out)
 * q.k runs on the matrix cores in FP8 (E4M3 x E4M3, fp32 accumulation), the
 * softmax in fp32 (base 2); the weights p_j * v_scale_j are rounded to bf16
 * (relative error at most 2^-8 each) and multiplied with the exactly decoded
 * values on the bf16 matrix cores (fp32 accumulation); out is rounded once to
 * bf16.  Against the exact result the error is at most about
 * 2^-8 (sum_j p_j |v_j| / sum_j p_j + |out|).
 * Any Hq that is a multiple of Hkv.  Sizes: ceil(T/64) * B * Hq < 2^31 and
 * S < 2^31 (FP8Q_ESHAPE otherwise).
 */
fp8q_status fp8_attention_prefill(const uint8_t *q_q, const float *q_s,
                                  const uint8_t *k_cache, const float *k_scale,
                                  const uint8_t *v_cache, const float *v_scale,
                                  const int32_t *start, uint16_t *out,
                                  int32_t B, int32_t T, int32_t Hq, int32_t Hkv, int64_t S,
                                  void *stream);

/*
 * FP8 decode attention over the FP8 KV cache (same passage): one query token
 * per sequence,
 *   out[b][h] = sum_t softmax_t(q[b][h] . k[b][g][t] / sqrt(128)) * v[b][g][t]
 * over t < min(seq_len[b], S), with g = h / (Hq / Hkv) (grouped query heads)
 * and q, k, v the dequantized rows.
 *   q_q [B][Hq][128] E4M3, q_s [B][Hq] fp32: the query rows in 1x128 blocks
 *       (fp8_quant_act_1x128 of q viewed as [B*Hq][128])
 *   k_cache, k_scale, v_cache, v_scale as for fp8_kv_cache_append
 *   seq_len [B] int32, DEVICE memory (values outside [0, S] are clamped; a
 *       sequence with no tokens gives zeros)
 *   out [B][Hq][128] bf16 bits (out)
 *   Hq / Hkv must be 1, 2, 4 or 8 (FP8Q_ESHAPE otherwise).
 *   workspace, workspace_bytes: see fp8_attention_decode_workspace_size
 * q.k runs on the matrix cores in FP8 (E4M3 x E4M3, fp32 accumulation); the
 * softmax and the weighted sum of values run in fp32 on exactly decoded
 * values; out is rounded once to bf16.  Results agree with the exact value
 * to within fp32 arithmetic and that rounding.
 * Sizes: B * Hkv < 2^24 (FP8Q_ESHAPE otherwise).
 */
fp8q_status fp8_attention_decode(const uint8_t *q_q, const float *q_s,
                                 const uint8_t *k_cache, const float *k_scale,
                                 const uint8_t *v_cache, const float *v_scale,
                                 const int32_t *seq_len, uint16_t *out,
                                 int32_t B, int32_t Hq, int32_t Hkv, int64_t S,
                                 void *workspace, int64_t workspace_bytes,
                                 void *stream);

/* Bytes of DEVICE workspace fp8_attention_decode needs to split sequences
 * into chunks that run in parallel when B*Hkv (sequence, head) pairs are too
 * few to fill the GPU (fewer than 512); 0 when no split is needed or for
 * invalid sizes.  A function of the sizes only.  With workspace == NULL the
 * call still works: one workgroup then covers a whole sequence.  A workspace
 * smaller than this size is FP8Q_EINVAL.  Its contents need no
 * initialisation; concurrent calls need their own. */
int64_t fp8_attention_decode_workspace_size(int32_t B, int32_t Hq, int32_t Hkv, int64_t S);

/*
 * MoE dispatch order on the device (the recipe's mixture-of-experts models:
 * page 1, "Leistungsgewinne in der Praxis" (Qwen3-30B) and "Warum dies fuer
 * die KI-Oekonomie wichtig ist" (Moonlight 16B)): from the routing table to
 * the group offsets and row map that fp8_grouped_gemm and
 * fp8_grouped_gemm_gather take, with no host synchronisation.
 *   expert_ids [T][k] int32 (in): expert of slot j of token t, entry t*k + j
 *   E          routed experts, 1 <= E <= 1024; n_shared >= 0 shared experts
 *   group_offsets [E+n_shared+1] int32 (out): first row of each group
 *   row_index  [T*(k+n_shared)] int32 (out): the token of every row
 *   entry_row  [T*k] int32 (out, may be NULL): the row of every entry
 *   workspace, workspace_bytes: DEVICE memory of at least
 *              fp8_moe_permute_workspace_size(T, k, E) bytes; its contents
 *              need no initialisation; concurrent calls need their own.
 * Rows: the entries sorted by expert, stable in entry order (so inside an
 * expert by token, then slot), group e = rows [offsets[e], offsets[e+1]);
 * then each shared expert as a group of all T tokens in order.  An id outside
 * [0, E) puts its entry in no group (entry_row -1); those entries leave the
 * last rows of row_index, after offsets[E+n_shared], holding -1.  With valid
 * ids offsets[E+n_shared] = T*(k+n_shared).  The result is deterministic and
 * equals the stable sort exactly.  T*(k+n_shared) < 2^31.
 */
fp8q_status fp8_moe_permute(const int32_t *expert_ids, int64_t T, int32_t k, int32_t E, int32_t n_shared,
                            int32_t *group_offsets, int32_t *row_index, int32_t *entry_row,
                            void *workspace, int64_t workspace_bytes, void *stream);

/* Bytes of workspace fp8_moe_permute needs (a function of the sizes only; 0
 * for invalid sizes). */
int64_t fp8_moe_permute_workspace_size(int64_t T, int32_t k, int32_t E);

/*
 * For callers that cannot allocate (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): fp8_attention_decode
 * without the workspace argument.  Same arguments otherwise, same results bit
 * for bit as fp8_attention_decode with a workspace of
 * fp8_attention_decode_workspace_size() bytes.
 *   The chunked path's workspace is a static device array of
 *   FP8Q_NOALLOC_SCRATCH_BYTES inside the library, one per GPU, held until the
 *   process ends.  That size covers every (B, Hq, Hkv, S) the call accepts
 *   (FP8Q_ESHAPE otherwise).  The call allocates nothing and calls no
 *   allocating routine.  Every call on one GPU shares that GPU's array and
 *   needs none of its contents: calls that overlap on one GPU (several
 *   streams, or host threads, at once) race and must not be issued.
 */
#define FP8Q_NOALLOC_SCRATCH_BYTES 4251520
fp8q_status fp8_attention_decode_noalloc(const uint8_t *q_q, const float *q_s,
                                         const uint8_t *k_cache, const float *k_scale,
                                         const uint8_t *v_cache, const float *v_scale,
                                         const int32_t *seq_len, uint16_t *out,
                                         int32_t B, int32_t Hq, int32_t Hkv, int64_t S,
                                         void *stream);

/* Informational: the tile plan of an M x N dense GEMM output.  The tiles of
 * token rows [0, R) and 256-row weight panels [0, P) run as 256-token x 256
 * tiles, every other tile as a 128-token x 256 tile.  Returns P and, when
 * rows_large is not NULL, stores R there: R = M and P = ceil(N/256) for all
 * large tiles, R = 0 and P = 0 for all small ones, R = M with a smaller P for a
 * split by weight panels, R < M with all panels for a split by token rows.
 * swiglu = 0 for fp8_blockscaled_gemm and its pow2, weight-gradient and
 * quantized-output variants (their output may be split), 1 for
 * fp8_blockscaled_gemm_swiglu_quant (one tile height).  -1 for invalid sizes.
 * No device access. */
int32_t fp8_blockscaled_gemm_tile_plan(int64_t M, int64_t N, int swiglu, int64_t *rows_large);

/* Static English text of a status code (never NULL). */
const char *fp8q_status_string(int status);

/* Message of the last failing call on the calling thread ("" if none).  The
 * pointer stays valid until the next call of this library on the thread. */
const char *fp8q_last_error(void);

/* FP8Q_ABI_VERSION of the built library. */
int fp8q_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP8Q_H */
