/*
 * fp8q_oracle.c -- plain, slow, obviously correct CPU reference for the
 * blockwise-scaled FP8 linear layer (E4M3 codes, 1x128 activation blocks,
 * 128x128 weight blocks, block-scaled GEMM).
 *
 * TEST INFRASTRUCTURE, NOT PRODUCT CODE.  Only the test suite, the package's
 * smoke check and the CPU-baseline leg of the benchmark may load this file's
 * library.  It shares no code, header, table or constant with the HIP path and
 * includes nothing from it.
 *
 * Sources (the pages, cited by title and section):
 *  [P1-D]  "NVIDIA NeMo RL erreicht 48% Geschwindigkeitssteigerung mit
 *          End-to-End FP8-Praezisionstraining", section "Der technische
 *          Durchbruch": FP8 in the E4M3 format, blocks of 128x128 for weights
 *          and 1x128 for activations; linear layers run in FP8.
 *  [P1-L]  same page, section "Leistungsgewinne in der Praxis": the
 *          quantization scales are recalibrated dynamically after every
 *          training step.
 *  [P1-O]  same page, section "Warum dies fuer die KI-Oekonomie wichtig ist":
 *          scaling factors may be restricted to powers of two.
 *  [P2-P]  "FP8 Trainingsinfrastructuur: Numerieke Precisie van de Volgende
 *          Generatie", section "Het landschap van numerieke precisie": E4M3
 *          has 4 exponent and 3 mantissa bits and reaches +-448.
 *
 * Readings where the pages leave a step open (each one is listed with its
 * reason in the design notes):
 *  - E4M3 is the variant whose largest finite value is 448: exponent bias 7,
 *    subnormals m*2^-9, only S.1111.111 is NaN, no infinities.
 *  - conversion to E4M3 rounds to nearest, ties to an even mantissa, and
 *    saturates to +-448; the sign of a zero result is kept.
 *  - the stored scale s is the fp32 dequantisation multiplier (x ~ q*s):
 *    s = RN_fp32(amax/448) ("amax" mode) or the smallest power of two with
 *    448*s >= amax ("pow2" mode); an all-zero block has s = 1.
 *  - each element is divided by s with one correctly rounded fp32 division
 *    and the fp32 quotient is then converted to E4M3.
 *  - the GEMM is Y = X * W^T; it sums the dequantised products in fp64.
 *
 * Build: gcc -O2 -std=c11 -fPIC -shared -fopenmp -ffp-contract=off (no
 * fast-math, no flush-to-zero).  OpenMP only spreads independent blocks or
 * output elements over threads; the arithmetic of each one is unchanged.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define ORACLE_MODE_AMAX 0
#define ORACLE_MODE_POW2 1
#define BLK 128

/* ------------------------------------------------------------------------ */
/* E4M3 code <-> value                                                       */
/* ------------------------------------------------------------------------ */

/* Value of one E4M3 byte, from its bit fields [P2-P]: sign, 4-bit exponent
 * with bias 7, 3-bit mantissa.  Exponent field 0 holds the subnormals
 * m * 2^-9; S.1111.111 is NaN. */
double oracle_e4m3_decode(uint8_t c)
{
    int sign = c >> 7;
    int e = (c >> 3) & 0xF;
    int m = c & 0x7;
    double mag;
    if (e == 0xF && m == 0x7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return sign ? -mag : mag;
}

void oracle_e4m3_decode_table(double *out256)
{
    for (int c = 0; c < 256; c++)
        out256[c] = oracle_e4m3_decode((uint8_t)c);
}

/* Round a non-negative double to an integer, ties to the even integer. */
static double round_half_even(double n)
{
    double fl = floor(n);
    double frac = n - fl; /* exact */
    if (frac > 0.5)
        return fl + 1.0;
    if (frac < 0.5)
        return fl;
    return (fmod(fl, 2.0) == 0.0) ? fl : fl + 1.0;
}

/* fp32 -> E4M3 byte: nearest grid value, ties to even mantissa, saturating
 * at +-448; the sign of zero is kept.  Input must not be NaN. */
uint8_t oracle_e4m3_encode(float r)
{
    uint8_t sign = signbit(r) ? 0x80 : 0x00;
    double a = fabs((double)r);
    double quantum, k, v, f;
    int E;

    if (a >= 448.0)
        return sign | 0x7E;

    /* spacing of the E4M3 grid near a: 2^-9 below 2^-6 (subnormals),
     * otherwise 2^(e-3) inside the binade [2^e, 2^(e+1)). */
    if (a < ldexp(1.0, -6)) {
        quantum = ldexp(1.0, -9);
    } else {
        frexp(a, &E); /* a in [2^(E-1), 2^E) */
        quantum = ldexp(1.0, (E - 1) - 3);
    }
    k = round_half_even(a / quantum); /* a/quantum is exact */
    v = k * quantum;                  /* nearest grid value, <= 448 */

    if (v == 0.0)
        return sign;
    if (v < ldexp(1.0, -6))
        return sign | (uint8_t)k; /* subnormal code: mantissa = k */
    f = frexp(v, &E);             /* v = (2f) * 2^(E-1), 2f in [1,2) */
    {
        int ebits = (E - 1) + 7;
        int mbits = (int)((2.0 * f - 1.0) * 8.0); /* exact */
        return sign | (uint8_t)((ebits << 3) | mbits);
    }
}

void oracle_e4m3_encode_array(const float *r, int64_t n, uint8_t *q)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < n; i++)
        q[i] = oracle_e4m3_encode(r[i]);
}

/* ------------------------------------------------------------------------ */
/* Block scale                                                               */
/* ------------------------------------------------------------------------ */

/* Scale of a block with largest magnitude amax (>= 0, finite).
 *  amax mode: s = amax / 448 in fp32, correctly rounded (IEEE division).
 *  pow2 mode [P1-O]: s = 2^e with e the smallest integer such that
 *             448 * 2^e >= amax, decided by exact comparison, but not below
 *             -127: a power-of-two scale is an E8M0 value (2^-127 .. 2^127).
 *             For amax <= 448 * 2^-127 the scale is 2^-127, which still
 *             satisfies 448 * s >= amax, so nothing saturates.
 *  amax == 0: s = 1. */
float oracle_block_scale(float amax, int mode)
{
    int e;
    if (amax == 0.0f)
        return 1.0f;
    if (mode == ORACLE_MODE_AMAX)
        return amax / 448.0f;
    frexp((double)amax, &e); /* a first guess; the loops settle it */
    e -= 9;
    while (ldexp(448.0, e) < (double)amax)
        e++;
    while (ldexp(448.0, e - 1) >= (double)amax)
        e--;
    if (e < -127)
        e = -127;
    return (float)ldexp(1.0, e);
}

/* ------------------------------------------------------------------------ */
/* Quantizers                                                                */
/* ------------------------------------------------------------------------ */

static float bf16_bits_to_float(uint16_t b)
{
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Activation quantization [P1-D], [P1-L]: every row of X[M][K] (bf16 bits,
 * row-major, K a multiple of 128) is cut into blocks of 128 consecutive
 * elements; each block gets its own scale.
 * Outputs: q[M][K] E4M3 bytes, s[M][K/128] fp32 scales, both row-major. */
void oracle_quant_act_1x128(const uint16_t *x, int64_t M, int64_t K, int mode,
                            uint8_t *q, float *s)
{
    int64_t KB = K / BLK;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; m++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            const uint16_t *blk = x + m * K + kb * BLK;
            uint8_t *qb = q + m * K + kb * BLK;
            float amax = 0.0f, sc;
            for (int i = 0; i < BLK; i++) {
                float a = fabsf(bf16_bits_to_float(blk[i]));
                if (a > amax)
                    amax = a;
            }
            sc = oracle_block_scale(amax, mode);
            s[m * KB + kb] = sc;
            for (int i = 0; i < BLK; i++)
                qb[i] = oracle_e4m3_encode(bf16_bits_to_float(blk[i]) / sc);
        }
    }
}

/* Weight quantization [P1-D], [P1-L], [P1-O]: W[N][K] (bf16 bits, row-major,
 * N and K multiples of 128) is cut into 128x128 tiles aligned at (0,0); each
 * tile gets one scale.  Outputs: q[N][K] bytes, s[N/128][K/128] scales. */
void oracle_quant_weight_128x128(const uint16_t *w, int64_t N, int64_t K,
                                 int mode, uint8_t *q, float *s)
{
    int64_t NB = N / BLK, KB = K / BLK;
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t nb = 0; nb < NB; nb++) {
        for (int64_t kb = 0; kb < KB; kb++) {
            float amax = 0.0f, sc;
            for (int64_t i = 0; i < BLK; i++)
                for (int64_t j = 0; j < BLK; j++) {
                    float a = fabsf(bf16_bits_to_float(
                        w[(nb * BLK + i) * K + kb * BLK + j]));
                    if (a > amax)
                        amax = a;
                }
            sc = oracle_block_scale(amax, mode);
            s[nb * KB + kb] = sc;
            for (int64_t i = 0; i < BLK; i++)
                for (int64_t j = 0; j < BLK; j++) {
                    int64_t idx = (nb * BLK + i) * K + kb * BLK + j;
                    q[idx] = oracle_e4m3_encode(bf16_bits_to_float(w[idx]) / sc);
                }
        }
    }
}

/* ------------------------------------------------------------------------ */
/* Block-scaled GEMM, fp64 accumulation                                      */
/* ------------------------------------------------------------------------ */

/* One output element of Y = X * W^T with dequantised operands:
 *   Y[m][n] = sum_k (dec(aq[m][k]) * as[m][k/128]) * (dec(bq[n][k]) * bs[n/128][k/128])
 * summed in fp64 in increasing k. */
static double gemm_element(const double *dec, const uint8_t *aq, const float *as,
                           const uint8_t *bq, const float *bs, int64_t m,
                           int64_t n, int64_t K)
{
    int64_t KB = K / BLK;
    double acc = 0.0;
    for (int64_t k = 0; k < K; k++) {
        double a = dec[aq[m * K + k]] * (double)as[m * KB + k / BLK];
        double b = dec[bq[n * K + k]] * (double)bs[(n / BLK) * KB + k / BLK];
        acc += a * b;
    }
    return acc;
}

/* Full product.  aq[M][K], as[M][K/128], bq[N][K], bs[N/128][K/128];
 * y[M][N] fp64, row-major. */
void oracle_gemm_f64(const uint8_t *aq, const float *as, const uint8_t *bq,
                     const float *bs, int64_t M, int64_t N, int64_t K, double *y)
{
    double dec[256];
    oracle_e4m3_decode_table(dec);
#pragma omp parallel for collapse(2) schedule(static)
    for (int64_t m = 0; m < M; m++)
        for (int64_t n = 0; n < N; n++)
            y[m * N + n] = gemm_element(dec, aq, as, bq, bs, m, n, K);
}

/* Selected elements only: y[i] = Y[ms[i]][ns[i]] for i < count. */
void oracle_gemm_sampled_f64(const uint8_t *aq, const float *as,
                             const uint8_t *bq, const float *bs, int64_t M,
                             int64_t N, int64_t K, const int64_t *ms,
                             const int64_t *ns, int64_t count, double *y)
{
    double dec[256];
    (void)M;
    (void)N;
    oracle_e4m3_decode_table(dec);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++)
        y[i] = gemm_element(dec, aq, as, bq, bs, ms[i], ns[i], K);
}

/* Grouped product for mixture-of-experts layers: group g owns rows
 * [off[g], off[g+1]) of aq/as/y and uses weights bq + g*N*K and scales
 * bs + g*(N/128)*(K/128).  off (host) is non-decreasing with off[0] = 0,
 * off[G] = M_total. */
void oracle_grouped_gemm_f64(const uint8_t *aq, const float *as,
                             const uint8_t *bq, const float *bs,
                             const int32_t *off, int32_t G, int64_t M_total,
                             int64_t N, int64_t K, double *y)
{
    double dec[256];
    int64_t KB = K / BLK;
    (void)M_total;
    oracle_e4m3_decode_table(dec);
    for (int32_t g = 0; g < G; g++) {
        const uint8_t *bqg = bq + (int64_t)g * N * K;
        const float *bsg = bs + (int64_t)g * (N / BLK) * KB;
        int64_t r0 = off[g], r1 = off[g + 1];
#pragma omp parallel for collapse(2) schedule(static)
        for (int64_t m = r0; m < r1; m++)
            for (int64_t n = 0; n < N; n++)
                y[m * N + n] = gemm_element(dec, aq, as, bqg, bsg, m, n, K);
    }
}

/* Selected elements of the grouped product; grp[i] is the group of row ms[i]. */
void oracle_grouped_gemm_sampled_f64(const uint8_t *aq, const float *as,
                                     const uint8_t *bq, const float *bs,
                                     int64_t N, int64_t K, const int32_t *grp,
                                     const int64_t *ms, const int64_t *ns,
                                     int64_t count, double *y)
{
    double dec[256];
    int64_t KB = K / BLK;
    oracle_e4m3_decode_table(dec);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < count; i++) {
        const uint8_t *bqg = bq + (int64_t)grp[i] * N * K;
        const float *bsg = bs + (int64_t)grp[i] * (N / BLK) * KB;
        y[i] = gemm_element(dec, aq, as, bqg, bsg, ms[i], ns[i], K);
    }
}

/* Number of OpenMP threads a parallel region of this library uses. */
int oracle_num_threads(void)
{
    int n = 1;
#pragma omp parallel
    {
#pragma omp single
        {
#ifdef _OPENMP
            n = omp_get_num_threads();
#endif
        }
    }
    return n;
}

/* Threads for the following parallel regions of this library (the CPU
 * baseline's single-thread run); n < 1 restores the default. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    static int dflt = 0;
    if (dflt == 0)
        dflt = omp_get_max_threads();
    omp_set_num_threads(n >= 1 ? n : dflt);
#else
    (void)n;
#endif
}
