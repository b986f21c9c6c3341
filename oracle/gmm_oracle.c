/*
 * CPU oracle for the MoE grouped matrix multiply (GMM) -- TEST INFRASTRUCTURE.
 *
 * Only the test suite, the smoke check and the benchmark's CPU-baseline leg
 * may load this file's library.  The product path (the HIP library) never
 * calls it, and the two share no code: this file has its own FP8 codec, its
 * own quantiser and its own fp64 reference loops.
 *
 * Everything here is the plain definition, written out without blocking,
 * fusion or reordering beyond what the definition states.  Sources:
 *
 *  [Q2]  "GEMM Kernel 性能优化十问" (Ten questions on GEMM kernel
 *        optimisation), Q2: activations (LHS) get one scale per row per 128
 *        K-elements (1x128), weights (RHS) one scale per 128x128 block.
 *  [Q3]  same page, Q3: the K-tile holds several 128-wide quantisation
 *        blocks (subchannels); each block's partial product is scaled and
 *        accumulated separately.
 *  [Q4]  same page, Q4: tgmm computes dW[K,N] += X^T[K,M] x dY[M,N] (the
 *        reduction runs over M).
 *  [Q5]  same page, Q5: the backward pass is unquantised bf16.
 *  [V2q] "实现差距：GMM Kernel（V1 vs V2）" (Implementation gap: GMM kernel
 *        V1 vs V2), section 3.3: per-block abs-max, scale = absmax/dtype_max,
 *        inverse = 0 where scale == 0 else 1/scale, codes = (x * inverse)
 *        cast to the FP8 type, block product rescaled by the LHS scale and
 *        the RHS scale, then accumulated.
 *  [V1s] same page, section 2.1: subchannel loop, one dot per quant block,
 *        scaled, then added to the accumulator.
 *  [V2z] same page, section 3.6: output rows past the last group are zero.
 *  [V2a] same page, sections 3.5 and 4.2: the gate and up projections are
 *        one GMM against weights concatenated along N (gate columns first,
 *        then up), and the kernel returns silu(gate) * up.
 *  [GG]  "MoE 优化的探索：从 MiniMax-01、Comet、FlashMoE 到 DeepSeek-V4",
 *        section 3.7.2: a grouped GEMM is one independent GEMM per expert,
 *        X_e W_e, over that expert's contiguous rows.
 *  [V2s] "实现差距：GMM Kernel（V1 vs V2）", sections 3.4 and 4.1: V2 takes
 *        RHS weights in sub-byte types (int4, float4_e2m1fn) and unpacks
 *        them in the kernel; MXFP4 weights are the high-priority case.
 *  [MX]  OCP Microscaling Formats (MX) specification v1.0: an MXFP4 block
 *        is 32 E2M1 elements (sign, 2 exponent bits with bias 1, 1 mantissa
 *        bit; values 0, 0.5, 1, 1.5, 2, 3, 4, 6) sharing one E8M0 scale
 *        2^(e-127); a block V is converted with shared exponent
 *        floor(log2(max|V|)) - 2 (2 = the largest E2M1 exponent) and each
 *        element rounded to E2M1, clamped to +-6.
 *
 * Readings where the pages are silent (the same list is kept with the
 * design notes):
 *  - FP8 format is OCP E4M3 ("fn"): bias 7, max 448, 0x7F/0xFF NaN, no inf.
 *  - Encoding rounds to nearest, ties to even, saturates finite values
 *    beyond 464 to +-448, and keeps the sign of zero (0x80).
 *  - The quantiser's three operations (a/448, 1/s, x*inv) are single IEEE
 *    fp32 operations, correctly rounded; no fused multiply-add.  This file
 *    must be compiled with -ffp-contract=off and without fast-math.
 *  - Dequantise-and-accumulate is fp64.  The per-block inner sum of FP8
 *    products is exact in fp64 (each product has at most 8 significant bits
 *    and 128 of them need at most 43 bits).
 *  - A block with a non-zero abs-max below 2^-100 is outside the contract
 *    (its inverse scale may overflow fp32); such inputs are not tested.
 *  - MXFP4 weights ([V2s], [MX]): blocks of 32 run along K (the reduction
 *    index) for each expert and column; the LHS keeps the FP8 1x128 recipe,
 *    so a forward block product is the 1x128 LHS block against four MXFP4
 *    blocks.  E2M1 rounding is to nearest, ties to the even mantissa, the
 *    sign of zero is kept (code 8), the shared exponent is clamped to
 *    [-127, 127], and an all-zero block gets E8M0 code 0 with zero codes.
 *    The division by the power-of-two scale is exact (done in fp64).  The
 *    per-block inner sum is exact in fp64 here too (each product has at
 *    most 6 significant bits and the exponents of 128 of them span far
 *    fewer than 53 - 6 - 7 binades for any finite scaled input).
 *  - int4 weights ([V2s] names the type, nothing more): codes are signed
 *    4-bit integers in [-8, 7] with the FP8 path's 128x128 RHS blocks and
 *    fp32 block scales [Q2]; the quantiser is [V2q]'s recipe with the int4
 *    maximum 7 in place of 448: s = a/7, inv = (s == 0 ? 0 : 1/s), code =
 *    round-half-even(w*inv) clamped to [-8, 7] (|w*inv| <= 7 for this
 *    quantiser, so its codes are the symmetric [-7, 7]; -8 can only come
 *    from another quantiser).  The LHS keeps the FP8 1x128 recipe.  The
 *    per-block inner sum is exact in fp64 (integer codes times e4m3 values).
 *
 * Parity pins: every function here is checked in tests/test_oracle_*.py
 * against something other than itself (torch's float8_e4m3fn cast, numpy
 * fp32/fp64 arithmetic, exact rational arithmetic, closed forms and
 * invariants).  No function is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>
#include <string.h>
#include <stdlib.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#if defined(__FAST_MATH__)
#error "the oracle must not be compiled with fast-math"
#endif

#define QBLOCK 128
#define E4M3_MAX 448.0f

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ---------------------------------------------------------------- codec -- */

/* Value of an OCP E4M3 code: normal (8+m)*2^(e-10), subnormal m*2^-9. */
double oracle_e4m3_decode(uint8_t code)
{
    int sign = code >> 7;
    int e = (code >> 3) & 0xF;
    int m = code & 0x7;
    double v;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);
    else
        v = ldexp((double)(8 + m), e - 10);
    return sign ? -v : v;
}

/* Round an fp32 value to the nearest E4M3 value (ties to even), saturating
 * finite magnitudes above the representable range to 448.  NaN -> 0x7F. */
uint8_t oracle_e4m3_encode(float x)
{
    uint8_t sign;
    double a, quantum, r, v;
    int ex;
    if (isnan(x))
        return 0x7F;
    sign = signbit(x) ? 0x80 : 0x00;
    a = fabs((double)x);
    if (a > 464.0) /* beyond the midpoint between 448 and the (absent) 480 */
        return sign | 0x7E;
    /* grid spacing of E4M3 around a: subnormal range below 2^-6 */
    if (a < ldexp(1.0, -6)) {
        quantum = ldexp(1.0, -9);
    } else {
        frexp(a, &ex); /* a = f*2^ex, f in [0.5,1) -> floor(log2 a) = ex-1 */
        quantum = ldexp(1.0, ex - 1 - 3);
    }
    r = nearbyint(a / quantum); /* a/quantum is exact; default mode is RNE */
    v = r * quantum;            /* exact */
    if (v == 0.0)
        return sign;
    if (v > 448.0) /* only reachable for a in (448, 464]; RNE gives 448 */
        v = 448.0;
    if (v < ldexp(1.0, -6)) /* subnormal code */
        return sign | (uint8_t)(v / ldexp(1.0, -9));
    frexp(v, &ex);
    {
        int E = ex - 1;                      /* v = (1+m/8) * 2^E */
        int mant = (int)(v / ldexp(1.0, E - 3)) - 8;
        return sign | (uint8_t)(((E + 7) << 3) | mant);
    }
}

void oracle_e4m3_encode_array(const float *x, int64_t n, uint8_t *out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        out[i] = oracle_e4m3_encode(x[i]);
}

/* --------------------------------------------------------- quantisation -- */

/* One quantisation block per [V2q]/[Q2]: abs-max over the block's values,
 * s = a/448, inv = (s == 0 ? 0 : 1/s), code = e4m3(x*inv).  `vals` holds
 * the block's n values (already exact fp32), the codes go to `codes`. */
/* The block scale and its guarded inverse ([V2q]): s = a/448, inv = (s == 0
 * ? 0 : 1/s), each one IEEE fp32 division. */
static void scale_pair(float a, float *s, float *inv)
{
    *s = a / E4M3_MAX;
    *inv = (*s == 0.0f) ? 0.0f : 1.0f / *s;
}

/* scale_pair over n block abs-maxima (the step on its own, for checking a
 * quantiser's scale arithmetic on every input it may see). */
void oracle_quant_scales(const float *amax, int64_t n, float *scale, float *inv)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i)
        scale_pair(amax[i], scale + i, inv + i);
}

static float quantize_block(const float *vals, int n, uint8_t *codes)
{
    float a = 0.0f, s, inv;
    int i;
    for (i = 0; i < n; ++i) {
        float v = fabsf(vals[i]);
        if (v > a)
            a = v;
    }
    scale_pair(a, &s, &inv);
    for (i = 0; i < n; ++i) {
        float y = vals[i] * inv;
        codes[i] = oracle_e4m3_encode(y);
    }
    return s;
}

/* LHS 1x128 quantisation [Q2], [V2q].
 * x: [M,K] row-major fp32 (bf16 inputs are passed widened, which is exact).
 * q: [M,K] E4M3 codes; scale: [M,K/128] fp32.  K % 128 == 0. */
void oracle_quantize_lhs(const float *x, int64_t M, int64_t K, uint8_t *q,
                         float *scale)
{
    int64_t m;
    int64_t nb = K / QBLOCK;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t b;
        for (b = 0; b < nb; ++b)
            scale[m * nb + b] = quantize_block(x + m * K + b * QBLOCK, QBLOCK,
                                               q + m * K + b * QBLOCK);
    }
}

/* RHS 128x128 quantisation [Q2]: one scale per (g, k-block, n-block).
 * w: [G,K,N] row-major fp32; q: [G,K,N] codes (same layout as w);
 * scale: [G,K/128,N/128].  K % 128 == 0 and N % 128 == 0. */
void oracle_quantize_rhs(const float *w, int64_t G, int64_t K, int64_t N,
                         uint8_t *q, float *scale)
{
    int64_t kb_n = K / QBLOCK, nb_n = N / QBLOCK;
    int64_t t, total = G * kb_n * nb_n;
#pragma omp parallel for schedule(static)
    for (t = 0; t < total; ++t) {
        int64_t g = t / (kb_n * nb_n);
        int64_t kb = (t / nb_n) % kb_n;
        int64_t nb = t % nb_n;
        float *vals = (float *)malloc(sizeof(float) * QBLOCK * QBLOCK);
        uint8_t *codes = (uint8_t *)malloc(QBLOCK * QBLOCK);
        int64_t i, j;
        for (i = 0; i < QBLOCK; ++i)
            for (j = 0; j < QBLOCK; ++j)
                vals[i * QBLOCK + j] =
                    w[(g * K + kb * QBLOCK + i) * N + nb * QBLOCK + j];
        scale[t] = quantize_block(vals, QBLOCK * QBLOCK, codes);
        for (i = 0; i < QBLOCK; ++i)
            for (j = 0; j < QBLOCK; ++j)
                q[(g * K + kb * QBLOCK + i) * N + nb * QBLOCK + j] =
                    codes[i * QBLOCK + j];
        free(vals);
        free(codes);
    }
}

/* ------------------------------------------------------- group metadata -- */

/* Exclusive prefix sum of group sizes, offsets[G+1].  Returns 0 when every
 * size is non-negative and the total fits in M, else -1. */
int oracle_group_offsets(const int32_t *group_sizes, int64_t G, int64_t M,
                         int64_t *offsets)
{
    int64_t g;
    offsets[0] = 0;
    for (g = 0; g < G; ++g) {
        if (group_sizes[g] < 0)
            return -1;
        offsets[g + 1] = offsets[g] + group_sizes[g];
    }
    return offsets[G] <= M ? 0 : -1;
}

/* Work list of the grouped GEMM ([GG]: every tile belongs to one expert;
 * [V2z]: rows past the last group are zeroed).  Row tiles of height tm are
 * aligned to absolute row indices.  For every group g whose rows
 * [lo_g, hi_g) are non-empty, in group order, and every tile t that
 * intersects them, one entry (g, t, max(lo_g, t*tm), min(hi_g, (t+1)*tm)).
 * Then one entry per tile that holds rows >= total: (G, t, max(total, t*tm),
 * min(M, (t+1)*tm)).  Inside the contract (sizes >= 0 summing to at most M)
 * lo_g = o_g and hi_g = o_g + s_g.  Outside it the library's reading is
 * taken: a negative size counts as 0, o_g sums the sizes so read, and every
 * range is cut at M: lo_g = min(o_g, M), hi_g = min(o_g + s_g, M),
 * total = min(sum, M).
 * work: [cap][4] int32; returns the entry count (or -1 on overflow). */
int64_t oracle_work_list(const int32_t *group_sizes, int64_t G, int64_t M,
                         int64_t tm, int32_t *work, int64_t cap)
{
    int64_t n = 0, g, o = 0, t, total;
    for (g = 0; g < G; ++g) {
        int64_t s = group_sizes[g] > 0 ? group_sizes[g] : 0;
        int64_t glo = o < M ? o : M;
        int64_t ghi = o + s < M ? o + s : M;
        for (t = glo / tm; glo < ghi && t * tm < ghi; ++t) {
            int64_t lo = glo > t * tm ? glo : t * tm;
            int64_t hi = ghi < (t + 1) * tm ? ghi : (t + 1) * tm;
            if (n >= cap)
                return -1;
            work[4 * n + 0] = (int32_t)g;
            work[4 * n + 1] = (int32_t)t;
            work[4 * n + 2] = (int32_t)lo;
            work[4 * n + 3] = (int32_t)hi;
            ++n;
        }
        o += s;
    }
    total = o < M ? o : M;
    for (t = total / tm; t * tm < M; ++t) {
        int64_t lo = total > t * tm ? total : t * tm;
        int64_t hi = M < (t + 1) * tm ? M : (t + 1) * tm;
        if (lo >= hi)
            continue;
        if (n >= cap)
            return -1;
        work[4 * n + 0] = (int32_t)G;
        work[4 * n + 1] = (int32_t)t;
        work[4 * n + 2] = (int32_t)lo;
        work[4 * n + 3] = (int32_t)hi;
        ++n;
    }
    return n;
}

/* Group of each row (G for rows past the total). */
static void row_groups(const int32_t *group_sizes, int64_t G, int64_t M,
                       int32_t *gid)
{
    int64_t g, m = 0, r;
    for (g = 0; g < G; ++g)
        for (r = 0; r < group_sizes[g]; ++r)
            gid[m++] = (int32_t)g;
    while (m < M)
        gid[m++] = (int32_t)G;
}

/* --------------------------------------------------------- FP8 forward -- */

/* out[m,n] = sum_b ( sum_{k in block b} dec(ql[m,k]) dec(qr[g,k,n]) )
 *                   * scale_l[m,b] * scale_r[g,b,n/128]
 * for m in group g ([Q3], [V1s], [V2q], [GG]); rows past the total are 0
 * ([V2z]).  ql: [M,K] codes, sl: [M,K/128], qr: [G,K,N] codes,
 * sr: [G,K/128,N/128]; out: [M,N] fp64. */
void oracle_gmm_fp8(const uint8_t *ql, const float *sl, const uint8_t *qr,
                    const float *sr, const int32_t *group_sizes, int64_t M,
                    int64_t K, int64_t N, int64_t G, double *out)
{
    int64_t nkb = K / QBLOCK, nnb = N / QBLOCK, m;
    int32_t *gid = (int32_t *)malloc(sizeof(int32_t) * (M > 0 ? M : 1));
    double lut[256];
    int c;
    for (c = 0; c < 256; ++c)
        lut[c] = oracle_e4m3_decode((uint8_t)c);
    row_groups(group_sizes, G, M, gid);
#pragma omp parallel
    {
        double *part = (double *)malloc(sizeof(double) * N);
        double *lrow = (double *)malloc(sizeof(double) * QBLOCK);
#pragma omp for schedule(dynamic, 4)
        for (m = 0; m < M; ++m) {
            int64_t g = gid[m], b, k, n;
            double *o = out + m * N;
            for (n = 0; n < N; ++n)
                o[n] = 0.0;
            if (g >= G)
                continue;
            for (b = 0; b < nkb; ++b) {
                const uint8_t *wq = qr + (g * K + b * QBLOCK) * N;
                double s_l = (double)sl[m * nkb + b];
                for (n = 0; n < N; ++n)
                    part[n] = 0.0;
                for (k = 0; k < QBLOCK; ++k)
                    lrow[k] = lut[ql[m * K + b * QBLOCK + k]];
                for (k = 0; k < QBLOCK; ++k) {
                    double a = lrow[k];
                    const uint8_t *wr = wq + k * N;
                    for (n = 0; n < N; ++n)
                        part[n] += a * lut[wr[n]];
                }
                for (n = 0; n < N; ++n)
                    o[n] += part[n] * s_l *
                            (double)sr[(g * nkb + b) * nnb + n / QBLOCK];
            }
        }
        free(part);
        free(lrow);
    }
    free(gid);
}

/* ------------------------------------------------- int4 weights -- */

/* One 128x128 int4 block ([V2s] with the [V2q] recipe; reading above):
 * s = a/7, inv = (s == 0 ? 0 : 1/s), code = round-half-even(w*inv) in
 * [-8, 7].  Each step one IEEE fp32 operation; nearbyintf rounds half to
 * even in the default rounding mode. */
static float quantize_block_int4(const float *vals, int n, int8_t *codes)
{
    float a = 0.0f, s, inv;
    int i;
    for (i = 0; i < n; ++i) {
        float v = fabsf(vals[i]);
        if (v > a)
            a = v;
    }
    s = a / 7.0f;
    inv = (s == 0.0f) ? 0.0f : 1.0f / s;
    for (i = 0; i < n; ++i) {
        float y = nearbyintf(vals[i] * inv);
        if (y > 7.0f)
            y = 7.0f;
        if (y < -8.0f)
            y = -8.0f;
        codes[i] = (int8_t)y;
    }
    return s;
}

/* w: [G,K,N] fp32 -> codes [G,K,N] int8 (values in [-8, 7]) and scales
 * [G,K/128,N/128] fp32, one per 128x128 block as for the FP8 RHS [Q2]. */
void oracle_quantize_rhs_int4(const float *w, int64_t G, int64_t K, int64_t N,
                              int8_t *q, float *scale)
{
    int64_t kb_n = K / QBLOCK, nb_n = N / QBLOCK;
    int64_t t, total = G * kb_n * nb_n;
#pragma omp parallel for schedule(static)
    for (t = 0; t < total; ++t) {
        int64_t g = t / (kb_n * nb_n);
        int64_t kb = (t / nb_n) % kb_n;
        int64_t nb = t % nb_n;
        float *vals = (float *)malloc(sizeof(float) * QBLOCK * QBLOCK);
        int8_t *codes = (int8_t *)malloc(QBLOCK * QBLOCK);
        int64_t i, j;
        for (i = 0; i < QBLOCK; ++i)
            for (j = 0; j < QBLOCK; ++j)
                vals[i * QBLOCK + j] =
                    w[(g * K + kb * QBLOCK + i) * N + nb * QBLOCK + j];
        scale[t] = quantize_block_int4(vals, QBLOCK * QBLOCK, codes);
        for (i = 0; i < QBLOCK; ++i)
            for (j = 0; j < QBLOCK; ++j)
                q[(g * K + kb * QBLOCK + i) * N + nb * QBLOCK + j] =
                    codes[i * QBLOCK + j];
        free(vals);
        free(codes);
    }
}

/* out[m,n] = sum_b ( sum_{k in block b} dec(ql[m,k]) * q4[g,k,n] )
 *                   * scale_l[m,b] * scale_r[g,b,n/128]
 * for m in group g; rows past the total are 0 ([Q2], [Q3], [V1s], [V2s],
 * [GG], [V2z]).  ql: [M,K] E4M3 codes, sl: [M,K/128], q4: [G,K,N] int4
 * values (int8), sr: [G,K/128,N/128]; out: [M,N] fp64. */
void oracle_gmm_fp8_int4(const uint8_t *ql, const float *sl, const int8_t *q4,
                         const float *sr, const int32_t *group_sizes, int64_t M,
                         int64_t K, int64_t N, int64_t G, double *out)
{
    int64_t nkb = K / QBLOCK, nnb = N / QBLOCK, m;
    int32_t *gid = (int32_t *)malloc(sizeof(int32_t) * (M > 0 ? M : 1));
    double lut[256];
    int c;
    for (c = 0; c < 256; ++c)
        lut[c] = oracle_e4m3_decode((uint8_t)c);
    row_groups(group_sizes, G, M, gid);
#pragma omp parallel
    {
        double *part = (double *)malloc(sizeof(double) * N);
#pragma omp for schedule(dynamic, 4)
        for (m = 0; m < M; ++m) {
            int64_t g = gid[m], b, k, n;
            double *o = out + m * N;
            for (n = 0; n < N; ++n)
                o[n] = 0.0;
            if (g >= G)
                continue;
            for (b = 0; b < nkb; ++b) {
                double s_l = (double)sl[m * nkb + b];
                for (n = 0; n < N; ++n)
                    part[n] = 0.0;
                for (k = 0; k < QBLOCK; ++k) {
                    double a = lut[ql[m * K + b * QBLOCK + k]];
                    const int8_t *wr = q4 + (g * K + b * QBLOCK + k) * N;
                    for (n = 0; n < N; ++n)
                        part[n] += a * (double)wr[n];
                }
                for (n = 0; n < N; ++n)
                    o[n] += part[n] * s_l *
                            (double)sr[(g * nkb + b) * nnb + n / QBLOCK];
            }
        }
        free(part);
    }
    free(gid);
}

/* ------------------------------------------------- MXFP4 weights -- */

/* E2M1 code (low 4 bits) -> value ([MX]). */
double oracle_e2m1_decode(uint8_t code)
{
    int e = (code >> 1) & 3, m = code & 1;
    double v = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return (code & 8) ? -v : v;
}

/* Nearest E2M1 value to y, ties to the code with mantissa bit 0, |y| >= 6
 * saturating to 6, sign kept ([MX]; reading above). */
uint8_t oracle_e2m1_encode(double y)
{
    uint8_t sign = (y < 0 || (y == 0 && signbit(y))) ? 8 : 0;
    double a = fabs(y), best_d = 1e300;
    uint8_t best = 0, c;
    if (a >= 6.0)
        return sign | 7;
    for (c = 0; c < 8; ++c) {
        double d = fabs(a - oracle_e2m1_decode(c));
        if (d < best_d || (d == best_d && (c & 1) == 0 && (best & 1) == 1)) {
            best_d = d;
            best = c;
        }
    }
    return sign | best;
}

/* One MXFP4 block of n values: E8M0 code of the shared scale, element
 * codes ([MX]). */
static uint8_t mx_block(const float *vals, int64_t stride, int n, uint8_t *codes,
                        int64_t cstride)
{
    double amax = 0.0;
    int i, e;
    for (i = 0; i < n; ++i)
        if (fabs((double)vals[i * stride]) > amax)
            amax = fabs((double)vals[i * stride]);
    if (amax == 0.0) {
        for (i = 0; i < n; ++i)
            codes[i * cstride] = 0;
        return 0;
    }
    frexp(amax, &e);          /* amax = f 2^e, f in [0.5, 1): floor(log2) = e-1 */
    e = e - 1 - 2;
    if (e < -127)
        e = -127;
    if (e > 127)
        e = 127;
    for (i = 0; i < n; ++i)
        codes[i * cstride] = oracle_e2m1_encode(ldexp((double)vals[i * stride], -e));
    return (uint8_t)(e + 127);
}

/* w: [G,K,N] -> codes [G,K,N] (one E2M1 code per byte) and E8M0 scales
 * [G,K/32,N]: blocks of 32 consecutive k for each (g, n) ([V2s], [MX]). */
void oracle_quantize_rhs_mxfp4(const float *w, int64_t G, int64_t K, int64_t N,
                               uint8_t *q, uint8_t *e8)
{
    int64_t nb = K / 32, g;
#pragma omp parallel for collapse(2) schedule(static)
    for (g = 0; g < G; ++g)
        for (int64_t b = 0; b < nb; ++b)
            for (int64_t n = 0; n < N; ++n) {
                int64_t off = (g * K + b * 32) * N + n;
                e8[(g * nb + b) * N + n] = mx_block(w + off, N, 32, q + off, N);
            }
}

/* out[m,n] = sum_b scale_l[m,b] * sum_{k in 128-block b}
 *            dec8(ql[m,k]) * dec4(q4[g,k,n]) * 2^(e8[g,k/32,n] - 127)
 * for m in group g; rows past the total are 0 ([Q2], [Q3], [V2s], [MX],
 * [GG], [V2z]).  ql [M,K], sl [M,K/128], q4 [G,K,N] codes, e8 [G,K/32,N]. */
void oracle_gmm_fp8_mxfp4(const uint8_t *ql, const float *sl, const uint8_t *q4,
                          const uint8_t *e8, const int32_t *group_sizes, int64_t M,
                          int64_t K, int64_t N, int64_t G, double *out)
{
    int64_t nkb = K / QBLOCK, m;
    int32_t *gid = (int32_t *)malloc(sizeof(int32_t) * (M > 0 ? M : 1));
    double lut8[256], lut4[16];
    int c;
    for (c = 0; c < 256; ++c)
        lut8[c] = oracle_e4m3_decode((uint8_t)c);
    for (c = 0; c < 16; ++c)
        lut4[c] = oracle_e2m1_decode((uint8_t)c);
    row_groups(group_sizes, G, M, gid);
#pragma omp parallel
    {
        double *part = (double *)malloc(sizeof(double) * N);
#pragma omp for schedule(dynamic, 4)
        for (m = 0; m < M; ++m) {
            int64_t g = gid[m], b, k, n;
            double *o = out + m * N;
            for (n = 0; n < N; ++n)
                o[n] = 0.0;
            if (g >= G)
                continue;
            for (b = 0; b < nkb; ++b) {
                for (n = 0; n < N; ++n)
                    part[n] = 0.0;
                for (k = b * QBLOCK; k < (b + 1) * QBLOCK; ++k) {
                    double a = lut8[ql[m * K + k]];
                    const uint8_t *wr = q4 + (g * K + k) * N;
                    const uint8_t *er = e8 + (g * (K / 32) + k / 32) * N;
                    for (n = 0; n < N; ++n)
                        part[n] += a * ldexp(lut4[wr[n] & 15], (int)er[n] - 127);
                }
                for (n = 0; n < N; ++n)
                    o[n] += part[n] * (double)sl[m * nkb + b];
            }
        }
        free(part);
    }
    free(gid);
}

/* ---------------------------------------------- gate+up activation -- */

/* out[m,j] = silu(gu[m,j]) * gu[m,N+j], silu(z) = z / (1 + exp(-z)), in fp64
 * ([V2a]).  gu: [M,2N] (gate columns, then up columns), out: [M,N]. */
void oracle_swiglu(const double *gu, int64_t M, int64_t N, double *out)
{
    int64_t m, j;
    for (m = 0; m < M; ++m)
        for (j = 0; j < N; ++j) {
            double gate = gu[m * 2 * N + j], up = gu[m * 2 * N + N + j];
            out[m * N + j] = gate / (1.0 + exp(-gate)) * up;
        }
}

/* ------------------------------------------------- unquantised (bf16) -- */

/* out[m,:] = x[m,:] . w[g(m)] in fp64 ([GG]); rows past the total are 0.
 * x: [M,K], w: [G,K,N], out: [M,N]. */
void oracle_gmm_f64(const float *x, const float *w, const int32_t *group_sizes,
                    int64_t M, int64_t K, int64_t N, int64_t G, double *out)
{
    int64_t m;
    int32_t *gid = (int32_t *)malloc(sizeof(int32_t) * (M > 0 ? M : 1));
    row_groups(group_sizes, G, M, gid);
#pragma omp parallel for schedule(dynamic, 4)
    for (m = 0; m < M; ++m) {
        int64_t g = gid[m], k, n;
        double *o = out + m * N;
        for (n = 0; n < N; ++n)
            o[n] = 0.0;
        if (g >= G)
            continue;
        for (k = 0; k < K; ++k) {
            double a = (double)x[m * K + k];
            const float *wr = w + (g * K + k) * N;
            for (n = 0; n < N; ++n)
                o[n] += a * (double)wr[n];
        }
    }
    free(gid);
}

/* dW[g] = sum_{m in group g} x[m,:]^T dy[m,:] in fp64 ([Q4]); an empty group
 * gives exactly 0.  x: [M,K], dy: [M,N], dw: [G,K,N]. */
void oracle_tgmm_f64(const float *x, const float *dy, const int32_t *group_sizes,
                     int64_t M, int64_t K, int64_t N, int64_t G, double *dw)
{
    int64_t *off = (int64_t *)malloc(sizeof(int64_t) * (G + 1));
    int64_t t;
    (void)M;
    oracle_group_offsets(group_sizes, G, M, off);
#pragma omp parallel for schedule(dynamic, 1)
    for (t = 0; t < G * K; ++t) {
        int64_t g = t / K, k = t % K, m, n;
        double *o = dw + (g * K + k) * N;
        for (n = 0; n < N; ++n)
            o[n] = 0.0;
        for (m = off[g]; m < off[g + 1]; ++m) {
            double a = (double)x[m * K + k];
            const float *d = dy + m * N;
            for (n = 0; n < N; ++n)
                o[n] += a * (double)d[n];
        }
    }
    free(off);
}

/* dX[m,:] = dy[m,:] . w[g(m)]^T in fp64, contracting over N ([Q5]); rows
 * past the total are 0.  dy: [M,N], w: [G,K,N], dx: [M,K]. */
void oracle_dx_f64(const float *dy, const float *w, const int32_t *group_sizes,
                   int64_t M, int64_t K, int64_t N, int64_t G, double *dx)
{
    int64_t m;
    int32_t *gid = (int32_t *)malloc(sizeof(int32_t) * (M > 0 ? M : 1));
    row_groups(group_sizes, G, M, gid);
#pragma omp parallel for schedule(dynamic, 4)
    for (m = 0; m < M; ++m) {
        int64_t g = gid[m], k, n;
        double *o = dx + m * K;
        for (k = 0; k < K; ++k)
            o[k] = 0.0;
        if (g >= G)
            continue;
        for (k = 0; k < K; ++k) {
            const float *wr = w + (g * K + k) * N;
            const float *d = dy + m * N;
            double acc = 0.0;
            for (n = 0; n < N; ++n)
                acc += (double)d[n] * (double)wr[n];
            o[k] = acc;
        }
    }
    free(gid);
}
