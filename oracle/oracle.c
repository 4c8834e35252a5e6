/*
 * CPU oracle for group-wise low-bit weight quantization (asymmetric min/max,
 * and the symmetric absolute-maximum variant) and the dequantize-then-multiply
 * decode product.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no code, header, table or constant
 * generator with the GPU library.
 *
 * Sources (cited by page title and section):
 *   [KVQ]  "What actually happens when you quantize a KV cache" — §3 steps 3-5
 *          (min/max, scale, zero point, encode, nibble packing, 4-byte header)
 *          and §4 "The math on paper" (the four-line summary of the codec and
 *          the |x - x_hat| <= s/2 bound).
 *   [QIO]  "Quantization & inference optimisation" — section "Quantization"
 *          (groups of consecutive weights from one row; the kernel
 *          reconstructs the float from the integer and the group header as it
 *          reads) and "Bandwidth, not compute" (Y = X W^T at batch B).
 *   [SMU]  "Serving many users at once: batching and quantization" — section
 *          "Quantization" (groups of consecutive weights of a (out, in)
 *          weight, i.e. along K).
 *
 * Arithmetic.  Every fp16 value is an integer multiple of 2^-24, so each input
 * is held exactly as an int64 count of 2^-24 units.  All quantization
 * decisions are then exact rational arithmetic on integers; rounding happens
 * only where a value is stored (scale and zero point in fp16) or where the
 * pages round (the zero point and the codes, round half to even as the
 * pages' code blocks do).  Dequantization and the product run in double.
 *
 * Readings of points the pages leave open (each is stated where it is used):
 *   - round() is round-half-to-even everywhere;
 *   - the scale is the exact quotient (max-min)/(2^b-1) rounded once to fp16,
 *     and every later step uses that stored value;
 *   - a group whose scale rounds to fp16 zero (max == min, or a range of a few
 *     fp16 subnormal steps) gets scale 1.0;
 *   - the zero point is stored in fp16 (round half to even), saturating to
 *     +-65504 instead of overflowing; a zero point of 0 is stored as +0.0;
 *   - codes use the stored zero point;
 *   - codes of one row form a little-endian bit stream: code k occupies bits
 *     [k*b, k*b+b) of the row, which is the pages' "even channel in the low
 *     nibble" at b = 4 and one byte per code at b = 8;
 *   - NaN and Inf weights are rejected.
 *
 * Float-offset variant (oracle_quantize_offset), readings: the scale as
 * above; the offset is the group minimum itself in fp16 (exact); codes
 * round((x - min)/s) half to even, clamped to [0, 2^b - 1]; x_hat = q*s + min.
 *
 * Symmetric variant (oracle_quantize_sym), readings:
 *   - the scale is max|x| / (2^(b-1) - 1), the exact quotient rounded once to
 *     fp16 as above; an all-zero scope gets scale 1.0;
 *   - the signed integer clamps to [-2^(b-1), 2^(b-1) - 1] (the pages' clamp
 *     keeps the extra negative level) and is stored offset by 2^(b-1), with
 *     that offset as the fp16 zero point;
 *   - one scale per tensor is stored as that scale repeated in every group
 *     header, so every scope shares one layout.
 */
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <math.h>

#define ORACLE_OK 0
#define ORACLE_EINVAL 1
#define ORACLE_ENONFINITE 2
#define ORACLE_ENOMEM 3

/* fp16 bits -> exact value in units of 2^-24.  Returns -1 for NaN/Inf. */
static int fp16_to_units(uint16_t h, int64_t *out)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 31;
    int64_t f = h & 1023;
    int64_t mag;
    if (e == 31)
        return -1;
    if (e == 0)
        mag = f;                         /* subnormal: f * 2^-24 */
    else
        mag = (1024 + f) << (e - 1);     /* (1 + f/1024) * 2^(e-15) */
    *out = sign ? -mag : mag;
    return 0;
}

/* fp16 bits -> double (exact). */
static double fp16_to_double(uint16_t h)
{
    int64_t u;
    if (fp16_to_units(h, &u) != 0)
        return NAN;
    return ldexp((double)u, -24);
}

/* Round-half-to-even quotient of p >= 0 by q > 0. */
static int64_t rne_div_nonneg(int64_t p, int64_t q)
{
    int64_t fl = p / q;
    int64_t rem = p % q;
    if (2 * rem > q || (2 * rem == q && (fl & 1)))
        fl += 1;
    return fl;
}

/* Round-half-to-even quotient of p by q > 0 (rounding is symmetric in sign). */
static int64_t rne_div(int64_t p, int64_t q)
{
    return p < 0 ? -rne_div_nonneg(-p, q) : rne_div_nonneg(p, q);
}

/*
 * Nearest fp16 (ties to even significand) to the nonnegative rational
 * num / den, measured in units of 2^-24.  The finite fp16 grid in these units
 * is {k : 0 <= k < 1024} (zero and subnormals) and {k * 2^sh : 1024 <= k <
 * 2048, 0 <= sh <= 29}.  Sets *overflow when the result would exceed 65504.
 */
static uint16_t fp16_nearest_ratio(int64_t num, int64_t den, int *overflow)
{
    int sh = 0;
    int64_t sig;
    *overflow = 0;
    while (sh < 30 && num >= ((int64_t)2048 * den) << sh)
        sh++;
    sig = rne_div_nonneg(num, den << sh);
    if (sig == 2048) {                   /* rounded up into the next binade */
        sig = 1024;
        sh += 1;
    }
    if (sh >= 30) {
        *overflow = 1;
        return 0x7BFF;
    }
    if (sh == 0 && sig < 1024)
        return (uint16_t)sig;            /* zero or subnormal */
    return (uint16_t)(((sh + 1) << 10) | (sig - 1024));
}

/* fp16 storage of an integer zero point: round half to even, saturating. */
static uint16_t zero_point_to_fp16(int64_t z)
{
    int64_t mag = z < 0 ? -z : z;
    int ovf = 0;
    uint16_t bits;
    if (mag == 0)
        return 0x0000;                   /* +0.0, never -0.0 */
    if (mag >= ((int64_t)1 << 38))
        ovf = 1, bits = 0x7BFF;
    else
        bits = fp16_nearest_ratio(mag << 24, 1, &ovf);
    if (ovf)
        bits = 0x7BFF;                   /* saturate at 65504 */
    return (uint16_t)(z < 0 ? (bits | 0x8000) : bits);
}

static int check_shape(int64_t N, int64_t K, int32_t group, int32_t bits)
{
    if (N < 0 || K < 1 || group < 1 || bits < 2 || bits > 8)
        return ORACLE_EINVAL;
    if (K % group != 0)
        return ORACLE_EINVAL;
    if ((K * bits) % 8 != 0)
        return ORACLE_EINVAL;
    return ORACLE_OK;
}

/* Write code q (b bits) at bit offset k*b of a row (little-endian stream). */
static void put_code(uint8_t *row, int64_t k, int bits, unsigned q)
{
    int64_t bit = k * bits;
    int i;
    for (i = 0; i < bits; i++, bit++)
        if ((q >> i) & 1u)
            row[bit >> 3] |= (uint8_t)(1u << (bit & 7));
}

static unsigned get_code(const uint8_t *row, int64_t k, int bits)
{
    int64_t bit = k * bits;
    unsigned q = 0;
    int i;
    for (i = 0; i < bits; i++, bit++)
        q |= (unsigned)((row[bit >> 3] >> (bit & 7)) & 1u) << i;
    return q;
}

/*
 * Quantize one group of G values (int64 units of 2^-24) following [KVQ] §3
 * steps 3-4 and §4:
 *   min, max over the group                          (one pass)
 *   s = (max - min) / (2^b - 1)                      stored in fp16
 *   z = round(-min / s)                              stored in fp16
 *   q = clamp(round(x / s) + z, 0, 2^b - 1)
 */
static void quantize_group(const int64_t *x, int64_t G, int bits,
                           unsigned *q, uint16_t *scale_bits, uint16_t *zero_bits)
{
    const int64_t M = ((int64_t)1 << bits) - 1;
    int64_t mn = x[0], mx = x[0], S = 0, Zu = 0, Z;
    int64_t i, z;
    int ovf;
    uint16_t sb, zb;

    for (i = 1; i < G; i++) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    /* s: exact quotient of the range by the number of steps, rounded once to
     * fp16.  M >= 3 and range <= 2*65504 keep it below the fp16 maximum. */
    sb = fp16_nearest_ratio(mx - mn, M, &ovf);
    if (sb == 0)
        sb = 0x3C00;                     /* degenerate group: s = 1.0 */
    fp16_to_units(sb, &S);

    /* z: the integer code that decodes to zero, from the stored scale. */
    z = rne_div(-mn, S);
    zb = zero_point_to_fp16(z);
    fp16_to_units(zb, &Zu);
    Z = Zu / ((int64_t)1 << 24);         /* stored zero points are integers */

    for (i = 0; i < G; i++) {
        int64_t c = rne_div(x[i], S) + Z;
        if (c < 0) c = 0;
        if (c > M) c = M;
        q[i] = (unsigned)c;
    }
    *scale_bits = sb;
    *zero_bits = zb;
}

/*
 * W fp16 [N, K] row-major -> codes u8 [N, K*bits/8], scales fp16 [N, K/group],
 * zeros fp16 [N, K/group].  Groups are `group` consecutive k of one row
 * ([QIO] "Quantization"; [SMU] "Quantization").
 */
int oracle_quantize(const uint16_t *W, int64_t N, int64_t K, int32_t group,
                    int32_t bits, uint8_t *codes, uint16_t *scales, uint16_t *zeros)
{
    const int64_t row_bytes = K * bits / 8;
    const int64_t ngroups = K / group;
    int64_t n;
    int err = check_shape(N, K, group, bits);
    if (err)
        return err;
    for (n = 0; n < N * K; n++) {
        int64_t u;
        if (fp16_to_units(W[n], &u) != 0)
            return ORACLE_ENONFINITE;
    }
    memset(codes, 0, (size_t)(N * row_bytes));
    err = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; n++) {
        int64_t *xu = (int64_t *)malloc(sizeof(int64_t) * (size_t)group);
        unsigned *q = (unsigned *)malloc(sizeof(unsigned) * (size_t)group);
        int64_t g, i;
        if (!xu || !q) {
            err = ORACLE_ENOMEM;
            free(xu);
            free(q);
            continue;
        }
        for (g = 0; g < ngroups; g++) {
            const uint16_t *src = W + n * K + g * group;
            for (i = 0; i < group; i++)
                fp16_to_units(src[i], &xu[i]);
            quantize_group(xu, group, bits, q, &scales[n * ngroups + g],
                           &zeros[n * ngroups + g]);
            for (i = 0; i < group; i++)
                put_code(codes + n * row_bytes, g * group + i, bits, q[i]);
        }
        free(xu);
        free(q);
    }
    return err;
}

/*
 * Symmetric absolute-maximum quantization of one group ([QIO] "Quantize a
 * matrix by hand" and "Per-channel, and what it buys"; [SMU]
 * "Quantization: rounding the weights"):
 *   qmax = 2^(b-1) - 1
 *   s = A / qmax, A = max |x| over the scale's scope   stored in fp16
 *   q = clamp(round(x / s), -qmax - 1, qmax)
 * The signed q is stored as the code q + 2^(b-1) with the zero point 2^(b-1)
 * (exact in fp16), so (code - zero) * s is the page's q * s and the
 * asymmetric decoder reads it unchanged.  A is passed in: the group's own
 * maximum, or the whole matrix's for one scale per tensor.
 */
static void quantize_group_sym(const int64_t *x, int64_t G, int bits, int64_t A,
                               unsigned *q, uint16_t *scale_bits, uint16_t *zero_bits)
{
    const int64_t qmax = ((int64_t)1 << (bits - 1)) - 1;
    const int64_t half = (int64_t)1 << (bits - 1);
    int64_t S = 0, i;
    int ovf;
    uint16_t sb = fp16_nearest_ratio(A, qmax, &ovf);
    if (sb == 0)
        sb = 0x3C00;                     /* all-zero scope (or a few subnormal steps): s = 1.0 */
    fp16_to_units(sb, &S);
    for (i = 0; i < G; i++) {
        int64_t c = rne_div(x[i], S);
        if (c < -qmax - 1) c = -qmax - 1;
        if (c > qmax) c = qmax;
        q[i] = (unsigned)(c + half);
    }
    *scale_bits = sb;
    *zero_bits = zero_point_to_fp16(half);
}

/*
 * Symmetric variant of oracle_quantize: same layout and packing.  per_tensor
 * = 0 takes A per group (group = K is one scale per output channel);
 * per_tensor = 1 takes one A over the whole matrix and repeats its scale in
 * every group header.
 */
int oracle_quantize_sym(const uint16_t *W, int64_t N, int64_t K, int32_t group,
                        int32_t bits, int32_t per_tensor, uint8_t *codes,
                        uint16_t *scales, uint16_t *zeros)
{
    const int64_t row_bytes = K * bits / 8;
    const int64_t ngroups = K / group;
    int64_t n, Aall = 0;
    int err = check_shape(N, K, group, bits);
    if (err)
        return err;
    for (n = 0; n < N * K; n++) {
        int64_t u;
        if (fp16_to_units(W[n], &u) != 0)
            return ORACLE_ENONFINITE;
        if (u < 0) u = -u;
        if (u > Aall) Aall = u;
    }
    memset(codes, 0, (size_t)(N * row_bytes));
    err = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; n++) {
        int64_t *xu = (int64_t *)malloc(sizeof(int64_t) * (size_t)group);
        unsigned *q = (unsigned *)malloc(sizeof(unsigned) * (size_t)group);
        int64_t g, i;
        if (!xu || !q) {
            err = ORACLE_ENOMEM;
            free(xu);
            free(q);
            continue;
        }
        for (g = 0; g < ngroups; g++) {
            const uint16_t *src = W + n * K + g * group;
            int64_t A = 0;
            for (i = 0; i < group; i++) {
                fp16_to_units(src[i], &xu[i]);
                if (xu[i] > A) A = xu[i];
                if (-xu[i] > A) A = -xu[i];
            }
            quantize_group_sym(xu, group, bits, per_tensor ? Aall : A, q,
                               &scales[n * ngroups + g], &zeros[n * ngroups + g]);
            for (i = 0; i < group; i++)
                put_code(codes + n * row_bytes, g * group + i, bits, q[i]);
        }
        free(xu);
        free(q);
    }
    return err;
}

/*
 * Float-offset variant ([QIO] "Quantization", the affine per-group code
 * block): the group's minimum is kept as a float offset instead of an
 * integer zero point.
 *   s = (max - min) / (2^b - 1)            stored in fp16 (as above)
 *   m = min                                stored in fp16 (exact: an input)
 *   q = clamp(round((x - m) / s), 0, 2^b - 1)
 *   x_hat = q * s + m
 * The clamp only acts when the fp16 scale rounded below the exact quotient.
 */
static void quantize_group_offset(const int64_t *x, int64_t G, int bits, unsigned *q,
                                  uint16_t *scale_bits, uint16_t *min_bits)
{
    const int64_t M = ((int64_t)1 << bits) - 1;
    int64_t mn = x[0], mx = x[0], S = 0, i;
    int ovf;
    uint16_t sb;
    for (i = 1; i < G; i++) {
        if (x[i] < mn) mn = x[i];
        if (x[i] > mx) mx = x[i];
    }
    sb = fp16_nearest_ratio(mx - mn, M, &ovf);
    if (sb == 0)
        sb = 0x3C00;
    fp16_to_units(sb, &S);
    for (i = 0; i < G; i++) {
        int64_t c = rne_div(x[i] - mn, S);
        if (c > M) c = M;
        q[i] = (unsigned)c;              /* x - mn >= 0, so c >= 0 */
    }
    *scale_bits = sb;
    *min_bits = 0;
    {
        /* the minimum is one of the fp16 inputs: recover its bits */
        int64_t mag = mn < 0 ? -mn : mn;
        uint16_t b = 0;
        if (mag != 0) {
            int dummy;
            b = fp16_nearest_ratio(mag, 1, &dummy);
        }
        *min_bits = (uint16_t)(mn < 0 ? (b | 0x8000) : b);
    }
}

int oracle_quantize_offset(const uint16_t *W, int64_t N, int64_t K, int32_t group,
                           int32_t bits, uint8_t *codes, uint16_t *scales, uint16_t *mins)
{
    const int64_t row_bytes = K * bits / 8;
    const int64_t ngroups = K / group;
    int64_t n;
    int err = check_shape(N, K, group, bits);
    if (err)
        return err;
    for (n = 0; n < N * K; n++) {
        int64_t u;
        if (fp16_to_units(W[n], &u) != 0)
            return ORACLE_ENONFINITE;
    }
    memset(codes, 0, (size_t)(N * row_bytes));
    err = ORACLE_OK;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; n++) {
        int64_t *xu = (int64_t *)malloc(sizeof(int64_t) * (size_t)group);
        unsigned *q = (unsigned *)malloc(sizeof(unsigned) * (size_t)group);
        int64_t g, i;
        if (!xu || !q) {
            err = ORACLE_ENOMEM;
            free(xu);
            free(q);
            continue;
        }
        for (g = 0; g < ngroups; g++) {
            const uint16_t *src = W + n * K + g * group;
            for (i = 0; i < group; i++)
                fp16_to_units(src[i], &xu[i]);
            quantize_group_offset(xu, group, bits, q, &scales[n * ngroups + g],
                                  &mins[n * ngroups + g]);
            for (i = 0; i < group; i++)
                put_code(codes + n * row_bytes, g * group + i, bits, q[i]);
        }
        free(xu);
        free(q);
    }
    return err;
}

/* Dequantize one row: w_hat[k] = (q - z) * s in double ([KVQ] §3 step 4, §4). */
static void dequant_row(const uint8_t *row, const uint16_t *scales,
                        const uint16_t *zeros, int64_t K, int32_t group,
                        int32_t bits, double *out)
{
    int64_t k;
    for (k = 0; k < K; k++) {
        double s = fp16_to_double(scales[k / group]);
        double z = fp16_to_double(zeros[k / group]);
        out[k] = ((double)get_code(row, k, bits) - z) * s;
    }
}

/* W_hat double [N, K] from the packed representation. */
int oracle_dequantize(const uint8_t *codes, const uint16_t *scales,
                      const uint16_t *zeros, int64_t N, int64_t K, int32_t group,
                      int32_t bits, double *W_hat)
{
    const int64_t row_bytes = K * bits / 8;
    const int64_t ngroups = K / group;
    int64_t n;
    int err = check_shape(N, K, group, bits);
    if (err)
        return err;
#pragma omp parallel for schedule(static)
    for (n = 0; n < N; n++)
        dequant_row(codes + n * row_bytes, scales + n * ngroups, zeros + n * ngroups,
                    K, group, bits, W_hat + n * K);
    return ORACLE_OK;
}

/*
 * Y[b, n] = sum_k X[b, k] * W_hat[n, k] in double, k ascending, for the
 * output rows listed in `rows` (all rows when rows == NULL; then nrows == N).
 * Y is [B, nrows].  ([QIO] "Bandwidth, not compute": every weight is used once
 * per sequence of the batch; [SMU] "Batching": the batch's rows are stacked
 * and multiplied once.)
 */
int oracle_gemm_rows(const uint16_t *X, const uint8_t *codes, const uint16_t *scales,
                     const uint16_t *zeros, int64_t B, int64_t K, int64_t N,
                     int32_t group, int32_t bits, const int64_t *rows,
                     int64_t nrows, double *Y)
{
    const int64_t row_bytes = K * bits / 8;
    const int64_t ngroups = K / group;
    double *xd;
    int64_t i, j;
    int err = check_shape(N, K, group, bits);
    if (err)
        return err;
    if (B < 0 || nrows < 0)
        return ORACLE_EINVAL;
    if (rows)
        for (j = 0; j < nrows; j++)
            if (rows[j] < 0 || rows[j] >= N)
                return ORACLE_EINVAL;
    xd = (double *)malloc(sizeof(double) * (size_t)(B * K + 1));
    if (!xd)
        return ORACLE_ENOMEM;
    for (i = 0; i < B * K; i++)
        xd[i] = fp16_to_double(X[i]);
    err = ORACLE_OK;
#pragma omp parallel for schedule(dynamic, 4)
    for (j = 0; j < nrows; j++) {
        int64_t n = rows ? rows[j] : j;
        double *w = (double *)malloc(sizeof(double) * (size_t)K);
        int64_t b, k;
        if (!w) {
            err = ORACLE_ENOMEM;
            continue;
        }
        dequant_row(codes + n * row_bytes, scales + n * ngroups, zeros + n * ngroups,
                    K, group, bits, w);
        for (b = 0; b < B; b++) {
            double acc = 0.0;
            for (k = 0; k < K; k++)
                acc += xd[b * K + k] * w[k];
            Y[b * nrows + j] = acc;
        }
        free(w);
    }
    free(xd);
    return err;
}

int oracle_gemm(const uint16_t *X, const uint8_t *codes, const uint16_t *scales,
                const uint16_t *zeros, int64_t B, int64_t K, int64_t N,
                int32_t group, int32_t bits, double *Y)
{
    return oracle_gemm_rows(X, codes, scales, zeros, B, K, N, group, bits, NULL, N, Y);
}

/* Threads the OpenMP runtime will use (reported with CPU timings). */
int oracle_num_threads(void)
{
#ifdef _OPENMP
    extern int omp_get_max_threads(void);
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the number of OpenMP threads later calls use (timing of the oracle on
 * one core and on all of them; no effect on any result). */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    extern void omp_set_num_threads(int);
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
