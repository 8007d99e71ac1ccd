/*
 * oracle.c -- plain, slow, fp64 CPU oracle for block-quantized weight GEMV.
 *
 * TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the benchmark's
 * CPU-baseline leg load this library.  It shares no code, header, table or
 * constant with the HIP library and includes no HIP header.
 *
 * What it computes (the plain definition, nothing blocked, fused or reordered):
 *   every weight is decoded from its canonical block to an fp64 value, every
 *   activation is widened to fp64, and each output is the naive dot product of
 *   one weight row with one activation vector, summed with k ascending.
 *
 * Sources for the formats:
 *   - Q8_0 and Q4_0 are named as the GGUF weight formats the engines stream
 *     (Imparo README, opening notes on the LFM2.5-8B-A1B Q4_0 route and the
 *     M3 Pro table's Q8_0 model; imp README, "Supported models" / "Features"
 *     table, Quantization row).  Their block layouts (32 weights, one fp16
 *     scale, Q4_0 zero point 8, nibble split) are the workload definitions;
 *     the pages print no byte layout.
 *   - MXFP4 is 4-bit E2M1 values with UE8M0 block scales at 4.25 bits per
 *     weight (imp release notes, v0.6, "Highlights" and "Features").  4.25 = 4 + 8/32, so a
 *     block is 32 E2M1 codes plus one 8-bit power-of-two scale.
 *   - E2M1 values follow from the name: 1 sign bit, 2 exponent bits with bias
 *     1, 1 mantissa bit, exponent field 0 subnormal, no inf/NaN codes.
 *   - UE8M0 is an unsigned 8-bit biased exponent (bias 127), value 2^(E-127);
 *     E = 255 is read as NaN.
 * Parity pins for every function live in tests/test_oracle.py.
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_Q8_0 = 0, ORC_Q4_0 = 1, ORC_MXFP4 = 2 };

/* Threads an OpenMP region of the oracle uses (1 without OpenMP). */
int orc_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Sets the threads of the oracle's parallel loops (timing legs only: results
 * do not depend on it, every row is summed by one thread in index order). */
void orc_set_threads(int n)
{
#ifdef _OPENMP
    if (n > 0) omp_set_num_threads(n);
#else
    (void)n;
#endif
}
enum { ORC_X_F32 = 0, ORC_X_BF16 = 1 };
enum { ORC_MOE_GATE_UP = 0, ORC_MOE_DOWN = 1 };

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
double orc_fp16(uint16_t h)
{
    int s = h >> 15, e = (h >> 10) & 31, f = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-14 / 1024 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);   /* (1 + f/1024) * 2^(e-15) */
    return s ? -v : v;
}

/* bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits. */
double orc_bf16(uint16_t b)
{
    int s = b >> 15, e = (b >> 7) & 255, f = b & 127;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);              /* f * 2^-126 / 128 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + f), e - 134);   /* (1 + f/128) * 2^(e-127) */
    return s ? -v : v;
}

/* UE8M0 block scale: 2^(E-127); 255 is NaN. */
double orc_e8m0(uint8_t e)
{
    if (e == 255)
        return NAN;
    return ldexp(1.0, (int)e - 127);
}

/* FP4 E2M1 code c (low 4 bits): sign bit 3, exponent bits 2..1, mantissa bit 0. */
double orc_e2m1(uint8_t c)
{
    int s = (c >> 3) & 1, e = (c >> 1) & 3, m = c & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

static int block_bytes(int fmt)
{
    return fmt == ORC_Q8_0 ? 34 : fmt == ORC_Q4_0 ? 18 : fmt == ORC_MXFP4 ? 17 : 0;
}

/* Weight i (0..31) of one canonical block. */
static double block_weight(int fmt, const uint8_t *blk, int i)
{
    if (fmt == ORC_Q8_0) {
        double d = orc_fp16((uint16_t)(blk[0] | (blk[1] << 8)));
        return d * (double)(int8_t)blk[2 + i];
    }
    if (fmt == ORC_Q4_0) {
        double d = orc_fp16((uint16_t)(blk[0] | (blk[1] << 8)));
        uint8_t byte = blk[2 + (i & 15)];
        int q = (i < 16) ? (byte & 15) : (byte >> 4);
        return d * (double)(q - 8);
    }
    /* MXFP4 */
    {
        double sc = orc_e8m0(blk[0]);
        uint8_t byte = blk[1 + (i & 15)];
        uint8_t c = (i < 16) ? (byte & 15) : (byte >> 4);
        return orc_e2m1(c) * sc;
    }
}

static double act(const void *x, int xt, int64_t idx)
{
    if (xt == ORC_X_F32)
        return (double)((const float *)x)[idx];
    return orc_bf16(((const uint16_t *)x)[idx]);
}

/* Element (r, c) of an n x k matrix of canonical blocks. */
static double weight_at(int fmt, const uint8_t *blocks, int64_t k, int64_t r, int64_t c)
{
    int64_t nb = k / 32;
    const uint8_t *blk = blocks + (r * nb + c / 32) * (int64_t)block_bytes(fmt);
    return block_weight(fmt, blk, (int)(c % 32));
}

static int check(int fmt, int64_t n, int64_t k, int xt)
{
    if (block_bytes(fmt) == 0 || n <= 0 || k <= 0 || (k % 32) != 0)
        return 1;
    if (xt != ORC_X_F32 && xt != ORC_X_BF16)
        return 1;
    return 0;
}

/* w[r][c] for all n x k elements. */
int orc_decode(int fmt, const uint8_t *blocks, int64_t n, int64_t k, double *w)
{
    if (check(fmt, n, k, ORC_X_F32))
        return 1;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c)
            w[r * k + c] = weight_at(fmt, blocks, k, r, c);
    return 0;
}

/*
 * Dense product for m activation vectors x[t][0..k) (t < m):
 *   y[t][i]  = sum_{c ascending} W[row_i][c] * x[t][c]
 *   l1[t][i] = sum_c |W[row_i][c] * x[t][c]|
 * rows == NULL means row_i = i for i < nrows (nrows = n).
 */
int orc_gemv(int fmt, const uint8_t *blocks, int64_t n, int64_t k,
             const void *x, int xt, int64_t m,
             const int64_t *rows, int64_t nrows, double *y, double *l1)
{
    if (check(fmt, n, k, xt) || m <= 0 || nrows <= 0)
        return 1;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows && (rows[i] < 0 || rows[i] >= n))
            return 1;
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        for (int64_t t = 0; t < m; ++t) {
            double s = 0.0, a = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                double p = weight_at(fmt, blocks, k, r, c) * act(x, xt, t * k + c);
                s += p;
                a += fabs(p);
            }
            y[t * nrows + i] = s;
            l1[t * nrows + i] = a;
        }
    }
    return 0;
}

/*
 * Top-k expert product.  experts: n_experts matrices of n x k canonical blocks,
 * back to back.  ids[t][j], g[t][j] for t < m, j < top_k.
 *   GATE_UP: x [m][k];        y[t][j][i] = W_{ids[t][j]}[row_i] . x[t]
 *            l1 likewise with |products|.
 *   DOWN:    x [m][top_k][k]; y[t][i] = sum_{j ascending} g[t][j] * (W_{ids[t][j]}[row_i] . x[t][j])
 *            l1[t][i] = sum_j |g[t][j]| * sum_c |W . x| .
 */
int orc_moe(int fmt, const uint8_t *experts, int64_t n_experts, int64_t n, int64_t k,
            const int32_t *ids, const float *g, int64_t m, int64_t top_k,
            const void *x, int xt, int mode,
            const int64_t *rows, int64_t nrows, double *y, double *l1)
{
    if (check(fmt, n, k, xt) || m <= 0 || nrows <= 0 || n_experts <= 0 || top_k <= 0)
        return 1;
    if (mode != ORC_MOE_GATE_UP && mode != ORC_MOE_DOWN)
        return 1;
    if (mode == ORC_MOE_DOWN && g == NULL)
        return 1;
    for (int64_t s = 0; s < m * top_k; ++s)
        if (ids[s] < 0 || ids[s] >= n_experts)
            return 1;
    for (int64_t i = 0; i < nrows; ++i)
        if (rows && (rows[i] < 0 || rows[i] >= n))
            return 1;
    int64_t mat_bytes = n * (k / 32) * (int64_t)block_bytes(fmt);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        for (int64_t t = 0; t < m; ++t) {
            double ys = 0.0, ya = 0.0;
            for (int64_t j = 0; j < top_k; ++j) {
                const uint8_t *W = experts + (int64_t)ids[t * top_k + j] * mat_bytes;
                int64_t xoff = (mode == ORC_MOE_GATE_UP) ? t * k : (t * top_k + j) * k;
                double s = 0.0, a = 0.0;
                for (int64_t c = 0; c < k; ++c) {
                    double p = weight_at(fmt, W, k, r, c) * act(x, xt, xoff + c);
                    s += p;
                    a += fabs(p);
                }
                if (mode == ORC_MOE_GATE_UP) {
                    y[(t * top_k + j) * nrows + i] = s;
                    l1[(t * top_k + j) * nrows + i] = a;
                } else {
                    double gj = (double)g[t * top_k + j];
                    ys += gj * s;
                    ya += fabs(gj) * a;
                }
            }
            if (mode == ORC_MOE_DOWN) {
                y[t * nrows + i] = ys;
                l1[t * nrows + i] = ya;
            }
        }
    }
    return 0;
}
