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
 *   - NVFP4 is the 4-bit format of imp's decode cache and sm_120a GEMV (imp
 *     README, "Why this exists" and the "Features" table's sm_120a row: FP4
 *     values with packed E2M1 and E4M3 conversions); the pages name it but do
 *     not define it.  Its public definition: blocks of 16 E2M1 values, one
 *     FP8 E4M3 scale per block, and one fp32 scale per tensor;
 *     w = E2M1(c) * E4M3(s) * s_tensor.  E4M3 here is the OCP FP8 E4M3 format:
 *     1 sign, 4 exponent bits (bias 7), 3 mantissa bits, exponent field 0
 *     subnormal, S.1111.111 NaN, no infinities (largest finite 448).
 *     Canonical byte layout (a reading): per 16 weights, the E4M3 scale byte
 *     then 8 code bytes, byte j holding element j in its low nibble and
 *     element j+8 in its high nibble; a tensor is its n * (k/16) blocks
 *     row-major followed by the fp32 tensor scale, little-endian.
 *   - The NVFP4 quantizer (imp's load-time "decode cache" from Q8_0: imp
 *     README, "Why this exists") follows the same public recipe: the tensor
 *     scale maps the tensor's largest magnitude to 6 * 448, each block scale is
 *     the block's largest magnitude over 6 in units of the tensor scale,
 *     rounded to E4M3, and each value is rounded to E2M1 in units of the
 *     decoded block scale; roundings are to nearest, ties to the even code,
 *     saturating at the largest finite value.  Its arithmetic is fp32, in the
 *     order written in orc_nvfp4_quantize.
 *   - Q4_K and Q6_K are the K-quant super-block formats of the imp engine's
 *     GGUF models (imp README, "Features" table, Quantization row; imp
 *     release notes v0.7.0, Gemma-4 Q4_K_M decode; a Q4_K_M file mixes Q4_K
 *     and Q6_K tensors).  The pages name them but do not define them; their
 *     public GGUF definitions, 256 weights per super-block:
 *       Q4_K, 144 bytes: d (fp16), dmin (fp16), 12 bytes of 6-bit scales and
 *         mins, 128 bytes of 4-bit codes.  Sub-block j (weights 32j..32j+31)
 *         has scale sc_j and min m_j: for j < 4, sc_j = s[j] & 63 and
 *         m_j = s[j+4] & 63; for j >= 4, sc_j = (s[j+4] & 15) | (s[j-4] >> 6) << 4
 *         and m_j = (s[j+4] >> 4) | (s[j] >> 6) << 4.  The codes of the 64
 *         weights 64c..64c+63 are the 32 bytes qs[32c..32c+31]: weight 64c+l
 *         is the low nibble of qs[32c+l], weight 64c+32+l its high nibble.
 *         w = d * sc_j * q - dmin * m_j.
 *       Q6_K, 210 bytes: ql (128 bytes, low 4 bits), qh (64 bytes, high 2
 *         bits), 16 int8 scales (one per 16 weights), d (fp16).  Weight
 *         128h + 32r + l (h < 2, r < 4, l < 32) has low bits from
 *         ql[64h + l + 32(r & 1)] (low nibble for r < 2, high for r >= 2),
 *         high bits (qh[32h + l] >> 2r) & 3, scale sc[8h + 2r + l / 16], and
 *         w = d * sc * (q - 32), q = low | high << 4.
 *     The value is the exact real number of these products (the reading
 *     taken: fp64 here, where it is exact).
 * Parity pins for every function live in tests/test_oracle.py (K-quants:
 * tests/test_oracle_kquants.py).
 */
#include <math.h>
#include <stdint.h>
#include <stddef.h>

#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_Q8_0 = 0, ORC_Q4_0 = 1, ORC_MXFP4 = 2, ORC_NVFP4 = 3, ORC_Q4_K = 4, ORC_Q6_K = 5 };

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

/* OCP FP8 E4M3 s: sign bit 7, exponent bits 6..3 (bias 7), mantissa bits 2..0;
 * exponent field 0 is subnormal (m/8 * 2^-6); S.1111.111 is NaN; no infinity. */
double orc_e4m3(uint8_t b)
{
    int s = b >> 7, e = (b >> 3) & 15, m = b & 7;
    double mag;
    if (e == 15 && m == 7)
        return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp(1.0 + m / 8.0, e - 7);
    return s ? -mag : mag;
}

/* Bytes of one canonical block (32 weights; 16 for NVFP4, 256 for the K-quants). */
static int block_bytes(int fmt)
{
    return fmt == ORC_Q8_0 ? 34 : fmt == ORC_Q4_0 ? 18 : fmt == ORC_MXFP4 ? 17 : fmt == ORC_NVFP4 ? 9
         : fmt == ORC_Q4_K ? 144 : fmt == ORC_Q6_K ? 210 : 0;
}

static int block_len(int fmt) { return fmt == ORC_NVFP4 ? 16 : (fmt == ORC_Q4_K || fmt == ORC_Q6_K) ? 256 : 32; }

/* k must be a multiple of 32, and of the super-block (256) for the K-quants. */
static int bad_k(int fmt, int64_t k) { return k <= 0 || (k % 32) != 0 || (k % block_len(fmt)) != 0; }

/* Bytes of one canonical n x k tensor (NVFP4: blocks, then the fp32 tensor scale). */
int64_t orc_tensor_bytes(int fmt, int64_t n, int64_t k)
{
    if (block_bytes(fmt) == 0 || n <= 0 || bad_k(fmt, k))
        return -1;
    return n * (k / block_len(fmt)) * (int64_t)block_bytes(fmt) + (fmt == ORC_NVFP4 ? 4 : 0);
}

/* The fp32 tensor scale stored after an NVFP4 tensor's blocks. */
static double nvfp4_tensor_scale(const uint8_t *blocks, int64_t n, int64_t k)
{
    const uint8_t *p = blocks + n * (k / 16) * 9;
    union { uint32_t u; float f; } v;
    v.u = (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) | ((uint32_t)p[3] << 24);
    return (double)v.f;
}

/* Q4_K sub-block j's 6-bit scale and min. */
static void q4k_scale_min(const uint8_t *s, int j, int *sc, int *m)
{
    if (j < 4) {
        *sc = s[j] & 63;
        *m = s[j + 4] & 63;
    } else {
        *sc = (s[j + 4] & 15) | ((s[j - 4] >> 6) << 4);
        *m = (s[j + 4] >> 4) | ((s[j] >> 6) << 4);
    }
}

/* Weight i (0..255) of a Q4_K super-block. */
static double q4k_weight(const uint8_t *blk, int i)
{
    const double d = orc_fp16((uint16_t)(blk[0] | (blk[1] << 8)));
    const double dmin = orc_fp16((uint16_t)(blk[2] | (blk[3] << 8)));
    int sc, m;
    q4k_scale_min(blk + 4, i / 32, &sc, &m);
    const int c = i / 64, l = i % 64;
    const uint8_t byte = blk[16 + 32 * c + (l % 32)];
    const int q = l < 32 ? (byte & 15) : (byte >> 4);
    return d * sc * q - dmin * m;
}

/* Weight i (0..255) of a Q6_K super-block. */
static double q6k_weight(const uint8_t *blk, int i)
{
    const int h = i / 128, r = (i % 128) / 32, l = i % 32;
    const uint8_t lo_byte = blk[64 * h + l + 32 * (r & 1)];
    const int lo = r < 2 ? (lo_byte & 15) : (lo_byte >> 4);
    const int hi = (blk[128 + 32 * h + l] >> (2 * r)) & 3;
    const int sc = (int8_t)blk[192 + 8 * h + 2 * r + l / 16];
    const double d = orc_fp16((uint16_t)(blk[208] | (blk[209] << 8)));
    return d * sc * ((lo | (hi << 4)) - 32);
}

/* Weight i (0..31; 0..15 for NVFP4, 0..255 for the K-quants) of one canonical block. */
static double block_weight(int fmt, const uint8_t *blk, int i)
{
    if (fmt == ORC_Q4_K)
        return q4k_weight(blk, i);
    if (fmt == ORC_Q6_K)
        return q6k_weight(blk, i);
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
    if (fmt == ORC_NVFP4) {                      /* i in 0..15; the tensor scale is applied by the caller */
        uint8_t byte = blk[1 + (i & 7)];
        uint8_t c = (i < 8) ? (byte & 15) : (byte >> 4);
        return orc_e2m1(c) * orc_e4m3(blk[0]);
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

/* Element (r, c) of an n x k matrix of canonical blocks (ts: the NVFP4 tensor
 * scale, 1 for the other formats). */
static double weight_at(int fmt, const uint8_t *blocks, int64_t k, int64_t r, int64_t c, double ts)
{
    const int bl = block_len(fmt);
    int64_t nb = k / bl;
    const uint8_t *blk = blocks + (r * nb + c / bl) * (int64_t)block_bytes(fmt);
    return block_weight(fmt, blk, (int)(c % bl)) * ts;
}

static double tensor_scale(int fmt, const uint8_t *blocks, int64_t n, int64_t k)
{
    return fmt == ORC_NVFP4 ? nvfp4_tensor_scale(blocks, n, k) : 1.0;
}

static int check(int fmt, int64_t n, int64_t k, int xt)
{
    if (block_bytes(fmt) == 0 || n <= 0 || bad_k(fmt, k))
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
    const double ts = tensor_scale(fmt, blocks, n, k);
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r)
        for (int64_t c = 0; c < k; ++c)
            w[r * k + c] = weight_at(fmt, blocks, k, r, c, ts);
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
    const double ts = tensor_scale(fmt, blocks, n, k);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        for (int64_t t = 0; t < m; ++t) {
            double s = 0.0, a = 0.0;
            for (int64_t c = 0; c < k; ++c) {
                double p = weight_at(fmt, blocks, k, r, c, ts) * act(x, xt, t * k + c);
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
    int64_t mat_bytes = orc_tensor_bytes(fmt, n, k);
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < nrows; ++i) {
        int64_t r = rows ? rows[i] : i;
        for (int64_t t = 0; t < m; ++t) {
            double ys = 0.0, ya = 0.0;
            for (int64_t j = 0; j < top_k; ++j) {
                const uint8_t *W = experts + (int64_t)ids[t * top_k + j] * mat_bytes;
                const double ts = tensor_scale(fmt, W, n, k);
                int64_t xoff = (mode == ORC_MOE_GATE_UP) ? t * k : (t * top_k + j) * k;
                double s = 0.0, a = 0.0;
                for (int64_t c = 0; c < k; ++c) {
                    double p = weight_at(fmt, W, k, r, c, ts) * act(x, xt, xoff + c);
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

/* ------------------------------------------------------------ NVFP4 quantizer */
/* Round v >= 0 to the nearest non-negative finite E4M3 value (ties to the even
 * code), saturating at 448: the code, by searching every candidate. */
uint8_t orc_e4m3_round(float v)
{
    if (v >= 448.0f)
        return 0x7E;
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 0x7E; ++c) {
        double d = fabs(orc_e4m3((uint8_t)c) - (double)v);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = c;
        }
    }
    return (uint8_t)best;
}

/* Round r to the nearest E2M1 value (ties to the even code, saturating at +-6):
 * the 4-bit code, with the sign bit only on a non-zero magnitude. */
uint8_t orc_e2m1_round(float r)
{
    double a = fabs((double)r);
    if (a >= 6.0)
        return (uint8_t)(r < 0 ? 15 : 7);
    int best = 0;
    double bd = INFINITY;
    for (int c = 0; c <= 7; ++c) {
        double d = fabs(orc_e2m1((uint8_t)c) - a);
        if (d < bd || (d == bd && (c & 1) == 0 && (best & 1) == 1)) {
            bd = d;
            best = c;
        }
    }
    if (best != 0 && r < 0)
        best |= 8;
    return (uint8_t)best;
}

/* fp32 weights w[n][k] -> one canonical NVFP4 tensor (orc_tensor_bytes bytes).
 * fp32 arithmetic, in this order:
 *   A   = max |w| over the tensor;  s_t = A / 2688 (6 * 448), or 1 if A = 0
 *   per block of 16:  a = max |w|;  s8 = E4M3 rounding of (a / 6) / s_t
 *                     S = E4M3(s8) * s_t
 *                     code = 0 where S = 0, else E2M1 rounding of w / S */
int orc_nvfp4_quantize(const float *w, int64_t n, int64_t k, uint8_t *out)
{
    if (n <= 0 || k <= 0 || (k % 32) != 0)
        return 1;
    float A = 0.0f;
    for (int64_t i = 0; i < n * k; ++i)
        if (fabsf(w[i]) > A)
            A = fabsf(w[i]);
    const float st = A > 0.0f ? A / 2688.0f : 1.0f;
#pragma omp parallel for schedule(static)
    for (int64_t r = 0; r < n; ++r) {
        for (int64_t b = 0; b < k / 16; ++b) {
            const float *wb = w + r * k + b * 16;
            uint8_t *blk = out + (r * (k / 16) + b) * 9;
            float a = 0.0f;
            for (int i = 0; i < 16; ++i)
                if (fabsf(wb[i]) > a)
                    a = fabsf(wb[i]);
            const float u = a / 6.0f;
            const float v = u / st;
            const uint8_t s8 = orc_e4m3_round(v);
            const float S = (float)orc_e4m3(s8) * st;
            uint8_t code[16];
            for (int i = 0; i < 16; ++i)
                code[i] = S == 0.0f ? 0 : orc_e2m1_round(wb[i] / S);
            blk[0] = s8;
            for (int j = 0; j < 8; ++j)
                blk[1 + j] = (uint8_t)(code[j] | (code[j + 8] << 4));
        }
    }
    union { uint32_t u; float f; } t;
    t.f = st;
    uint8_t *p = out + n * (k / 16) * 9;
    p[0] = (uint8_t)t.u;
    p[1] = (uint8_t)(t.u >> 8);
    p[2] = (uint8_t)(t.u >> 16);
    p[3] = (uint8_t)(t.u >> 24);
    return 0;
}
