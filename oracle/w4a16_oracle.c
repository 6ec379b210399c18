/*
 * CPU oracle for the W4A16 decode GEMV -- TEST INFRASTRUCTURE ONLY.
 *
 * Only the test suite, the smoke check and the bench's CPU-baseline leg may load this.
 * The product library never links, loads or calls it, and this file shares no code,
 * header, table or constant with the HIP path.
 *
 * What it computes (one thread, float64, no SIMD intrinsics, no reordering):
 *
 *     y[n] = sum_{k=0}^{K-1} q[n,k] * s[n, k / G] * x[k]
 *
 * The local-kimi README (github.1485827954.workers.dev/RightNow-AI/local-kimi), technical-detail section,
 * paragraph on the GEMV rewrite, describes the operation as a true matrix-vector product
 * over packed INT4 weights with 16-bit activations that reduces along K, the axis the
 * packed weights keep contiguous; the grouped-expert form applies the same product to
 * the weights of router-selected experts. The pages print no formula, so the plain
 * definition above is written out here: dequantise each group (q times its scale, exact
 * in float64) and take the float64 dot product with x.
 *
 * Storage (the plainest reading of "packed INT4 weights, reduction axis contiguous";
 * the pages give no further layout):
 *   qweight  uint32[N][K/8]: value k = 8w + i sits in bits [4i, 4i+3] of word w of its
 *            row; the nibble is a two's-complement integer in [-8, 7] (no zero point).
 *   scales   IEEE binary16 bit patterns [N][K/G], one per G-wide K group.
 *   x        bfloat16 bit patterns [K] (the upper half of an IEEE binary32).
 *
 * Alongside y it returns mag[n] = sum_k |q s x|, the per-element tolerance basis
 * |err| <= 1e-3 * mag + 1e-5 that the parity tests apply.
 */
#include <math.h>
#include <stddef.h>
#include <stdint.h>
#include <string.h>

#define ORACLE_OK 0
#define ORACLE_BAD_ARG 1

/* IEEE-754 binary16 -> double, decoded from the bit fields by hand (exact). */
double oracle_f16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);              /* zero or subnormal: frac * 2^-24 */
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + frac), expo - 25); /* (1 + frac/1024) * 2^(expo-15) */
    }
    return sign ? -v : v;
}

/* bfloat16 -> double: sign, 8-bit exponent (bias 127), 7-bit fraction (exact). */
double oracle_bf16_to_double(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int expo = (b >> 7) & 0xFF;
    int frac = b & 0x7F;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -133);             /* subnormal: frac/128 * 2^-126 */
    } else if (expo == 255) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + frac), expo - 134);
    }
    return sign ? -v : v;
}

/* Signed 4-bit value number k of a packed row. */
int oracle_nibble(const uint32_t *row, int64_t k)
{
    uint32_t word = row[k / 8];
    int u = (int)((word >> (4 * (k % 8))) & 0xFu);
    return u >= 8 ? u - 16 : u;
}

/* q_out[N][K] = the signed nibble values of qweight[N][K/8]. */
int oracle_unpack(const uint32_t *qweight, int8_t *q_out, int64_t N, int64_t K)
{
    if (!qweight || !q_out || N < 0 || K < 0 || K % 8)
        return ORACLE_BAD_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            q_out[n * K + k] = (int8_t)oracle_nibble(qweight + n * (K / 8), k);
    return ORACLE_OK;
}

/* One output element: the dequantise-then-dot of row `row` against activation row `x`. */
static void dot_row(const uint32_t *row, const uint16_t *srow, const uint16_t *x,
                    int64_t K, int64_t G, double *y, double *mag)
{
    double acc = 0.0, m = 0.0;
    for (int64_t g = 0; g < K / G; ++g) {
        double s = oracle_f16_to_double(srow[g]);
        for (int64_t k = g * G; k < (g + 1) * G; ++k) {
            double w = (double)oracle_nibble(row, k) * s;   /* exact: 4 x 11 bits */
            double p = w * oracle_bf16_to_double(x[k]);     /* exact: 15 x 8 bits */
            acc += p;
            m += fabs(p);
        }
    }
    *y = acc;
    *mag = m;
}

static int check_dense(const uint32_t *qweight, const uint16_t *scales, const void *x,
                       int64_t N, int64_t K, int32_t G, const int64_t *rows, int64_t n_rows,
                       const double *y, const double *mag)
{
    if (!qweight || !scales || !x || !y || !mag)
        return ORACLE_BAD_ARG;
    if (N < 1 || K < 1 || G < 8 || G % 8 || K % G || n_rows < 0)
        return ORACLE_BAD_ARG;
    if (rows)
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= N)
                return ORACLE_BAD_ARG;
    return ORACLE_OK;
}

/*
 * y[r], mag[r] for the rows listed in rows[0..n_rows) (rows == NULL: all N rows, and
 * n_rows must be N). Lets the tests check sampled rows of full-size matrices.
 */
int oracle_gemv(const uint32_t *qweight, const uint16_t *scales, const uint16_t *x,
                int64_t N, int64_t K, int32_t G, const int64_t *rows, int64_t n_rows,
                double *y, double *mag)
{
    if (check_dense(qweight, scales, x, N, K, G, rows, n_rows, y, mag))
        return ORACLE_BAD_ARG;
    if (!rows && n_rows != N)
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t n = rows ? rows[r] : r;
        dot_row(qweight + n * (K / 8), scales + n * (K / G), x, K, G, &y[r], &mag[r]);
    }
    return ORACLE_OK;
}

/*
 * Batched form: Y[m][r] for activation rows X[m] (row stride ldx elements), m < M.
 * Output layout [M][n_rows], row-major.
 */
int oracle_gemv_batched(const uint32_t *qweight, const uint16_t *scales,
                        const uint16_t *X, int64_t ldx, int32_t M, int64_t N, int64_t K,
                        int32_t G, const int64_t *rows, int64_t n_rows, double *Y, double *mag)
{
    if (check_dense(qweight, scales, X, N, K, G, rows, n_rows, Y, mag))
        return ORACLE_BAD_ARG;
    if (M < 1 || ldx < K || (!rows && n_rows != N))
        return ORACLE_BAD_ARG;
    for (int32_t m = 0; m < M; ++m)
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t n = rows ? rows[r] : r;
            dot_row(qweight + n * (K / 8), scales + n * (K / G), X + m * ldx, K, G,
                    &Y[m * n_rows + r], &mag[m * n_rows + r]);
        }
    return ORACLE_OK;
}

/*
 * Grouped-expert form: y[t][r] is the product of expert ids[t]'s weights with x.
 * qweight uint32[E][N][K/8], scales fp16 bits [E][N][K/G]. An id outside [0, E) names
 * no expert; its output row is defined as zero (with mag zero).
 */
int oracle_moe_gemv(const uint32_t *qweight, const uint16_t *scales, const int32_t *ids,
                    int32_t topk, int32_t E, const uint16_t *x, int64_t N, int64_t K,
                    int32_t G, const int64_t *rows, int64_t n_rows, double *y, double *mag)
{
    if (check_dense(qweight, scales, x, N, K, G, rows, n_rows, y, mag))
        return ORACLE_BAD_ARG;
    if (!ids || topk < 1 || E < 1 || (!rows && n_rows != N))
        return ORACLE_BAD_ARG;
    for (int32_t t = 0; t < topk; ++t) {
        int32_t e = ids[t];
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t n = rows ? rows[r] : r;
            double *yo = &y[(int64_t)t * n_rows + r], *mo = &mag[(int64_t)t * n_rows + r];
            if (e < 0 || e >= E) {
                *yo = 0.0;
                *mo = 0.0;
                continue;
            }
            const uint32_t *wq = qweight + ((int64_t)e * N + n) * (K / 8);
            const uint16_t *ws = scales + ((int64_t)e * N + n) * (K / G);
            dot_row(wq, ws, x, K, G, yo, mo);
        }
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------
 * The expert tail after the grouped gate+up product (the local-kimi README, technical-detail
 * section, names a SwiGLU variant of the grouped kernel beside the plain one; the pages do not
 * define it further). Readings taken here:
 *   - an expert's gate+up weights hold 2I rows: rows [0, I) are the gate projection, rows
 *     [I, 2I) the up projection;
 *   - SwiGLU is h = silu(g) * u with silu(g) = g / (1 + e^-g);
 *   - h is an activation, so it is stored as bfloat16 (round to nearest, ties to even) before
 *     the down projection consumes it;
 *   - the down projection of slot t uses expert ids[t]'s weights on h[t], and the slots are
 *     summed with the router's weights w[t]: out = sum_t w[t] * W_down[ids[t]] h[t].
 * ------------------------------------------------------------------------------------------ */

/* double -> bfloat16 bit pattern, round to nearest with ties to even, decided in double. */
uint16_t oracle_double_to_bf16(double v)
{
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7FC0u);
    if (isinf(a))
        return (uint16_t)(sign | 0x7F80u);
    if (a == 0.0)
        return sign;
    /* Spacing of bfloat16 values around a: 2^(e-7) for a normal a in [2^e, 2^(e+1)),
     * 2^-133 below the smallest normal 2^-126. */
    int ex;
    frexp(a, &ex);                     /* a = m * 2^ex, m in [0.5, 1): leading bit 2^(ex-1) */
    int qexp = ex - 1 - 7;
    if (qexp < -133)
        qexp = -133;
    double r = rint(ldexp(a, -qexp));  /* default rounding mode: nearest, ties to even */
    double q = ldexp(r, qexp);
    if (q >= ldexp(1.0, 128))
        return (uint16_t)(sign | 0x7F80u);
    float f = (float)q;                /* exact: at most 8 significant bits, in float range */
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    return (uint16_t)(sign | (uint16_t)((bits >> 16) & 0x7FFFu));
}

double oracle_silu(double g) { return g / (1.0 + exp(-g)); }

/*
 * Grouped gate+up product with the SwiGLU epilogue, all I outputs of every slot:
 *   g = W_e[n] x, u = W_e[I + n] x (e = ids[t]), h = silu(g) * u,
 * written as [topk][I] arrays: h (double), h_bf16 (its rounded bits), g, u and the tolerance
 * bases mag_g = sum|q s x| over the gate row and mag_u over the up row. An id outside [0, E)
 * gives zeros everywhere.
 */
int oracle_moe_swiglu(const uint32_t *qweight, const uint16_t *scales, const int32_t *ids,
                      int32_t topk, int32_t E, const uint16_t *x, int64_t I, int64_t K,
                      int32_t G, double *h, uint16_t *h_bf16, double *g, double *u,
                      double *mag_g, double *mag_u)
{
    if (!qweight || !scales || !ids || !x || !h || !h_bf16 || !g || !u || !mag_g || !mag_u)
        return ORACLE_BAD_ARG;
    if (topk < 1 || E < 1 || I < 1 || K < 1 || G < 8 || G % 8 || K % G)
        return ORACLE_BAD_ARG;
    for (int32_t t = 0; t < topk; ++t) {
        int32_t e = ids[t];
        for (int64_t n = 0; n < I; ++n) {
            int64_t o = (int64_t)t * I + n;
            if (e < 0 || e >= E) {
                h[o] = g[o] = u[o] = mag_g[o] = mag_u[o] = 0.0;
                h_bf16[o] = 0;
                continue;
            }
            int64_t rg = (int64_t)e * 2 * I + n, ru = rg + I;
            dot_row(qweight + rg * (K / 8), scales + rg * (K / G), x, K, G, &g[o], &mag_g[o]);
            dot_row(qweight + ru * (K / 8), scales + ru * (K / G), x, K, G, &u[o], &mag_u[o]);
            h[o] = oracle_silu(g[o]) * u[o];
            h_bf16[o] = oracle_double_to_bf16(h[o]);
        }
    }
    return ORACLE_OK;
}

/*
 * Down projection of every slot's own activation row and the router-weighted sum:
 *   out[r] = sum_t w[t] * sum_k q_e[n,k] s_e[n, k/G] h[t][k],  e = ids[t], n = rows[r],
 * qweight uint32[E][H][I/8], scales fp16 bits [E][H][I/G], h bf16 bits [topk][I],
 * w float[topk]. Slots whose id is outside [0, E) contribute nothing. mag[r] is
 * sum_t |w[t]| * sum_k |q s h|.
 */
int oracle_moe_down_combine(const uint32_t *qweight, const uint16_t *scales, const int32_t *ids,
                            const float *w, int32_t topk, int32_t E, const uint16_t *h,
                            int64_t H, int64_t I, int32_t G, const int64_t *rows,
                            int64_t n_rows, double *out, double *mag)
{
    if (check_dense(qweight, scales, h, H, I, G, rows, n_rows, out, mag))
        return ORACLE_BAD_ARG;
    if (!ids || !w || topk < 1 || E < 1 || (!rows && n_rows != H))
        return ORACLE_BAD_ARG;
    for (int64_t r = 0; r < n_rows; ++r) {
        int64_t n = rows ? rows[r] : r;
        double acc = 0.0, m = 0.0;
        for (int32_t t = 0; t < topk; ++t) {
            int32_t e = ids[t];
            if (e < 0 || e >= E)
                continue;
            double y, ym;
            int64_t row = (int64_t)e * H + n;
            dot_row(qweight + row * (I / 8), scales + row * (I / G), h + (int64_t)t * I, I, G,
                    &y, &ym);
            acc += (double)w[t] * y;
            m += fabs((double)w[t]) * ym;
        }
        out[r] = acc;
        mag[r] = m;
    }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------
 * The step before the path: turning bf16 weights into the packed format. The pages say only
 * that the INT4 artifact was built from the bf16 checkpoint ("selective INT4"); the method is
 * this library's reading, the plainest symmetric round-to-nearest scheme for the format:
 *   per row n and 128-wide group g:  amax = max |w|,  s = fp16(amax / 7)  (float32 division,
 *   round to nearest even; a result beyond the largest finite fp16 saturates to 65504),
 *   q = clamp(rint(w / s), -8, 7) with w / s a float32 division and rint ties-to-even,
 *   and q = 0 for the whole group when s is zero.
 * Every decision is taken in float32, as the definition states, so the codes and scales are
 * exact targets for any implementation of it.
 * ------------------------------------------------------------------------------------------ */

/* float -> IEEE binary16 bit pattern, round to nearest even; values beyond the largest finite
 * binary16 saturate to +-65504 (0x7BFF). NaN gives a quiet NaN. */
uint16_t oracle_float_to_f16_sat(float f)
{
    double v = (double)f;      /* exact */
    uint16_t sign = signbit(v) ? 0x8000u : 0u;
    double a = fabs(v);
    if (isnan(v))
        return (uint16_t)(sign | 0x7E00u);
    if (a == 0.0)
        return sign;
    int ex;
    frexp(a, &ex);                     /* leading bit 2^(ex-1) */
    int qexp = ex - 1 - 10;            /* spacing of binary16 values: 2^(e-10), e >= -14 */
    if (qexp < -24)
        qexp = -24;                    /* subnormal spacing 2^-24 */
    double r = rint(ldexp(a, -qexp));  /* nearest, ties to even */
    double q = ldexp(r, qexp);
    if (q > 65504.0)
        return (uint16_t)(sign | 0x7BFFu);
    /* encode q (exactly representable) */
    if (q < ldexp(1.0, -14))
        return (uint16_t)(sign | (uint16_t)rint(ldexp(q, 24)));      /* subnormal or zero */
    frexp(q, &ex);
    int e = ex - 1;                                                    /* q = m * 2^e, m in [1,2) */
    int frac = (int)rint(ldexp(q, 10 - e)) - 1024;
    return (uint16_t)(sign | (uint16_t)((e + 15) << 10) | (uint16_t)frac);
}

/* The float32 value of a bf16 pattern (exact). */
static float bf16_to_float(uint16_t b)
{
    uint32_t bits = (uint32_t)b << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/*
 * Quantise and pack w (bf16 bits, N rows of stride ldw elements, K values each) into
 * qweight uint32[N][K/8] (value k in bits [4(k%8), 4(k%8)+3] of word k/8, two's complement) and
 * scales fp16 bits [N][K/G]. K % G == 0, G % 8 == 0.
 */
int oracle_quantize_pack(const uint16_t *w, int64_t ldw, int64_t N, int64_t K, int32_t G,
                         uint32_t *qweight, uint16_t *scales)
{
    if (!w || !qweight || !scales || N < 1 || K < 1 || G < 8 || G % 8 || K % G || ldw < K)
        return ORACLE_BAD_ARG;
    for (int64_t n = 0; n < N; ++n) {
        const uint16_t *row = w + n * ldw;
        for (int64_t g = 0; g < K / G; ++g) {
            float amax = 0.0f;
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                float a = fabsf(bf16_to_float(row[k]));
                if (a > amax)
                    amax = a;
            }
            volatile float s32 = amax / 7.0f;            /* one float32 division */
            uint16_t sbits = oracle_float_to_f16_sat(s32);
            scales[n * (K / G) + g] = sbits;
            float s = (float)oracle_f16_to_double(sbits);
            for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                int q = 0;
                if (s != 0.0f) {
                    volatile float r = bf16_to_float(row[k]) / s;   /* one float32 division */
                    float qi = rintf(r);
                    q = qi < -8.0f ? -8 : (qi > 7.0f ? 7 : (int)qi);
                }
                uint32_t *word = &qweight[n * (K / 8) + k / 8];
                uint32_t nib = (uint32_t)q & 0xFu;
                int shift = 4 * (int)(k % 8);
                *word = (*word & ~(0xFu << shift)) | (nib << shift);
            }
        }
    }
    return ORACLE_OK;
}

/*
 * Grouped-expert form for M tokens at once, each with its own topk experts:
 *   Y[m][t][r] = sum_k q_e[n,k] s_e[n, k/G] X[m][k],  e = ids[m * topk + t], n = rows[r],
 * qweight uint32[E][N][K/8], scales fp16 bits [E][N][K/G], ids int32[M][topk], X bf16 bits
 * [M][ldx]; Y and mag are [M][topk][n_rows]. An id outside [0, E) gives zeros. (How a kernel
 * shares one expert's weights between the tokens that chose it does not change the result.)
 */
int oracle_moe_gemv_batched(const uint32_t *qweight, const uint16_t *scales, const int32_t *ids,
                            int32_t M, int32_t topk, int32_t E, const uint16_t *X, int64_t ldx,
                            int64_t N, int64_t K, int32_t G, const int64_t *rows, int64_t n_rows,
                            double *Y, double *mag)
{
    if (check_dense(qweight, scales, X, N, K, G, rows, n_rows, Y, mag))
        return ORACLE_BAD_ARG;
    if (!ids || M < 1 || topk < 1 || E < 1 || ldx < K || (!rows && n_rows != N))
        return ORACLE_BAD_ARG;
    for (int32_t m = 0; m < M; ++m)
        for (int32_t t = 0; t < topk; ++t) {
            int32_t e = ids[(int64_t)m * topk + t];
            for (int64_t r = 0; r < n_rows; ++r) {
                int64_t n = rows ? rows[r] : r;
                int64_t o = ((int64_t)m * topk + t) * n_rows + r;
                if (e < 0 || e >= E) {
                    Y[o] = 0.0;
                    mag[o] = 0.0;
                    continue;
                }
                int64_t row = (int64_t)e * N + n;
                dot_row(qweight + row * (K / 8), scales + row * (K / G), X + m * ldx, K, G,
                        &Y[o], &mag[o]);
            }
        }
    return ORACLE_OK;
}

/* ------------------------------------------------------------------------------------------
 * Three-bit expert weights. The local-kimi README's hardware section says that fitting a
 * 24 GB card needs the expert weights near three bits and that the work is under way; the
 * pages define no format. The reading taken here keeps everything of the INT4 format except
 * the code width:
 *   - a code is a 3-bit two's-complement integer q in [-4, 3] (no zero point), scaled by the
 *     same fp16 scale per G-wide K group;
 *   - a row of K values is K/32 blocks of three uint32 words (12 bytes, 32 codes); in block b,
 *     code c (value k = 32 b + c) sits
 *       c = 10 t + j,     t in {0,1,2}, j in 0..4:  bits [3j, 3j+2]       of word t,
 *       c = 10 t + 5 + j, t in {0,1,2}, j in 0..4:  bits [16+3j, 16+3j+2] of word t,
 *       c = 30:  its bit i is bit 15 of word i,  i = 0, 1, 2,
 *       c = 31:  its bit i is bit 31 of word i;
 *   - qweight3 uint32[E][N][3K/32] (experts, then rows, then blocks), scales fp16 [E][N][K/G].
 * 3 bits per weight plus 16 bits per group: 0.390625 bytes per weight at G = 128.
 * ---------------------------------------------------------------------------------------- */

/* Code c (0..31) of one 3-word block, as a signed integer. */
static int code3_of_block(const uint32_t *blk, int c)
{
    unsigned u;
    if (c < 30) {
        int t = c / 10, r = c % 10;
        int shift = r < 5 ? 3 * r : 16 + 3 * (r - 5);
        u = (blk[t] >> shift) & 7u;
    } else {
        int bit = c == 30 ? 15 : 31;
        u = ((blk[0] >> bit) & 1u) | (((blk[1] >> bit) & 1u) << 1) | (((blk[2] >> bit) & 1u) << 2);
    }
    return u >= 4 ? (int)u - 8 : (int)u;
}

/* Signed codes of N rows of K values: q_out int8[N][K]. */
int oracle_unpack3(const uint32_t *qweight3, int8_t *q_out, int64_t N, int64_t K)
{
    if (!qweight3 || !q_out || N < 1 || K < 32 || K % 32)
        return ORACLE_BAD_ARG;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            q_out[n * K + k] = (int8_t)code3_of_block(qweight3 + n * (3 * K / 32) + 3 * (k / 32),
                                                     (int)(k % 32));
    return ORACLE_OK;
}

static void dot_row3(const uint32_t *row, const uint16_t *srow, const uint16_t *x, int64_t K,
                     int32_t G, double *y, double *mag)
{
    double acc = 0.0, m = 0.0;
    for (int64_t g = 0; g < K / G; ++g) {
        double s = oracle_f16_to_double(srow[g]);
        for (int64_t k = g * G; k < (g + 1) * G; ++k) {
            double w = (double)code3_of_block(row + 3 * (k / 32), (int)(k % 32)) * s;
            double p = w * oracle_bf16_to_double(x[k]);
            acc += p;
            m += fabs(p);
        }
    }
    *y = acc;
    *mag = m;
}

/*
 * Grouped-expert product over three-bit experts: y[t][r] = sum_k q3_e[n,k] s_e[n,k/G] x[k],
 * e = ids[t], n = rows[r]. An id outside [0, E) gives a zero row (with mag zero).
 */
int oracle_moe_gemv3(const uint32_t *qweight3, const uint16_t *scales, const int32_t *ids,
                     int32_t topk, int32_t E, const uint16_t *x, int64_t N, int64_t K,
                     int32_t G, const int64_t *rows, int64_t n_rows, double *y, double *mag)
{
    if (!qweight3 || !scales || !ids || !x || !y || !mag)
        return ORACLE_BAD_ARG;
    if (topk < 1 || E < 1 || N < 1 || K < 32 || K % 32 || G < 32 || G % 32 || K % G ||
        n_rows < 0 || (!rows && n_rows != N))
        return ORACLE_BAD_ARG;
    if (rows)
        for (int64_t r = 0; r < n_rows; ++r)
            if (rows[r] < 0 || rows[r] >= N)
                return ORACLE_BAD_ARG;
    for (int32_t t = 0; t < topk; ++t) {
        int32_t e = ids[t];
        for (int64_t r = 0; r < n_rows; ++r) {
            int64_t n = rows ? rows[r] : r;
            double *yo = &y[(int64_t)t * n_rows + r], *mo = &mag[(int64_t)t * n_rows + r];
            if (e < 0 || e >= E) {
                *yo = 0.0;
                *mo = 0.0;
                continue;
            }
            int64_t row = (int64_t)e * N + n;
            dot_row3(qweight3 + row * (3 * K / 32), scales + row * (K / G), x, K, G, yo, mo);
        }
    }
    return ORACLE_OK;
}
