/*
 * CPU oracle for the affine group-quantized matrix product.
 *
 * TEST INFRASTRUCTURE ONLY. Nothing in the product path may call, link or
 * load this file; only the tests, the smoke check and the benchmark's CPU
 * baseline leg use it. It shares no code with the GPU library.
 *
 * What it computes (plain definitions, fp64 throughout, no blocking, no
 * fusion, no reordering):
 *
 *   code    q[n,k]   = bits [k*b, k*b+b) of row n's bitstream, where stream
 *                      bit t is bit (t mod 32) of word t/32 (least
 *                      significant bit first).
 *   weight  w[n,k]   = s[n, k/G] * q[n,k] + b[n, k/G]
 *           (x, s and b are fp16, or all three bf16 in the _ex entry points)
 *   output  y[m,n]   = sum over k = 0..K-1, ascending, of w[n,k] * x[m,k]
 *   bound   A[m,n]   = sum over k of |w[n,k] * x[m,k]|
 *
 * The affine form w = s*q + b and its factored evaluation
 * C += s*P + b*XS (P = codes . x over a group, XS = sum of x over the group)
 * are stated in the vmlx-swift pull request #565 page, commit "LaneQMM"
 * (Metal 4 tensor-ops matmul over raw affine codes with the dequantization
 * applied after the dot product). The 4-bit/group-32, 4-bit/group-64 and
 * 8-bit formats are those listed as consumed as stored in the
 * "Qwen3.8 Flash Next performance and parity receipt" page, section
 * "MTPLX logic review". Bit order, the scale/bias layout and the weight
 * orientation are not fixed by the pages; the readings used here are the
 * plainest ones (least-significant-bit-first stream per output row,
 * separate [N, K/G] fp16 scale and bias arrays, weights stored [N, K] so
 * that y = x . W^T).
 *
 * Parity pins for every function here live in the CPU test suite
 * (closed forms, exhaustive brute force, library routines and invariants).
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---------------------------------------------------------------------
 * IEEE 754 binary16 -> double (exact). A half has 1 sign bit, 5 exponent
 * bits (bias 15) and 10 fraction bits; exponent 0 encodes zero and
 * subnormals (fraction * 2^-24), exponent 31 encodes inf and NaN.
 * ------------------------------------------------------------------- */
double qo_half_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -24);
    else if (expo == 31)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + frac), expo - 25);
    return sign ? -v : v;
}

void qo_half_array_to_double(const uint16_t *h, double *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = qo_half_to_double(h[i]);
}

/* ---------------------------------------------------------------------
 * bfloat16 -> double (exact). A bfloat16 is the upper half of an IEEE 754
 * binary32: 1 sign bit, 8 exponent bits (bias 127) and 7 fraction bits;
 * exponent 0 encodes zero and subnormals (fraction * 2^-133), exponent 255
 * encodes inf and NaN.
 * ------------------------------------------------------------------- */
double qo_bf16_to_double(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 7) & 0xff;
    int frac = h & 0x7f;
    double v;
    if (expo == 0)
        v = ldexp((double)frac, -133);
    else if (expo == 255)
        v = frac ? NAN : INFINITY;
    else
        v = ldexp((double)(128 + frac), expo - 134);
    return sign ? -v : v;
}

/* Operand types of x, scales and biases. */
enum { QO_F16 = 0, QO_BF16 = 1 };

static double decode(int dtype, uint16_t h)
{
    return dtype == QO_BF16 ? qo_bf16_to_double(h) : qo_half_to_double(h);
}

static void decode_array(int dtype, const uint16_t *h, double *out, int64_t count)
{
    for (int64_t i = 0; i < count; ++i)
        out[i] = decode(dtype, h[i]);
}

/* ---------------------------------------------------------------------
 * Packing. Row n of `codes` (K codes, only the low `bits` bits of each are
 * used) becomes K*bits/32 words. Code k occupies stream bits
 * k*bits .. k*bits+bits-1, least significant bit first; stream bit t is
 * bit (t mod 32) of word t/32 of the row.
 * ------------------------------------------------------------------- */
static int stream_bit(const uint32_t *row, int64_t t)
{
    return (int)((row[t / 32] >> (t % 32)) & 1u);
}

static uint32_t read_code(const uint32_t *row, int64_t k, int bits)
{
    uint32_t c = 0;
    for (int j = 0; j < bits; ++j)
        c |= (uint32_t)stream_bit(row, k * bits + j) << j;
    return c;
}

int qo_pack(const uint8_t *codes, uint32_t *words, int64_t N, int64_t K, int bits)
{
    if (bits < 1 || bits > 8 || N < 0 || K < 0 || (K * bits) % 32)
        return -1;
    int64_t W = K * bits / 32;
    for (int64_t n = 0; n < N; ++n) {
        uint32_t *row = words + n * W;
        memset(row, 0, (size_t)W * sizeof(uint32_t));
        for (int64_t k = 0; k < K; ++k) {
            uint32_t c = codes[n * K + k];
            for (int j = 0; j < bits; ++j) {
                int64_t t = k * bits + j;
                row[t / 32] |= ((c >> j) & 1u) << (t % 32);
            }
        }
    }
    return 0;
}

int qo_unpack(const uint32_t *words, uint8_t *codes, int64_t N, int64_t K, int bits)
{
    if (bits < 1 || bits > 8 || N < 0 || K < 0 || (K * bits) % 32)
        return -1;
    int64_t W = K * bits / 32;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            codes[n * K + k] = (uint8_t)read_code(words + n * W, k, bits);
    return 0;
}

/* ---------------------------------------------------------------------
 * Forward product, split over output rows n across host threads. The
 * arithmetic of each output element is the same whatever the thread count.
 * ------------------------------------------------------------------- */
struct job {
    const uint16_t *x, *s, *b;
    const uint32_t *words;
    double *y, *absum;
    int64_t M, K, N;
    int bits, G, factored;
    int dtype; /* QO_F16 or QO_BF16: type of x, s and b */
    int64_t n_begin, n_end;
    const int64_t *rows; /* optional list of output rows; y/absum are then [M, nrows] */
    int64_t out_stride;  /* row stride of y/absum: N, or nrows with a list */
};

/* Output row handled at position i of a job, and the column it is stored in. */
static int64_t job_row(const struct job *jb, int64_t i) { return jb->rows ? jb->rows[i] : i; }

/* Dequantize-then-dot: w[n,k] = s*q + b in fp64, then an ascending-k dot. */
static void rows_dequant_dot(const struct job *jb)
{
    const int64_t K = jb->K, M = jb->M, G = jb->G;
    const int64_t Kg = K / G, W = K * jb->bits / 32;
    double *w = (double *)malloc((size_t)K * sizeof(double));
    double *xd = (double *)malloc((size_t)(M * K) * sizeof(double));
    decode_array(jb->dtype, jb->x, xd, M * K);
    for (int64_t i = jb->n_begin; i < jb->n_end; ++i) {
        const int64_t n = job_row(jb, i);
        const uint32_t *row = jb->words + n * W;
        for (int64_t k = 0; k < K; ++k) {
            double q = (double)read_code(row, k, jb->bits);
            double s = decode(jb->dtype, jb->s[n * Kg + k / G]);
            double b = decode(jb->dtype, jb->b[n * Kg + k / G]);
            w[k] = s * q + b;
        }
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0, mag = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = w[k] * xd[m * K + k];
                acc += p;
                mag += fabs(p);
            }
            jb->y[m * jb->out_stride + i] = acc;
            if (jb->absum)
                jb->absum[m * jb->out_stride + i] = mag;
        }
    }
    free(w);
    free(xd);
}

/* The factored form: per group g, P = sum q*x and XS = sum x over the
 * group's k, then y = sum over groups of (s*P + b*XS). fp64. */
static void rows_factored(const struct job *jb)
{
    const int64_t K = jb->K, M = jb->M, G = jb->G;
    const int64_t Kg = K / G, W = K * jb->bits / 32;
    double *xd = (double *)malloc((size_t)(M * K) * sizeof(double));
    decode_array(jb->dtype, jb->x, xd, M * K);
    for (int64_t i = jb->n_begin; i < jb->n_end; ++i) {
        const int64_t n = job_row(jb, i);
        const uint32_t *row = jb->words + n * W;
        for (int64_t m = 0; m < M; ++m) {
            double acc = 0.0;
            for (int64_t g = 0; g < Kg; ++g) {
                double P = 0.0, XS = 0.0;
                for (int64_t k = g * G; k < (g + 1) * G; ++k) {
                    P += (double)read_code(row, k, jb->bits) * xd[m * K + k];
                    XS += xd[m * K + k];
                }
                acc += decode(jb->dtype, jb->s[n * Kg + g]) * P
                     + decode(jb->dtype, jb->b[n * Kg + g]) * XS;
            }
            jb->y[m * jb->out_stride + i] = acc;
        }
    }
    free(xd);
}

static void *run_job(void *arg)
{
    struct job *jb = (struct job *)arg;
    if (jb->factored)
        rows_factored(jb);
    else
        rows_dequant_dot(jb);
    return NULL;
}

static int run_forward(const uint16_t *x, const uint32_t *words, const uint16_t *s,
                       const uint16_t *b, double *y, double *absum, int64_t M,
                       int64_t K, int64_t N, int bits, int G, int nthreads, int factored,
                       const int64_t *rows, int64_t nrows, int dtype)
{
    if (!x || !words || !s || !b || !y)
        return -1;
    if (dtype != QO_F16 && dtype != QO_BF16)
        return -2;
    if (M < 1 || K < 1 || N < 1 || G < 1 || K % G || bits < 1 || bits > 8 || (K * bits) % 32)
        return -2;
    const int64_t count = rows ? nrows : N;
    for (int64_t i = 0; rows && i < nrows; ++i)
        if (rows[i] < 0 || rows[i] >= N)
            return -2;
    if (count < 1)
        return 0;
    if (nthreads < 1)
        nthreads = 1;
    if (nthreads > count)
        nthreads = (int)count;
    struct job *jobs = (struct job *)calloc((size_t)nthreads, sizeof(struct job));
    pthread_t *tids = (pthread_t *)calloc((size_t)nthreads, sizeof(pthread_t));
    for (int t = 0; t < nthreads; ++t) {
        struct job *jb = &jobs[t];
        jb->x = x; jb->s = s; jb->b = b; jb->words = words;
        jb->y = y; jb->absum = absum;
        jb->M = M; jb->K = K; jb->N = N; jb->bits = bits; jb->G = G;
        jb->factored = factored;
        jb->dtype = dtype;
        jb->rows = rows;
        jb->out_stride = count;
        jb->n_begin = count * t / nthreads;
        jb->n_end = count * (t + 1) / nthreads;
    }
    for (int t = 1; t < nthreads; ++t)
        pthread_create(&tids[t], NULL, run_job, &jobs[t]);
    run_job(&jobs[0]);
    for (int t = 1; t < nthreads; ++t)
        pthread_join(tids[t], NULL);
    free(jobs);
    free(tids);
    return 0;
}

int qo_forward(const uint16_t *x, const uint32_t *words, const uint16_t *s, const uint16_t *b,
               double *y, double *absum, int64_t M, int64_t K, int64_t N, int bits, int G,
               int nthreads)
{
    return run_forward(x, words, s, b, y, absum, M, K, N, bits, G, nthreads, 0, NULL, 0, QO_F16);
}

/* qo_forward with x, s and b of type dtype (0 fp16, 1 bf16). */
int qo_forward_ex(const uint16_t *x, const uint32_t *words, const uint16_t *s, const uint16_t *b,
                  double *y, double *absum, int64_t M, int64_t K, int64_t N, int bits, int G,
                  int dtype, int nthreads)
{
    return run_forward(x, words, s, b, y, absum, M, K, N, bits, G, nthreads, 0, NULL, 0, dtype);
}

/* Same as qo_forward for a list of output rows only: y and absum are
 * [M, nrows], column i holding output row rows[i]. */
int qo_forward_rows(const uint16_t *x, const uint32_t *words, const uint16_t *s,
                    const uint16_t *b, double *y, double *absum, int64_t M, int64_t K,
                    int64_t N, int bits, int G, const int64_t *rows, int64_t nrows,
                    int nthreads)
{
    if (!rows)
        return -1;
    return run_forward(x, words, s, b, y, absum, M, K, N, bits, G, nthreads, 0, rows, nrows, QO_F16);
}

int qo_forward_rows_ex(const uint16_t *x, const uint32_t *words, const uint16_t *s,
                       const uint16_t *b, double *y, double *absum, int64_t M, int64_t K,
                       int64_t N, int bits, int G, const int64_t *rows, int64_t nrows,
                       int dtype, int nthreads)
{
    if (!rows)
        return -1;
    return run_forward(x, words, s, b, y, absum, M, K, N, bits, G, nthreads, 0, rows, nrows, dtype);
}

int qo_forward_factored(const uint16_t *x, const uint32_t *words, const uint16_t *s,
                        const uint16_t *b, double *y, int64_t M, int64_t K, int64_t N,
                        int bits, int G, int nthreads)
{
    return run_forward(x, words, s, b, y, NULL, M, K, N, bits, G, nthreads, 1, NULL, 0, QO_F16);
}

/* ---------------------------------------------------------------------
 * Tiled layout (an optional re-layout of the packed weights, defined by
 * this library for its matrix-core path; the vmlx-swift pull request #565
 * page tiles its lane-matmul weights, commit "LaneQMM" and its tiling
 * policy, without printing a layout). Rows come in tiles of 16 (N padded
 * with zero rows). Code k of row n belongs to tile t = n/16, row i = n%16
 * of it, group g = k/G, lane block c = (k mod G)/(G/4), position
 * j = k mod (G/4) in that block's chunk. Lane L = 16c + i of tile t owns a
 * bit stream holding, for g = 0, 1, ..., the chunk c of group g; the code's
 * bits start at stream bit (g*(G/4) + j)*bits. Stream bit p is bit p mod 8 of
 * byte ((t*UB + p/128)*64 + L)*16 + (p mod 128)/8, UB = K*bits/512.
 * Scales and biases become words s | b<<16 (the fp16 bit patterns): row n,
 * group g at word ((t*(K/G)/4 + g/4)*16 + i)*4 + g mod 4.
 * The function scatters every code bit and every (s, b) pair to its place.
 * ------------------------------------------------------------------- */
int qo_repack_tiled(const uint32_t *words, const uint16_t *s, const uint16_t *b, uint8_t *tw,
                    uint32_t *tsb, int64_t N, int64_t K, int bits, int G)
{
    if (bits < 1 || bits > 8 || G < 4 || G % 4 || N < 1 || K < G || K % (4 * G) ||
        (K * bits) % 512)
        return -1;
    const int64_t W = K * bits / 32, Kg = K / G, UB = K * bits / 512;
    const int64_t Np = (N + 15) / 16 * 16;
    memset(tw, 0, (size_t)(Np * K * bits / 8));
    memset(tsb, 0, (size_t)(Np * Kg) * sizeof(uint32_t));
    for (int64_t n = 0; n < N; ++n) {
        const int64_t t = n / 16, i = n % 16;
        for (int64_t k = 0; k < K; ++k) {
            const uint32_t q = read_code(words + n * W, k, bits);
            const int64_t g = k / G, c = (k % G) / (G / 4), j = k % (G / 4);
            const int64_t L = 16 * c + i;
            for (int e = 0; e < bits; ++e) {
                if (!((q >> e) & 1u))
                    continue;
                const int64_t p = (g * (G / 4) + j) * bits + e;
                const int64_t byte = ((t * UB + p / 128) * 64 + L) * 16 + (p % 128) / 8;
                tw[byte] |= (uint8_t)(1u << (p % 8));
            }
        }
        for (int64_t g = 0; g < Kg; ++g)
            tsb[((t * (Kg / 4) + g / 4) * 16 + i) * 4 + g % 4] =
                (uint32_t)s[n * Kg + g] | ((uint32_t)b[n * Kg + g] << 16);
    }
    return 0;
}

