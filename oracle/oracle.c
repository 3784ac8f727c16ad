/*
 * oracle.c — plain, slow, obviously correct fp64 reference for the fused
 * dequantize-and-multiply over Q4_K-style weights.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code with
 * the HIP library (no headers, tables or helpers) and the HIP library never
 * calls it.
 *
 * What is computed (the method on the OpenJet multi-agent serving page, section
 * on moving the weights only once: every weight that is read serves all R
 * stacked rows, which changes the order of memory traffic, not the result):
 *
 *   w[n, k] = d * sc_s * q_k - dmin * m_s      (k = 256 j + 32 s + t, block (n, j))
 *   y[r, n] = sum_{k=0}^{K-1} w[n, k] * x[r, k]
 *
 * Steps, each written out plainly:
 *   1. read d, dmin (binary16), the sixteen 6-bit fields and the 256 nibbles of
 *      a 144-byte canonical super-block (byte layout in the generator's header
 *      comment and in the library header);
 *   2. decode binary16 and bfloat16 from their IEEE-754 / bfloat16 definitions
 *      into double (exact);
 *   3. form w in double.  d*sc*q has at most 21 significant bits and dmin*m at
 *      most 17, so both products are exact; their difference is exact when the
 *      two values' bits span at most 53 positions, which is checked for every
 *      block (error ORACLE_EINEXACT otherwise);
 *   4. y[r, n] accumulated in double in ascending k, one fixed order; threads
 *      split n only, so the result does not depend on the thread count;
 *   5. the fp32 dequantised weight is the double w rounded once to nearest-even
 *      (C's double -> float conversion under the default rounding mode);
 *   6. per-row argmax over y, lowest index on ties.
 *   7. greedy verification of the agents' draft tokens against the argmax rows.
 *
 * Build-time switch ORACLE_MUTANT (default 0) plants one deliberate mistake so
 * that the pin tests can show they would catch it; release builds never set it.
 */
#include <stdint.h>
#include <math.h>
#include <pthread.h>

#ifndef ORACLE_MUTANT
#define ORACLE_MUTANT 0
#endif

enum { ORACLE_OK = 0, ORACLE_EARG = -1, ORACLE_EINEXACT = -2 };

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_f16_to_f64(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -24);                 /* subnormal: f * 2^-24 */
    } else if (e == 31) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(1024 + f), e - 25);     /* (1 + f/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double oracle_bf16_to_f64(uint16_t b)
{
    int sign = (b >> 15) & 1;
    int e = (b >> 7) & 0xFF;
    int f = b & 0x7F;
    double v;
    if (e == 0) {
        v = ldexp((double)f, -133);                /* f * 2^-126 / 128 */
    } else if (e == 255) {
        v = f ? NAN : INFINITY;
    } else {
        v = ldexp((double)(128 + f), e - 134);     /* (1 + f/128) * 2^(e-127) */
    }
    return sign ? -v : v;
}

/* six-bit field number f of the 96-bit little-endian stream at p */
static unsigned field6(const uint8_t *p, int f)
{
    unsigned v = 0;
    for (int i = 0; i < 6; i++) {
        int bit = 6 * f + i;
        v |= (unsigned)((p[bit / 8] >> (bit % 8)) & 1) << i;
    }
    return v;
}

/* the span (in bit positions) of the nonzero finite value a, which has at most
 * `sig` significant bits: returns floor(log2|a|) in *hi and the exponent of
 * its lowest possible bit in *lo */
static void bit_range(double a, int sig, int *hi, int *lo)
{
    int e;
    frexp(a, &e);
    *hi = e - 1;
    *lo = e - sig;
}

/* Dequantise one canonical super-block into w[256] (double, exact). */
int oracle_dequant_block(const uint8_t *sb, double *w)
{
    double d = oracle_f16_to_f64((uint16_t)(sb[0] | (sb[1] << 8)));
    double dmin = oracle_f16_to_f64((uint16_t)(sb[2] | (sb[3] << 8)));
    for (int s = 0; s < 8; s++) {
        double sc = (double)field6(sb + 4, s);
        double m = (double)field6(sb + 4, 8 + s);
#if ORACLE_MUTANT == 4
        { double t = sc; sc = m; m = t; }           /* mutant: scale and min swapped */
#endif
        for (int t = 0; t < 32; t++) {
            int k = 32 * s + t;
            int byte = sb[16 + k / 2];
            int q = (k % 2 == 0) ? (byte & 0xF) : (byte >> 4);
#if ORACLE_MUTANT == 3
            q = (k % 2 == 0) ? (byte >> 4) : (byte & 0xF);   /* mutant: nibble order */
#endif
            double a = d * sc * (double)q;
            double b = dmin * m;
#if ORACLE_MUTANT == 1
            b = 0.0;                                         /* mutant: min term dropped */
#endif
            if (a != 0.0 && b != 0.0) {
                int ha, la, hb, lb;
                bit_range(a, 21, &ha, &la);
                bit_range(b, 17, &hb, &lb);
                int hi = ha > hb ? ha : hb, lo = la < lb ? la : lb;
                if (hi - lo + 1 > 53) return ORACLE_EINEXACT;
            }
#if ORACLE_MUTANT == 2
            w[k] = a + b;                                    /* mutant: wrong sign */
#else
            w[k] = a - b;
#endif
        }
    }
    return ORACLE_OK;
}

/* Rows [n0, n1) of the N x K matrix, as doubles, into w[(n1-n0) * K]. */
int oracle_dequant(const uint8_t *canon, int64_t N, int64_t K, int64_t n0, int64_t n1,
                   double *w)
{
    if (!canon || !w || K <= 0 || K % 256 || n0 < 0 || n1 > N || n0 > n1) return ORACLE_EARG;
    int64_t KB = K / 256;
    for (int64_t n = n0; n < n1; n++)
        for (int64_t j = 0; j < KB; j++) {
            int rc = oracle_dequant_block(canon + (n * KB + j) * 144, w + (n - n0) * K + j * 256);
            if (rc) return rc;
        }
    return ORACLE_OK;
}

/* Same, rounded once to float (nearest-even). */
int oracle_dequant_f32(const uint8_t *canon, int64_t N, int64_t K, int64_t n0, int64_t n1,
                       float *w)
{
    if (!canon || !w || K <= 0 || K % 256 || n0 < 0 || n1 > N || n0 > n1) return ORACLE_EARG;
    int64_t KB = K / 256;
    double blk[256];
    for (int64_t n = n0; n < n1; n++)
        for (int64_t j = 0; j < KB; j++) {
            int rc = oracle_dequant_block(canon + (n * KB + j) * 144, blk);
            if (rc) return rc;
            for (int i = 0; i < 256; i++) w[(n - n0) * K + j * 256 + i] = (float)blk[i];
        }
    return ORACLE_OK;
}

typedef struct {
    const uint8_t *canon;
    int64_t N, K, R, n0, n1;
    const uint16_t *x;
    double *y;
    int rc;
} gjob;

static void *gemm_rows(void *p)
{
    gjob *g = (gjob *)p;
    int64_t K = g->K, KB = K / 256, N = g->N;
    double wrow[256];
    for (int64_t n = g->n0; n < g->n1; n++) {
        for (int64_t r = 0; r < g->R; r++) g->y[r * N + n] = 0.0;
        for (int64_t j = 0; j < KB; j++) {
            int rc = oracle_dequant_block(g->canon + (n * KB + j) * 144, wrow);
            if (rc) { g->rc = rc; return 0; }
            for (int64_t r = 0; r < g->R; r++) {
                double acc = g->y[r * N + n];
                for (int i = 0; i < 256; i++) {
#if ORACLE_MUTANT == 5
                    double xv = oracle_bf16_to_f64(g->x[r * K + (K - 1 - (j * 256 + i))]); /* mutant: k reversed */
#else
                    double xv = oracle_bf16_to_f64(g->x[r * K + j * 256 + i]);
#endif
                    acc += wrow[i] * xv;
                }
                g->y[r * N + n] = acc;
            }
        }
    }
    return 0;
}

/* y[R x N] (row-major, double) = W[N x K] . x[R x K]^T, x given as bf16 bits.
 * Summation per (r, n) runs over k = 0, 1, ..., K-1 in that order. */
int oracle_gemm(const uint8_t *canon, int64_t N, int64_t K, const uint16_t *x, int64_t R,
                double *y, int nthreads)
{
    if (!canon || !x || !y || N < 0 || K <= 0 || K % 256 || R < 0) return ORACLE_EARG;
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads > N) nthreads = N > 0 ? (int)N : 1;
    pthread_t th[256];
    gjob jobs[256];
    for (int t = 0; t < nthreads; t++)
        jobs[t] = (gjob){canon, N, K, R, N * t / nthreads, N * (t + 1) / nthreads, x, y, 0};
    for (int t = 1; t < nthreads; t++) pthread_create(&th[t], 0, gemm_rows, &jobs[t]);
    gemm_rows(&jobs[0]);
    for (int t = 1; t < nthreads; t++) pthread_join(th[t], 0);
    for (int t = 0; t < nthreads; t++)
        if (jobs[t].rc) return jobs[t].rc;
    return ORACLE_OK;
}

/* 7. Greedy verification of the draft tokens of each agent.  Agent a owns rows
 * a (D + 1) .. a (D + 1) + D of the pass: its current token, then its D draft
 * tokens drafts[a D + i] (OpenJet multi-agent serving page, section on moving
 * the weights only once: every agent contributes its next token plus drafts,
 * and the drafts are checked in the same round).  Row i's argmax p_i is the
 * model's choice for the position after row i's input, so draft i (the input of
 * row i + 1) stands iff it equals p_i, and p_{i+1} is then valid too.  The agent
 * emits p_0, then p_{i+1} for each draft accepted in order, stopping at the
 * first rejected one: n_new[a] = 1 + (number of drafts accepted); tokens[a (D +
 * 1) + j] holds the j-th emitted token, -1 past n_new[a]. */
int oracle_verify_greedy(const int32_t *argmax, int64_t R, const int32_t *drafts, int64_t D,
                         int32_t *tokens, int32_t *n_new)
{
    if (!argmax || !tokens || !n_new || D < 0 || R < 0 || R % (D + 1) != 0) return ORACLE_EARG;
    if (D > 0 && !drafts) return ORACLE_EARG;
    const int64_t A = R / (D + 1);
    for (int64_t a = 0; a < A; a++) {
        const int64_t base = a * (D + 1);
        for (int64_t j = 0; j <= D; j++) tokens[base + j] = -1;
        int64_t n = 0;
        tokens[base + n++] = argmax[base];
        for (int64_t i = 0; i < D; i++) {
#if ORACLE_MUTANT == 6
            if (argmax[base + i + 1] != drafts[a * D + i]) break;     /* mutant: checked against the wrong row */
#else
            if (argmax[base + i] != drafts[a * D + i]) break;
#endif
            tokens[base + n++] = argmax[base + i + 1];
        }
#if ORACLE_MUTANT == 7
        /* mutant: a rejected draft does not stop the later ones */
        n = 1;
        for (int64_t j = 1; j <= D; j++) tokens[base + j] = -1;
        for (int64_t i = 0; i < D; i++)
            if (argmax[base + i] == drafts[a * D + i]) tokens[base + n++] = argmax[base + i + 1];
#endif
        n_new[a] = (int32_t)n;
    }
    return ORACLE_OK;
}

/* idx[r] = the smallest n with y[r, n] == max_n y[r, n]. */
int oracle_argmax_rows(const double *y, int64_t R, int64_t N, int32_t *idx)
{
    if (!y || !idx || R < 0 || N < 1) return ORACLE_EARG;
    for (int64_t r = 0; r < R; r++) {
        int64_t best = 0;
        for (int64_t n = 1; n < N; n++)
            if (y[r * N + n] > y[r * N + best]) best = n;
        idx[r] = (int32_t)best;
    }
    return ORACLE_OK;
}
