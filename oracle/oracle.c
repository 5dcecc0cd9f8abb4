/*
 * oracle.c -- plain, slow, obviously correct CPU oracle for the q4_K / q6_K x q8
 * prefill matrix multiply.  Declarations, sources and readings: oracle.h.
 *
 * TEST INFRASTRUCTURE ONLY: the product library never includes, links or calls
 * this file.  Build: gcc -O2 -std=c11 -ffp-contract=off -fPIC -shared (no
 * -ffast-math), so every float operation below is one IEEE binary32 operation
 * rounded to nearest-even, exactly as written.
 *
 * Precision: the quantizer works in binary32 because its reading fixes that
 * precision (its decisions are integers and must be reproduced exactly); every
 * term of the result is formed exactly in binary64 (an f16 times a small integer
 * times an f16 times an integer dot never needs more than 53 bits) and summed in
 * binary64.
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------- */
/* binary16                                                                   */
/* ------------------------------------------------------------------------- */

/* IEEE 754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.
 * Exponent field 0 holds zero and the subnormals m * 2^-24; field 31 holds
 * infinity and NaN; otherwise the value is (1024 + m) * 2^(e - 25).          */
double oracle_f16_to_f64(uint16_t h)
{
    const int sign = h >> 15;
    const int e = (h >> 10) & 31;
    const int m = h & 1023;
    double v;
    if (e == 0)
        v = ldexp((double)m, -24);
    else if (e == 31)
        v = m ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + m), e - 25);
    return sign ? -v : v;
}

float oracle_f16_to_f32(uint16_t h) { return (float)oracle_f16_to_f64(h); }

/* Value used for rounding decisions: the non-negative finite codes are ordered
 * like their values; the infinity code stands for 2^16, the first value past
 * the largest finite one (65504) in the unbounded-exponent format, which is how
 * IEEE rounding decides overflow.                                            */
static double f16_rounding_value(uint16_t code)
{
    return code == 0x7c00 ? 65536.0 : oracle_f16_to_f64(code);
}

/* Round to the nearest binary16, ties to the even code (even last fraction bit).
 * Done the plain way: bracket |f| between two adjacent codes by bisection over
 * the ordered codes, then take the nearer one.                               */
uint16_t oracle_f32_to_f16(float f)
{
    if (isnan(f))
        return 0x7e00;
    const uint16_t sign = signbit(f) ? 0x8000 : 0;
    const double a = fabs((double)f);
    if (a >= 65536.0)
        return sign | 0x7c00;
    uint16_t lo = 0, hi = 0x7c00; /* value(lo) <= a < value(hi) */
    while (hi - lo > 1) {
        const uint16_t mid = (uint16_t)((lo + hi) / 2);
        if (f16_rounding_value(mid) <= a)
            lo = mid;
        else
            hi = mid;
    }
    const double below = a - f16_rounding_value(lo);
    const double above = f16_rounding_value(hi) - a;
    uint16_t r;
    if (below < above)
        r = lo;
    else if (above < below)
        r = hi;
    else
        r = (lo & 1) ? hi : lo;
    return sign | r;
}

/* ------------------------------------------------------------------------- */
/* O1 -- weight decode                                                        */
/* ------------------------------------------------------------------------- */

/* q6_K super-block of 256 weights in 210 bytes [r56 sec. 1 and 3.2]:
 *   bytes   0..127  ql, the low 4 bits of the 6-bit codes
 *   bytes 128..191  qh, the high 2 bits
 *   bytes 192..207  sixteen signed 8-bit scales, one per 16 consecutive weights
 *   bytes 208..209  d, binary16 little-endian
 * weight = d * scale * (code - 32)  [r58 sec. 3.2: the centring by -32].
 * Element bit layout (reading: the ggml q6_K layout, restated): element e lies
 * in half h = e / 128; within the half let m = (e % 128) / 32 and l = e % 32.
 * Its low 4 bits are a nibble of ql[64h + 32(m mod 2) + l] (the low nibble when
 * m < 2, the high nibble otherwise) and its high 2 bits are bits 2m and 2m+1 of
 * qh[32h + l].                                                               */
static void decode_q6k_block(const uint8_t *B, int8_t *w, int8_t *sc, float *d)
{
    const uint8_t *ql = B;
    const uint8_t *qh = B + 128;
    for (int g = 0; g < 16; ++g)
        sc[g] = (int8_t)B[192 + g];
    *d = oracle_f16_to_f32((uint16_t)(B[208] | (B[209] << 8)));
    for (int e = 0; e < 256; ++e) {
        const int h = e / 128, m = (e % 128) / 32, l = e % 32;
        const uint8_t lowbyte = ql[64 * h + 32 * (m % 2) + l];
        const int low = (m < 2) ? (lowbyte & 15) : (lowbyte >> 4);
        const int high = (qh[32 * h + l] >> (2 * m)) & 3;
        w[e] = (int8_t)((low | (high << 4)) - 32);
    }
}

void oracle_decode_q6k(const uint8_t *raw, int64_t od, int64_t id,
                       int8_t *w, int8_t *sc, float *d)
{
    const int64_t nsb = id / 256;
    for (int64_t j = 0; j < od; ++j)
        for (int64_t b = 0; b < nsb; ++b)
            decode_q6k_block(raw + (j * nsb + b) * 210, w + j * id + 256 * b,
                             sc + j * (id / 16) + 16 * b, d + j * nsb + b);
}

/* q4_K super-block of 256 weights in 144 bytes [r58 sec. 2.2, 3.1]:
 *   bytes  0..1   d, binary16      bytes 2..3  dmin, binary16
 *   bytes  4..15  twelve bytes holding eight 6-bit scales and eight 6-bit mins,
 *                 one pair per 32-weight sub-block (get_scale_min_k4)
 *   bytes 16..143 qs, 4-bit codes
 * weight = d * scale_c * code - dmin * min_c  (reading: the minus sign of the
 * ggml convention).
 * Scale/min packing (reading: ggml's get_scale_min_k4, restated), P = bytes
 * 4..15: sub-block c < 4 takes its scale from the low 6 bits of P[c] and its
 * min from the low 6 bits of P[c+4]; sub-block c >= 4 takes its scale from the
 * low nibble of P[c+4] plus, as bits 4-5, the top two bits of P[c-4], and its
 * min from the high nibble of P[c+4] plus, as bits 4-5, the top two bits of P[c].
 * Code layout (reading: ggml): element e is a nibble of qs[32 (e / 64) + e % 32],
 * the low nibble when e % 64 < 32, the high nibble otherwise.               */
static void decode_q4k_block(const uint8_t *B, uint8_t *w, uint8_t *sc, uint8_t *mn,
                             float *d, float *dmin)
{
    const uint8_t *P = B + 4;
    const uint8_t *qs = B + 16;
    *d = oracle_f16_to_f32((uint16_t)(B[0] | (B[1] << 8)));
    *dmin = oracle_f16_to_f32((uint16_t)(B[2] | (B[3] << 8)));
    for (int c = 0; c < 8; ++c) {
        if (c < 4) {
            sc[c] = P[c] & 63;
            mn[c] = P[c + 4] & 63;
        } else {
            sc[c] = (uint8_t)((P[c + 4] & 15) | ((P[c - 4] >> 6) << 4));
            mn[c] = (uint8_t)((P[c + 4] >> 4) | ((P[c] >> 6) << 4));
        }
    }
    for (int e = 0; e < 256; ++e) {
        const uint8_t byte = qs[32 * (e / 64) + e % 32];
        w[e] = (e % 64 < 32) ? (byte & 15) : (byte >> 4);
    }
}

void oracle_decode_q4k(const uint8_t *raw, int64_t od, int64_t id,
                       uint8_t *w, uint8_t *sc, uint8_t *mn, float *d, float *dmin)
{
    const int64_t nsb = id / 256;
    for (int64_t j = 0; j < od; ++j)
        for (int64_t b = 0; b < nsb; ++b)
            decode_q4k_block(raw + (j * nsb + b) * 144, w + j * id + 256 * b,
                             sc + j * (id / 32) + 8 * b, mn + j * (id / 32) + 8 * b,
                             d + j * nsb + b, dmin + j * nsb + b);
}

/* ------------------------------------------------------------------------- */
/* O2 -- activation quantization                                              */
/* ------------------------------------------------------------------------- */

/* One q8 block per (token, 32 consecutive activations) [r45 sec. 2.3: 32 bytes
 * of q8 plus a 4-byte scale pair; r56 sec. 1: the pair is "d/ssum"].
 * Readings (the ggml q8_1 convention, with the stored scale used throughout):
 *   amax = max |x|;  d32 = amax / 127 (binary32 division);  dh = f16(d32);
 *   q = clamp(round-half-even(x / dh), -127, 127) (binary32 division), or 0
 *   when dh is 0;  S = sum of q;  s = f16(dh * S) (the binary32 product is exact).
 * The stored pair is (dh, s) as two binary16 values.                        */
int oracle_quantize(const float *x, int64_t n_tok, int64_t id,
                    int8_t *q, uint16_t *dh, uint16_t *s)
{
    if (n_tok < 0 || id <= 0 || id % 32 != 0)
        return -1;
    const int64_t nchunk = id / 32;
    for (int64_t t = 0; t < n_tok; ++t) {
        for (int64_t c = 0; c < nchunk; ++c) {
            const float *xc = x + t * id + 32 * c;
            int8_t *qc = q + t * id + 32 * c;
            float amax = 0.0f;
            for (int k = 0; k < 32; ++k) {
                if (!isfinite(xc[k]) || fabsf(xc[k]) > 2046.0f)
                    return -1;
                if (fabsf(xc[k]) > amax)
                    amax = fabsf(xc[k]);
            }
            const float d32 = amax / 127.0f;
            const uint16_t dbits = oracle_f32_to_f16(d32);
            const float dhf = oracle_f16_to_f32(dbits);
            int S = 0;
            for (int k = 0; k < 32; ++k) {
                int v = 0;
                if (dhf != 0.0f) {
                    const float r = xc[k] / dhf;
                    float n = rintf(r); /* default rounding mode: half to even */
                    if (n > 127.0f)
                        n = 127.0f;
                    if (n < -127.0f)
                        n = -127.0f;
                    v = (int)n;
                }
                qc[k] = (int8_t)v;
                S += v;
            }
            dh[t * nchunk + c] = dbits;
            s[t * nchunk + c] = oracle_f32_to_f16(dhf * (float)S);
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* O3 -- integer dots                                                         */
/* ------------------------------------------------------------------------- */

static int64_t idot(const int8_t *a, const int8_t *b, int n)
{
    int64_t acc = 0;
    for (int k = 0; k < n; ++k)
        acc += (int64_t)a[k] * (int64_t)b[k];
    return acc;
}

static int64_t udot(const uint8_t *a, const int8_t *b, int n)
{
    int64_t acc = 0;
    for (int k = 0; k < n; ++k)
        acc += (int64_t)a[k] * (int64_t)b[k];
    return acc;
}

void oracle_dots_q6k(const uint8_t *raw, int64_t od, int64_t id,
                     const int8_t *q, int64_t n_tok, int32_t *D16, int32_t *J)
{
    const int64_t ng = id / 16, nc = id / 32, nsb = id / 256;
    int8_t *w = malloc((size_t)id), *sc = malloc((size_t)ng);
    float *d = malloc(sizeof(float) * (size_t)nsb);
    if (!w || !sc || !d)
        goto done;
    for (int64_t j = 0; j < od; ++j) {
        oracle_decode_q6k(raw + j * nsb * 210, 1, id, w, sc, d);
        for (int64_t t = 0; t < n_tok; ++t) {
            for (int64_t c = 0; c < nc; ++c) {
                const int64_t d0 = idot(w + 32 * c, q + t * id + 32 * c, 16);
                const int64_t d1 = idot(w + 32 * c + 16, q + t * id + 32 * c + 16, 16);
                if (D16) {
                    D16[(t * od + j) * ng + 2 * c] = (int32_t)d0;
                    D16[(t * od + j) * ng + 2 * c + 1] = (int32_t)d1;
                }
                if (J)
                    J[(t * od + j) * nc + c] = (int32_t)(sc[2 * c] * d0 + sc[2 * c + 1] * d1);
            }
        }
    }
done:
    free(w);
    free(sc);
    free(d);
}

void oracle_dots_q4k(const uint8_t *raw, int64_t od, int64_t id,
                     const int8_t *q, int64_t n_tok, int32_t *D32)
{
    const int64_t nc = id / 32, nsb = id / 256;
    uint8_t *w = malloc((size_t)id), *sc = malloc((size_t)nc), *mn = malloc((size_t)nc);
    float *d = malloc(sizeof(float) * (size_t)nsb), *dm = malloc(sizeof(float) * (size_t)nsb);
    if (!w || !sc || !mn || !d || !dm)
        goto done;
    for (int64_t j = 0; j < od; ++j) {
        oracle_decode_q4k(raw + j * nsb * 144, 1, id, w, sc, mn, d, dm);
        for (int64_t t = 0; t < n_tok; ++t)
            for (int64_t c = 0; c < nc; ++c)
                D32[(t * od + j) * nc + c] =
                    (int32_t)udot(w + 32 * c, q + t * id + 32 * c, 32);
    }
done:
    free(w);
    free(sc);
    free(mn);
    free(d);
    free(dm);
}

/* ------------------------------------------------------------------------- */
/* O4 -- the result                                                           */
/* ------------------------------------------------------------------------- */

/* One decoded weight row. */
typedef struct {
    int type;
    int64_t id;
    int8_t *w6, *sc6;      /* q6_K */
    uint8_t *w4, *sc4, *mn4; /* q4_K */
    float *d, *dmin;
} row_t;

static int row_alloc(row_t *r, int type, int64_t id)
{
    memset(r, 0, sizeof *r);
    r->type = type;
    r->id = id;
    const size_t nsb = (size_t)(id / 256);
    r->d = malloc(sizeof(float) * nsb);
    r->dmin = malloc(sizeof(float) * nsb);
    if (type == ORACLE_Q6_K) {
        r->w6 = malloc((size_t)id);
        r->sc6 = malloc((size_t)(id / 16));
        return (r->d && r->dmin && r->w6 && r->sc6) ? 0 : -1;
    }
    r->w4 = malloc((size_t)id);
    r->sc4 = malloc((size_t)(id / 32));
    r->mn4 = malloc((size_t)(id / 32));
    return (r->d && r->dmin && r->w4 && r->sc4 && r->mn4) ? 0 : -1;
}

static void row_free(row_t *r)
{
    free(r->w6);
    free(r->sc6);
    free(r->w4);
    free(r->sc4);
    free(r->mn4);
    free(r->d);
    free(r->dmin);
}

static void row_decode(row_t *r, const uint8_t *raw, int64_t j)
{
    const int64_t nsb = r->id / 256;
    if (r->type == ORACLE_Q6_K)
        oracle_decode_q6k(raw + j * nsb * 210, 1, r->id, r->w6, r->sc6, r->d);
    else
        oracle_decode_q4k(raw + j * nsb * 144, 1, r->id, r->w4, r->sc4, r->mn4, r->d, r->dmin);
}

/* out[t][j] for one decoded row and one token (qrow = q[t], dhrow/srow = the
 * token's scale pairs).  Every term is exact in binary64.
 *   q6_K: sum over chunks c and halves h of  d * sc[2c+h] * dh[c] * D16[2c+h]
 *         (d*sc is the binary32 d-times-scale pair of [r56 sec. 2.2], exact)
 *   q4_K: sum over chunks c of  d * sc[c] * dh[c] * D32[c]  -  dmin * min[c] * s[c]
 * (the per-32 activation dot D times its activation scale dh, and the min term
 * against the stored scaled sum s).                                          */
static void pair_value(const row_t *r, const int8_t *qrow, const uint16_t *dhrow,
                       const uint16_t *srow, double *out, double *A)
{
    const int64_t nc = r->id / 32;
    double sum = 0.0, mag = 0.0;
    for (int64_t c = 0; c < nc; ++c) {
        const int64_t b = c / 8;
        const double dh = oracle_f16_to_f64(dhrow[c]);
        if (r->type == ORACLE_Q6_K) {
            for (int h = 0; h < 2; ++h) {
                const int64_t g = 2 * c + h;
                const int64_t D16 = idot(r->w6 + 16 * g, qrow + 16 * g, 16);
                const double tau = (double)r->d[b] * (double)r->sc6[g] * dh * (double)D16;
                sum += tau;
                mag += fabs(tau);
            }
        } else {
            const int64_t D32 = udot(r->w4 + 32 * c, qrow + 32 * c, 32);
            const double tau1 = (double)r->d[b] * (double)r->sc4[c] * dh * (double)D32;
            const double tau2 = -((double)r->dmin[b] * (double)r->mn4[c] *
                                  oracle_f16_to_f64(srow[c]));
            sum += tau1 + tau2;
            mag += fabs(tau1) + fabs(tau2);
        }
    }
    *out = sum;
    *A = mag;
}

static int check_args(int type, int64_t od, int64_t id, int64_t n_tok)
{
    if (type != ORACLE_Q4_K && type != ORACLE_Q6_K)
        return -1;
    if (od < 1 || id < 256 || id % 256 != 0 || n_tok < 0)
        return -1;
    return 0;
}

int oracle_mmq_rows(int type, const uint8_t *raw, int64_t od, int64_t id,
                    const int8_t *q, const uint16_t *dh, const uint16_t *s,
                    int64_t n_tok, int64_t j0, int64_t j1, double *out, double *A)
{
    if (check_args(type, od, id, n_tok) || j0 < 0 || j1 > od || j0 > j1)
        return -1;
    const int64_t nc = id / 32, w = j1 - j0;
    row_t r;
    if (row_alloc(&r, type, id)) {
        row_free(&r);
        return -1;
    }
    for (int64_t j = j0; j < j1; ++j) {
        row_decode(&r, raw, j);
        for (int64_t t = 0; t < n_tok; ++t)
            pair_value(&r, q + t * id, dh + t * nc, s + t * nc,
                       out + t * w + (j - j0), A + t * w + (j - j0));
    }
    row_free(&r);
    return 0;
}

int oracle_mmq(int type, const uint8_t *raw, int64_t od, int64_t id,
               const int8_t *q, const uint16_t *dh, const uint16_t *s,
               int64_t n_tok, double *out, double *A)
{
    return oracle_mmq_rows(type, raw, od, id, q, dh, s, n_tok, 0, od, out, A);
}

int oracle_mmq_at(int type, const uint8_t *raw, int64_t od, int64_t id,
                  const int8_t *q, const uint16_t *dh, const uint16_t *s,
                  int64_t n_tok, int64_t n, const int64_t *ts, const int64_t *js,
                  double *out, double *A)
{
    if (check_args(type, od, id, n_tok) || n < 0)
        return -1;
    for (int64_t i = 0; i < n; ++i)
        if (ts[i] < 0 || ts[i] >= n_tok || js[i] < 0 || js[i] >= od)
            return -1;
    const int64_t nc = id / 32;
    row_t r;
    if (row_alloc(&r, type, id)) {
        row_free(&r);
        return -1;
    }
    int64_t decoded = -1;
    for (int64_t i = 0; i < n; ++i) {
        if (js[i] != decoded) {
            row_decode(&r, raw, js[i]);
            decoded = js[i];
        }
        pair_value(&r, q + ts[i] * id, dh + ts[i] * nc, s + ts[i] * nc, out + i, A + i);
    }
    row_free(&r);
    return 0;
}
