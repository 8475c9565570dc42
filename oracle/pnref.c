/*
 * pnref.c - plain, slow, obviously correct CPU oracle for PN decode and GEMV.
 *
 * TEST INFRASTRUCTURE ONLY (see pnref.h).  Compiled with gcc -O2
 * -fno-fast-math; scalar C, no intrinsics, nothing shared with the HIP path.
 *
 * The PN format (tensorless, "Why a P100-native weight format"):
 *   - "Every block is 34 bytes": a 2-byte fp16 scale d, then eight 32-bit
 *     words of codes.  pn3t holds ten 3-bit codes per word (80 weights per
 *     block), pn4t eight 4-bit codes per word (64 weights per block).
 *   - "Codes never straddle the two halves of a word": codes go in pairs,
 *     even codes in the low 16 bits, odd codes in the high 16 bits, at the
 *     same offsets.
 *   - "Exact decode in fp32": w = d * (n - z), exact in binary32.
 *   - "Zero is a code, and the scale has a sign": mid-tread codes, range
 *     -4..+3 steps for pn3t; the scale is signed.
 *
 * Readings fixed here where the page is silent:
 *   - Field order: scale at bytes 0-1, word i at bytes 2+4i .. 5+4i, all
 *     little-endian, no padding.
 *   - Word i holds block slots C*i .. C*i+C-1.  Slot j of a word sits in half
 *     (j & 1) (0 = bits 0-15, 1 = bits 16-31) at bit offset b*(j >> 1) from
 *     that half's least significant bit.  Weight k of a row is slot k % W of
 *     block k / W.
 *   - z = 2^(b-1): 4 for pn3t, 8 for pn4t (pn4t range -8..+7).
 *   - pn3t bits 15 and 31 are unused: written as 0, ignored when read.
 */
#include "pnref.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define PN_BLOCK_BYTES 34
#define PN_WORDS 8

static int type_ok(int type) { return type == PNREF_PN3T || type == PNREF_PN4T; }
static int bits_of(int type) { return type == PNREF_PN3T ? 3 : 4; }
static int codes_per_word(int type) { return type == PNREF_PN3T ? 10 : 8; }

int pnref_block_bytes(void) { return PN_BLOCK_BYTES; }

int pnref_weights_per_block(int type)
{
    if (!type_ok(type)) return PNREF_EINVAL;
    return PN_WORDS * codes_per_word(type);
}

int pnref_zero_point(int type)
{
    if (!type_ok(type)) return PNREF_EINVAL;
    return 1 << (bits_of(type) - 1);
}

/* IEEE-754 binary16 -> binary32, written from the format's definition:
 * sign bit 15, biased exponent bits 10-14 (bias 15), fraction bits 0-9.
 * Every binary16 value is exactly representable in binary32. */
float pnref_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int f = h & 0x3ff;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);              /* zero or subnormal: f * 2^-24 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(1024 + f), e - 25);  /* (1 + f/1024) * 2^(e-15)      */
    return (float)(sign ? -v : v);
}

/* binary64 -> binary16, round to nearest, ties to even. */
uint16_t pnref_double_to_half(double v)
{
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (isnan(v)) return 0x7e00;
    if (a >= 65520.0) return sign | 0x7c00;     /* halfway to 2^16 rounds up to inf */
    if (a < ldexp(1.0, -14)) {
        /* subnormal range: quantum 2^-24; a count of 1024 is the smallest normal */
        double q = nearbyint(a * 16777216.0);
        return sign | (uint16_t)q;
    }
    int e2;
    frexp(a, &e2);                               /* a in [2^(e2-1), 2^e2) */
    int e = e2 - 1;                              /* unbiased exponent     */
    double q = nearbyint(ldexp(a, 10 - e));      /* in [1024, 2048]       */
    /* q == 2048 carries into the exponent field, which the sum below does. */
    return sign | (uint16_t)(((e + 15) << 10) + ((int)q - 1024));
}

static uint32_t load_le32(const uint8_t *p)
{
    return (uint32_t)p[0] | ((uint32_t)p[1] << 8) | ((uint32_t)p[2] << 16) |
           ((uint32_t)p[3] << 24);
}

int pnref_decode_block(int type, const uint8_t *blk, float *out)
{
    if (!type_ok(type) || !blk || !out) return PNREF_EINVAL;
    const int b = bits_of(type);
    const int c = codes_per_word(type);
    const int z = 1 << (b - 1);
    const uint32_t mask = (1u << b) - 1u;
    const float d = pnref_half_to_float((uint16_t)(blk[0] | (blk[1] << 8)));
    for (int i = 0; i < PN_WORDS; ++i) {
        const uint32_t q = load_le32(blk + 2 + 4 * i);
        for (int j = 0; j < c; ++j) {
            const int shift = 16 * (j & 1) + b * (j >> 1);
            const int n = (int)((q >> shift) & mask);
            /* one binary32 multiply; exact because 11 + 4 bits fit in 24 */
            out[i * c + j] = d * (float)(n - z);
        }
    }
    return PNREF_OK;
}

static int shape_check(int type, int64_t n, int64_t k)
{
    if (!type_ok(type)) return PNREF_EINVAL;
    const int w = PN_WORDS * codes_per_word(type);
    if (n < 0 || k < 0 || k % w != 0) return PNREF_ESHAPE;
    return PNREF_OK;
}

int pnref_dequantize(int type, const uint8_t *w, int64_t n, int64_t k, float *out)
{
    int st = shape_check(type, n, k);
    if (st) return st;
    const int wpb = PN_WORDS * codes_per_word(type);
    const int64_t nb = k / wpb;
    for (int64_t r = 0; r < n; ++r)
        for (int64_t j = 0; j < nb; ++j)
            pnref_decode_block(type, w + (r * nb + j) * PN_BLOCK_BYTES,
                               out + r * k + j * wpb);
    return PNREF_OK;
}

int pnref_set_threads(int nthreads)
{
#ifdef _OPENMP
    if (nthreads > 0) omp_set_num_threads(nthreads);
    return omp_get_max_threads();
#else
    (void)nthreads;
    return 1;
#endif
}

/* One output row: decode the row, then a sequential fp64 sum over k.
 * Each product of a decoded weight (<= 15 significant bits) and an fp16
 * activation (11 bits) is exact in fp64; only the running sum rounds. */
static void gemv_row(int type, const uint8_t *row, int64_t k, const double *xd,
                     float *wrow, double *y, double *a)
{
    const int wpb = PN_WORDS * codes_per_word(type);
    const int64_t nb = k / wpb;
    for (int64_t j = 0; j < nb; ++j)
        pnref_decode_block(type, row + j * PN_BLOCK_BYTES, wrow + j * wpb);
    double s = 0.0, t = 0.0;
    for (int64_t i = 0; i < k; ++i) {
        const double p = (double)wrow[i] * xd[i];
        s += p;
        t += fabs(p);
    }
    *y = s;
    if (a) *a = t;
}

int pnref_gemm_f64(int type, const uint8_t *w, int64_t n, int64_t k,
                   const uint16_t *xm, int64_t ldx, int m,
                   double *ym, int64_t ldy, double *am)
{
    int st = shape_check(type, n, k);
    if (st) return st;
    if (m < 1 || ldx < k || ldy < n) return PNREF_ESHAPE;
    if (!w || !xm || !ym) return PNREF_EINVAL;
    const int wpb = PN_WORDS * codes_per_word(type);
    const int64_t row_bytes = (k / wpb) * PN_BLOCK_BYTES;
    double *xd = (double *)malloc(sizeof(double) * (size_t)(k ? k : 1) * (size_t)m);
    if (!xd) return PNREF_EINVAL;
    for (int mi = 0; mi < m; ++mi)
        for (int64_t i = 0; i < k; ++i)
            xd[mi * k + i] = (double)pnref_half_to_float(xm[mi * ldx + i]);
    int failed = 0;
#pragma omp parallel
    {
        float *wrow = (float *)malloc(sizeof(float) * (size_t)(k ? k : 1));
        if (!wrow) {
#pragma omp atomic write
            failed = 1;
        } else {
#pragma omp for schedule(static)
            for (int64_t r = 0; r < n; ++r)
                for (int mi = 0; mi < m; ++mi)
                    gemv_row(type, w + r * row_bytes, k, xd + mi * k, wrow,
                             ym + mi * ldy + r, am ? am + mi * ldy + r : NULL);
            free(wrow);
        }
    }
    free(xd);
    return failed ? PNREF_EINVAL : PNREF_OK;
}

int pnref_gemv_f64(int type, const uint8_t *w, int64_t n, int64_t k,
                   const uint16_t *x, double *y, double *a)
{
    return pnref_gemm_f64(type, w, n, k, x, k, 1, y, n, a);
}

/* Signed-scale round-to-nearest quantizer, per block of W weights
 * ("Zero is a code, and the scale has a sign": the extra step points at the
 * side of the largest-magnitude weight, which gets the full range):
 *   1. i* = index of the largest |w_i|; ties go to the lowest index.
 *   2. if w[i*] == 0: d = +0 and every code is z.
 *   3. d = fp16_rne(-w[i*] / z), the quotient taken in fp64, so that w[i*]
 *      lands on the full -z step (code 0).  If d is not finite the block is
 *      out of range (error); if d rounds to zero every code is z.
 *   4. n_i = clamp(z + rint(w_i / d), 0, 2^b - 1), rint ties to even, fp64.
 *   5. pack per the layout above; unused pn3t bits are written 0. */
int pnref_quantize(int type, const float *w, int64_t n, int64_t k, uint8_t *out)
{
    int st = shape_check(type, n, k);
    if (st) return st;
    if (!w || !out) return PNREF_EINVAL;
    const int b = bits_of(type);
    const int c = codes_per_word(type);
    const int z = 1 << (b - 1);
    const int wpb = PN_WORDS * c;
    const int64_t nblocks = n * (k / wpb);
    for (int64_t g = 0; g < nblocks; ++g) {
        const float *src = w + g * wpb;
        uint8_t *blk = out + g * PN_BLOCK_BYTES;
        int istar = 0;
        for (int i = 1; i < wpb; ++i)
            if (fabsf(src[i]) > fabsf(src[istar])) istar = i;
        uint16_t dbits = 0;
        int codes[80];
        double d = 0.0;
        if (src[istar] != 0.0f) {
            dbits = pnref_double_to_half(-(double)src[istar] / (double)z);
            if ((dbits & 0x7c00) == 0x7c00) return PNREF_ERANGE;
            d = (double)pnref_half_to_float(dbits);
        }
        for (int i = 0; i < wpb; ++i) {
            int nn = z;
            if (d != 0.0) {
                double t = nearbyint((double)src[i] / d);
                double v = (double)z + t;
                if (v < 0.0) v = 0.0;
                if (v > (double)((1 << b) - 1)) v = (double)((1 << b) - 1);
                nn = (int)v;
            }
            codes[i] = nn;
        }
        blk[0] = (uint8_t)(dbits & 0xff);
        blk[1] = (uint8_t)(dbits >> 8);
        for (int i = 0; i < PN_WORDS; ++i) {
            uint32_t q = 0;
            for (int j = 0; j < c; ++j)
                q |= (uint32_t)codes[i * c + j] << (16 * (j & 1) + b * (j >> 1));
            for (int t = 0; t < 4; ++t) blk[2 + 4 * i + t] = (uint8_t)(q >> (8 * t));
        }
    }
    return PNREF_OK;
}

/* Blockwise Hadamard rotation (see pnref.h).  Readings fixed here where the
 * page is silent:
 *   - block size B = 1024 in the library (the largest power of two that
 *     divides every PN width of the model, 5120, 6144 and 17408); the oracle
 *     takes any power of 4 so that small cases can be worked by hand;
 *   - Sylvester order, H[i][j] = (-1)^popcount(i & j), and the orthonormal
 *     scale 1/sqrt(B) (a power of two for B a power of 4, so exact);
 *   - the result is rounded once to fp16 (the GEMV's activation type), ties
 *     to even; an exact zero is +0.
 * The sum runs sequentially in fp64 and is exact: every fp16 value is a
 * multiple of 2^-24 below 2^16, so every partial sum of at most 1024 of them
 * is a multiple of 2^-24 below 2^26, which binary64 holds exactly. */
int pnref_rotate(const uint16_t *x, int64_t k, int64_t block, uint16_t *out)
{
    if (!x || !out || block < 1 || k < 0) return PNREF_EINVAL;
    int lg = 0;
    while (((int64_t)1 << lg) < block) ++lg;
    if (((int64_t)1 << lg) != block || (lg & 1) || block > 1024) return PNREF_ESHAPE;
    if (k % block != 0) return PNREF_ESHAPE;
    const double scale = ldexp(1.0, -lg / 2);
    for (int64_t b0 = 0; b0 < k; b0 += block) {
        for (int64_t i = 0; i < block; ++i) {
            double s = 0.0;
            for (int64_t j = 0; j < block; ++j) {
                const double v = (double)pnref_half_to_float(x[b0 + j]);
                s += (__builtin_popcountll((uint64_t)(i & j)) & 1) ? -v : v;
            }
            out[b0 + i] = pnref_double_to_half(s * scale);  /* s starts at +0: an exact zero is +0 */
        }
    }
    return PNREF_OK;
}
