/*
 * pnref.h - CPU oracle for the PN weight format (pn3t / pn4t).
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may include, link or
 * call this code: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no source with the HIP library.
 *
 * Source of the definitions: the tensorless page "Why a P100-native weight
 * format", sections "Every block is 34 bytes", "Codes never straddle the two
 * halves of a word", "Exact decode in fp32" and "Zero is a code, and the scale
 * has a sign".  Points the page leaves open (bit order inside a half, z for
 * pn4t, quantizer tie rules) are fixed as documented beside each function in
 * pnref.c.
 *
 * All pointers are host pointers.  Functions return 0 on success and a
 * negative value on bad arguments (see PNREF_E*).
 */
#ifndef PNREF_H
#define PNREF_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum { PNREF_PN3T = 0, PNREF_PN4T = 1 };
enum { PNREF_OK = 0, PNREF_EINVAL = -1, PNREF_ESHAPE = -2, PNREF_ERANGE = -3 };

int    pnref_block_bytes(void);                 /* 34                         */
int    pnref_weights_per_block(int type);       /* 80 (pn3t) / 64 (pn4t)      */
int    pnref_zero_point(int type);              /* 4 (pn3t) / 8 (pn4t)        */

float  pnref_half_to_float(uint16_t h);         /* exact, hand-written        */
uint16_t pnref_double_to_half(double v);        /* round to nearest even      */

/* Decode one 34-byte block into W floats. */
int pnref_decode_block(int type, const uint8_t *blk, float *out);

/* Decode an N x K matrix of packed rows (row stride = K/W*34 bytes). */
int pnref_dequantize(int type, const uint8_t *w, int64_t n, int64_t k, float *out);

/* y[r] = sum_k w[r,k] x[k] accumulated in fp64, in k order; a[r] = sum_k |w x|.
 * x holds fp16 bit patterns.  a may be NULL. */
int pnref_gemv_f64(int type, const uint8_t *w, int64_t n, int64_t k,
                   const uint16_t *x, double *y, double *a);

/* Y[m*ldy + r] = sum_k w[r,k] X[m*ldx + k] for m < M, fp64 as above. */
int pnref_gemm_f64(int type, const uint8_t *w, int64_t n, int64_t k,
                   const uint16_t *xm, int64_t ldx, int m,
                   double *ym, int64_t ldy, double *am);

/* Signed-scale round-to-nearest quantizer: fp32 N x K -> packed rows. */
int pnref_quantize(int type, const float *w, int64_t n, int64_t k, uint8_t *out);

/* Blockwise Hadamard rotation of fp16 activations (tensorless, "How
 * Qwen3.8-27B-PN3 uses it": the engine rotates the activations that reach the
 * PN weights at run time; the page gives neither the size nor the scaling,
 * readings in pnref.c):
 *   out[b*B + i] = fp16_rne( sum_j H[i][j] x[b*B + j] / sqrt(B) ),
 *   H[i][j] = (-1)^popcount(i & j)  (Sylvester order),
 * for every block b of B = `block` elements; B a power of 4, k a multiple of
 * B.  x and out hold fp16 bit patterns and may not overlap. */
int pnref_rotate(const uint16_t *x, int64_t k, int64_t block, uint16_t *out);

/* Threads the fp64 GEMV may use (OpenMP over rows); returns the count used. */
int pnref_set_threads(int nthreads);

#ifdef __cplusplus
}
#endif
#endif
