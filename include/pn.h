/*
 * pn.h - C ABI of the PN decode GEMV library for AMD Instinct MI355X (gfx950).
 *
 * The PN weight format (tensorless, "Why a P100-native weight format"):
 *   - "Every block is 34 bytes": an fp16 scale d (2 bytes) followed by eight
 *     32-bit code words.  pn3t packs ten 3-bit codes per word (80 weights per
 *     block); pn4t packs eight 4-bit codes per word (64 weights per block).
 *     A row is made of whole blocks, so K is a multiple of 80 or 64.
 *   - "Codes never straddle the two halves of a word": even codes sit in the
 *     low 16 bits, odd codes in the high 16 bits, at the same offsets.
 *   - "Exact decode in fp32": weight = d * (n - z), exact in binary32.
 *   - "Zero is a code, and the scale has a sign": z = 4 for pn3t (range
 *     -4..+3 steps); this library takes z = 8 for pn4t (-8..+7).
 * Bit layout fixed by this library where the page is silent: scale at bytes
 * 0-1 and word i at bytes 2+4i..5+4i, little-endian; word i holds the
 * block's weights C*i .. C*i+C-1 (C = 10 or 8); weight j of a word sits in
 * half (j & 1) at bit offset b*(j >> 1) from that half's lowest bit; pn3t
 * bits 15 and 31 are ignored.
 *
 * Memory: every pointer is a DEVICE pointer owned by the caller (e.g. a torch
 * tensor's data_ptr()).  Weight matrices are N rows of K/W blocks, rows
 * contiguous (row stride pn_row_bytes(t, K)); the base only needs 2-byte
 * alignment.  Activations are IEEE fp16, 4-byte aligned; outputs are fp32,
 * 4-byte aligned, overwritten (never accumulated).
 *
 * Streams: `stream` is a hipStream_t (NULL = the default stream).  Calls
 * enqueue work and return without synchronising; device faults surface at
 * the caller's next synchronisation.  The calls allocate nothing (except
 * the group-create calls, documented there).
 *
 * Threads: the calls may be made from several host threads at once, with
 * two exceptions.  A group plan must not run concurrently with itself (two
 * runs of one plan on different streams, or graph launches of it that
 * overlap): some plans keep tile counters in the plan's device memory, and
 * two runs sharing them would each compute only part of the output.  (Such
 * runs still end: each wave or workgroup stops after more steps than any
 * correct run takes, and the outputs are then unspecified.)  And a
 * plan must not be destroyed while another thread runs it.  The kernel
 * selections (pn_set_gemv_kernel, pn_set_smallm_math) belong to the calling
 * host thread, and the variant census (pn_last_variant) too.  Per-device
 * facts the library caches (compute-unit count, occupancy, raised LDS
 * limits) are filled once, under a lock.
 *
 * Errors: arguments are checked on the host before any launch; a failing
 * check returns a negative pn_status and enqueues nothing.
 */
#ifndef PN_H
#define PN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { PN_PN3T = 0, PN_PN4T = 1 } pn_type;

typedef enum {
    PN_OK = 0,
    PN_EINVAL = -1,       /* null pointer, unknown type, bad count          */
    PN_ESHAPE = -2,       /* N < 1, K not a positive multiple of W, M/ld bad */
    PN_EALIGN = -3,       /* W not 2-aligned, x/X/y/Y not 4-aligned         */
    PN_EUNSUPPORTED = -4, /* shape outside what the kernels support         */
    PN_ELAUNCH = -5,      /* the HIP launch or a HIP runtime call failed    */
    PN_ENOMEM = -6        /* device allocation failed (pn_group_create)     */
} pn_status;

/* Weights per block: 80 (pn3t) or 64 (pn4t); 0 for an unknown type. */
int pn_weights_per_block(pn_type t);

/* Bytes of one packed row of K weights: (K / W) * 34, or 0 if K is not a
 * positive multiple of W. */
size_t pn_row_bytes(pn_type t, int64_t K);

/* y[r] = sum_k w[r,k] * x[k] for r < N.
 * "One lane, one word" and "Exact decode in fp32" on the pn-format page
 * describe the decode GEMV this computes: weights decoded exactly as
 * d * (n - z), products accumulated in fp32 (any order; the result is within
 * 1e-5 * sum_k |w[r,k] x[k]| of the exact value, row by row).
 *   W : N * pn_row_bytes(t, K) bytes, 2-byte aligned
 *   x : K fp16 values, 4-byte aligned
 *   y : N fp32 values, 4-byte aligned, overwritten */
pn_status pn_gemv(pn_type t, const void *W, int64_t N, int64_t K,
                  const void *x, float *y, void *stream);

/* Two matrices of the same type and shape against one activation, one
 * launch (the fused gate + up projection of a decoder layer):
 * y0 = W0 x, y1 = W1 x.  Arguments as for pn_gemv. */
pn_status pn_gemv2(pn_type t, const void *W0, const void *W1, int64_t N,
                   int64_t K, const void *x, float *y0, float *y1, void *stream);

/* Small-batch product for M <= 16 activation rows (speculative-decoding
 * verification width M = k + 1; v100-skinny README, "How QPN works"):
 * Y[m*ldy + r] = sum_k w[r,k] * X[m*ldx + k] for m < M, r < N.
 * Each weight is decoded exactly once and used M times; products accumulate
 * in fp32, within 1e-5 * sum_k |w[r,k] X[m,k]| of the exact value.
 *   X : M rows of fp16, leading dimension ldx >= K (elements), 4-byte aligned,
 *       ldx even
 *   Y : M rows of fp32, leading dimension ldy >= N (elements), overwritten
 *   M : 1..16
 * The arithmetic unit is the one pn_set_smallm_math selected.  With MFMA,
 * rows of whole 8-block periods (K a multiple of 640 for pn3t, 512 for pn4t)
 * and a 16-byte-aligned W are streamed into LDS by DMA (kernel gemm_rows)
 * unless pn_set_gemv_kernel chose PN_GEMV_STREAM; other problems, and the
 * VALU arithmetic, use register loads (gemm_stream).  Same accuracy bar. */
pn_status pn_gemm_smallm(pn_type t, const void *W, int64_t N, int64_t K,
                         const void *X, int64_t ldx, int M,
                         float *Y, int64_t ldy, void *stream);

/* Prefill: the same product for any number of activation rows (a prompt's
 * tokens),
 *   Y[m*ldy + r] = sum_k w[r,k] X[m*ldx + k],  m < M,  w = d * (n - z),
 * with the weights decoded inside the GEMM from the packed rows and never
 * written out (the pages' engine dequantizes PN weights for a chunked
 * prefill GEMM, "What the fork adds").  Products on MFMA in fp32, each
 * block's partial sum scaled by its d in fp32; within the tolerance above.
 *   W : packed rows, 4-byte aligned; K an even number of blocks (a multiple
 *       of 160 for pn3t, 128 for pn4t), else PN_EUNSUPPORTED
 *   X : M rows of fp16, 16-byte aligned, ldx >= K and a multiple of 8
 *   Y : M rows of fp32, 4-byte aligned, ldy >= N, overwritten
 *   M : >= 1 (at most 8,388,480)
 * Allocates nothing; enqueued on `stream`. */
pn_status pn_gemm_prefill(pn_type t, const void *W, int64_t N, int64_t K,
                          const uint16_t *X, int64_t ldx, int64_t M,
                          float *Y, int64_t ldy, void *stream);

/* Arithmetic of the small-batch kernels.  Both read the weights the same way
 * and agree within the tolerance above:
 *   PN_SMALLM_MFMA  decoded weights feed matrix-core products
 *                   (v_mfma_f32_16x16x16_f16 / 16x16x32_f16), one per block
 *                   and 16 rows, each scaled by its block's d in fp32; the
 *                   default (faster on MI355X at M = 8: 3.0 vs 5.9 ms per
 *                   64-layer token);
 *   PN_SMALLM_VALU  per-lane fp16 dot products (v_dot2_f32_f16) reduced
 *                   across the lanes of a row.
 * The setting belongs to the calling host thread (every thread starts with
 * PN_SMALLM_MFMA) and is read when that thread makes a call or creates a
 * group (a group keeps the choice it was created with).  Returns PN_EINVAL
 * for an unknown value. */
typedef enum { PN_SMALLM_MFMA = 0, PN_SMALLM_VALU = 1 } pn_smallm_math;
pn_status pn_set_smallm_math(pn_smallm_math m);
pn_smallm_math pn_get_smallm_math(void);

/* Which kernel runs the M = 1 products (pn_gemv, pn_gemv2 and pn_group_*;
 * for the small-batch products see pn_gemm_smallm):
 *   PN_GEMV_AUTO    the row-tile kernel where it applies and the launch is
 *                   large enough, else the register-pipeline kernel; the
 *                   default.  The row-tile kernel applies to rows of whole
 *                   8-block periods (K a multiple of 640 for pn3t, 512 for
 *                   pn4t) with 16-byte-aligned W and x; "large enough" is at
 *                   least 32 sixteen-row tiles per compute unit (8192 tiles,
 *                   131,072 rows, on a 256-CU MI355X), because one or two
 *                   problems are split among its waves in whole tiles;
 *   PN_GEMV_STREAM  always the register-pipeline kernel;
 *   PN_GEMV_ROWS    the row-tile kernel wherever it applies, whatever the
 *                   launch size.
 * All meet the same accuracy bar.  The setting belongs to the calling host
 * thread (every thread starts with PN_GEMV_AUTO) and is read when that
 * thread makes a call or creates a group.  Returns PN_EINVAL for an unknown
 * value. */
typedef enum { PN_GEMV_AUTO = 0, PN_GEMV_STREAM = 1, PN_GEMV_ROWS = 2 } pn_gemv_kernel;
pn_status pn_set_gemv_kernel(pn_gemv_kernel k);
pn_gemv_kernel pn_get_gemv_kernel(void);

/* Dense fp32 copy of the decoded weights, out[r*K + k] = d * (n - z),
 * bit-exact with the format's definition ("Exact decode in fp32": no
 * rounding in decode, so every correct decoder gives the same bits).
 *   out : N * K fp32, 4-byte aligned */
pn_status pn_dequantize(pn_type t, const void *W, int64_t N, int64_t K,
                        float *out, void *stream);

/* Blockwise Hadamard rotation of fp16 activations (tensorless, "How
 * Qwen3.8-27B-PN3 uses it": the model's engine rotates the activations that
 * reach the PN weights at run time; the page gives no size or scale, and
 * the reading here is the one the CPU oracle fixes):
 *   out[m*ldo + b*1024 + i] =
 *       fp16_rne( sum_j H[i][j] x[m*ldx + b*1024 + j] / 32 ),
 *   H[i][j] = (-1)^popcount(i & j)   (Sylvester order, 1024 x 1024),
 * for every row m < M and every 1024-element block b of the K columns.
 * Exact up to the one fp16 rounding (ties to even; an exact zero is +0), so
 * every correct implementation gives the same bits.
 *   x, out : fp16, device, 4-byte aligned, ldx and ldo even and >= K.
 *            out may be x (same ld): rotation in place.  Other overlaps are
 *            not allowed.
 *   K      : a multiple of 1024 (else PN_ESHAPE); M >= 1.
 * Enqueued on `stream`; returns without waiting. */
#define PN_ROTATE_BLOCK 1024
pn_status pn_rotate(const uint16_t *x, int64_t K, int M, int64_t ldx,
                    uint16_t *out, int64_t ldo, void *stream);

/* A group of independent GEMVs run by one kernel launch (a decoder layer's
 * projections, or a whole per-token weight sweep).  Each entry is one
 * pn_gemv problem; the entries may mix types and shapes. */
typedef struct pn_gemv_desc {
    const void *W;   /* packed rows, device          */
    const void *x;   /* fp16 [K], device             */
    float *y;        /* fp32 [N], device, overwritten */
    int64_t N;
    int64_t K;
    int32_t type;    /* pn_type                      */
    int32_t flags;   /* 0, or PN_DESC_ROTATE         */
} pn_gemv_desc;

/* Entry flag: x is in the model's unrotated basis; the plan multiplies by
 * pn_rotate's image of x (y = W H x).  Needs K a multiple of 1024.  The plan
 * keeps a device copy of each such x, rotated at the start of every run by
 * one extra launch ahead of the GEMV launch, on the same stream. */
#define PN_DESC_ROTATE 1

typedef struct pn_group pn_group;

/* Validate `count` descriptors (host array) and build a launch plan.  This
 * call allocates device memory for the plan's tables (and for the rotated
 * copies of PN_DESC_ROTATE inputs) and copies them there synchronously; the plan holds the descriptors' device pointers, which must
 * stay valid while the plan is used.  Returns PN_ENOMEM if allocation fails.
 * The plan runs on the row-tile kernel if that takes every problem and the
 * launch (see pn_set_gemv_kernel); otherwise every problem's rows must be
 * whole groups of 8 blocks (K a multiple of 640 for pn3t, 512 for pn4t) with
 * 2*K <= 64 KiB of activation, and other shapes return PN_EUNSUPPORTED
 * (pn_gemv takes them one at a time).  The kernel choice is made here, once,
 * for the device current at this call, and the plan's tables are placed in
 * that device's memory: pn_group_run returns PN_EUNSUPPORTED when another
 * device is current.  A plan must not run concurrently with itself (see
 * "Threads" above). */
pn_status pn_group_create(const pn_gemv_desc *descs, int count, pn_group **out);

/* The small-batch counterpart: each entry is one pn_gemm_smallm problem
 * (arguments and checks as there), all run by one launch.  Any K is taken.
 * Allocation and lifetime as for pn_group_create. */
typedef struct pn_gemm_desc {
    const void *W;   /* packed rows, device                     */
    const void *X;   /* fp16 [M][ldx], device                   */
    float *Y;        /* fp32 [M][ldy], device, overwritten      */
    int64_t N;
    int64_t K;
    int64_t ldx;     /* elements, >= K, even                    */
    int64_t ldy;     /* elements, >= N                          */
    int32_t type;    /* pn_type                                 */
    int32_t M;       /* 1..16 (pn_gemm_prefill_group: >= 1)     */
} pn_gemm_desc;

pn_status pn_group_create_smallm(const pn_gemm_desc *descs, int count, pn_group **out);

/* Several prefill products as one launch: the projections of a decoder layer
 * that can run together because their inputs are ready together (q, k and v;
 * gate and up), so that their tiles fill the device as one launch instead of
 * three or two that each leave part of it idle.  Each entry is one
 * pn_gemm_prefill problem (arguments, checks and results as there; M may
 * differ between entries); the entries may mix types and shapes.  At most
 * PN_PREFILL_GROUP_MAX entries, else PN_EINVAL; the first entry that fails a
 * check gives the status and nothing is enqueued.  Allocates nothing (the
 * entries travel in the launch's arguments); enqueued on `stream`. */
#define PN_PREFILL_GROUP_MAX 8
pn_status pn_gemm_prefill_group(const pn_gemm_desc *descs, int count, void *stream);

/* Enqueue all problems of a plan (either kind) as one launch on `stream`
 * (plus the rotation launch ahead of it for PN_DESC_ROTATE entries).  Runs
 * of one plan must be ordered (one stream, or waits between streams): a run
 * resets the plan's tile counters as its last wave finishes, ready for the
 * next run.  PN_EUNSUPPORTED if the device current at this call is not the
 * plan's. */
pn_status pn_group_run(const pn_group *g, void *stream);

/* Free a plan (NULL is allowed).  Synchronises the device first. */
void pn_group_destroy(pn_group *g);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, serving loops or harnesses that forbid hipMalloc): the problems of
 * a pn_group_create plan, run at once without a plan.  Results are those of
 * pn_group_create + pn_group_run on the same descriptors (the same kernel
 * choice and tile order; no PN_DESC_ROTATE entries).
 *
 * The plan (problem table, tile order, tile-pool counters) is written into a
 * library-owned device buffer of PN_BATCH_BYTES by one small kernel ahead of
 * the GEMV launch, both on `stream`; the buffer is a static device array, one
 * per GPU, held until the process ends.  The call allocates nothing and takes
 * the descriptors (a host array) by value.  Every call on a GPU shares that
 * GPU's buffer: calls on one stream are ordered, but calls that overlap on
 * one GPU (two streams, or other host threads) race and must not be made.
 *   count : 1..PN_BATCH_MAX_PROBLEMS, else PN_EINVAL (< 1) or
 *           PN_EUNSUPPORTED (too many)
 *   rows  : on the row-tile kernel at most PN_BATCH_MAX_ROWS rows in all
 *           (16-row tiles), else PN_EUNSUPPORTED
 * Other checks and errors as pn_group_create (PN_DESC_ROTATE entries return
 * PN_EUNSUPPORTED). */
#define PN_BATCH_MAX_PROBLEMS 32
#define PN_BATCH_MAX_ROWS (65536 * 16)
#define PN_BATCH_BYTES (17 * 4096 + 4096 + 4 * 65536)
pn_status pn_gemv_batch(const pn_gemv_desc *descs, int count, void *stream);

/* Streaming-read probe: the practical HBM read ceiling of the device,
 * measured in the same harness as the GEMV (the v100-skinny README, "Kernel
 * benchmarks", rates its kernels against a measured read-only ceiling).  One
 * launch reads `*bytes_read` bytes (the largest multiple of the launch's
 * granule, 1 KiB per wave, not above `bytes`) from `buf` with
 * 16-byte nontemporal DMA loads into LDS (each wave a contiguous share) and
 * writes a checksum word per lane to `scratch`.
 *   buf     : device, 16-byte aligned, `bytes` readable
 *   scratch : device, 4-byte aligned, pn_read_probe_scratch_bytes() bytes
 * Returns PN_ESHAPE if `bytes` is too small or `scratch_bytes` too small. */
size_t pn_read_probe_scratch_bytes(void);
pn_status pn_read_probe(const void *buf, size_t bytes, void *scratch, size_t scratch_bytes,
                        size_t *bytes_read, void *stream);

/* Text for a status code. */
const char *pn_status_str(pn_status e);

/* Kernel variant chosen by this thread's last successful enqueue (a census
 * for benchmarks so that no fallback route goes unreported); values are
 * listed by pn_variant_name. */
int pn_last_variant(void);
const char *pn_variant_name(int v);

#ifdef __cplusplus
}
#endif
#endif
