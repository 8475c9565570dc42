// pn_smallm.hip - small-batch PN GEMM (M <= 16 activation rows) for AMD
// Instinct MI355X (gfx950), and its C ABI: pn_gemm_smallm,
// pn_group_create_smallm, pn_set_smallm_math.
//
// Y[m, r] = sum_k w[r, k] X[m, k] for m < M <= 16, the verification width of
// speculative decoding, M = k + 1 (v100-skinny README, "How QPN works": a
// tile costs the same whether or not every row carries work, and k = 15 needs
// 16 rows).  Each weight is decoded once and used for all M rows.
//
// Work layout.  A wave owns 32 consecutive rows (two groups of 16) and walks
// their blocks in order, with a pipeline of U blocks of loads in flight.
// Lane l = 4j + g loads words 2g and 2g+1 (one dwordx2) of row j of each
// group, plus that block's scale.  The workgroup's activations sit in LDS,
// a chunk of whole blocks at a time.
//
// Two maths over the same loads (pn_set_smallm_math):
//   MFMA  the decoded weights of 16 rows x one block form the B operand of
//         v_mfma_f32_16x16x16_f16 (pn3t: 5 steps per block) or
//         v_mfma_f32_16x16x32_f16 (pn4t: 2 steps); X is the A operand (its 16
//         rows are the batch; rows past M are discarded).  Each
//         block starts a fresh accumulator, which is scaled by that block's d
//         in fp32 and added to the running sum: folding d into fp16 operands
//         would round.  The words and scale move to the operand layout (lane
//         16g + j for row j, k-group g) with ds_bpermute; lane (j, g) then
//         receives D[m = 4g + i][row j], i < 4, so one scale per lane serves
//         all four.
//   VALU  each lane dots its 20 (pn3t) or 16 (pn4t) decoded weights with each
//         of the M activation rows (v_dot2_f32_f16), scales by d and keeps M
//         sums per row; the four lanes (one quad) of a row are added at the end.
// Within a block, lane g's weights are the block's 20g..20g+19 (pn3t: words
// 2g and 2g+1 hold ten consecutive weights each) or 16g..16g+15 (pn4t), and
// the X operand is read at the same positions, so both maths pair every code
// with its own activation.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <atomic>

#include <type_traits>

#include "pn_device.h"
#include "pn_host.h"

using namespace pn;
using namespace pn::host;

namespace {

#ifndef PN_SM_WAVES
#define PN_SM_WAVES 8
#endif
#ifndef PN_SM_ITEMS
#define PN_SM_ITEMS 4
#endif
// MFMA math: loads are issued a group of U blocks at a time into 2U slots, so
// that each row's next U blocks are requested back to back (measured 3.06 ms
// vs 3.73 ms per M = 8 token).  The VALU math, bound by its arithmetic, keeps
// one block at a time in U slots and more waves per CU.
#ifndef PN_SM_GROUPED
#define PN_SM_GROUPED 1
#endif
// LDS budget of one workgroup's activation chunk, in KiB, per math.  The
// grouped MFMA pipeline's registers allow one 8-wave workgroup per CU, so it
// may take the whole LDS (at M = 8 only K > 10240 then needs more than one
// chunk); the VALU math runs two workgroups per CU.
#ifndef PN_SM_LDS_KB
#define PN_SM_LDS_KB 160
#endif
#ifndef PN_SM_VALU_LDS_KB
#define PN_SM_VALU_LDS_KB 80
#endif

constexpr int kSmWaves = PN_SM_WAVES;
constexpr int kSmThreads = 64 * kSmWaves;
constexpr int kSmU = PN_SM_ITEMS;
constexpr int kWaveRows = 32;
constexpr int kTileRows = kSmWaves * kWaveRows;
constexpr int kSmLdsMax = PN_SM_LDS_KB * 1024;
constexpr int kSmLdsValu = PN_SM_VALU_LDS_KB * 1024;
constexpr int kMaxM = 16;  // the MFMA tile has 16 activation rows
constexpr int kSmFlagDma = 0x10;  // group plan flag: run by gemm_rows

typedef _Float16 half4_t __attribute__((ext_vector_type(4)));
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// One small-M problem as the device sees it.
struct SmProb {
    const uint8_t *W;  // packed rows
    const uint8_t *X;  // fp16; row m at X + 2 * ldx * m
    float *Y;          // fp32; row m at Y + ldy * m
    int64_t ldx, ldy;  // leading dimensions, elements
    int32_t N, nb;     // rows, blocks per row
    int32_t M, type;
    int32_t tile0;     // first tile of this problem in the launch
    int32_t cb;        // blocks per activation chunk
    int32_t nchunks;
    int32_t stride;    // LDS bytes per staged activation row (256 k + 56 for pn3t, 256 k + 48 for pn4t)
};

#define PN_CONST __attribute__((address_space(4)))

struct SmArgs {
    const PN_CONST SmProb *table;  // device table, or null for the single problem p0
    const PN_CONST uint32_t *lut;  // plans: tile t of the launch is problem lut[t]
    uint32_t *counters;            // gemm_rows plan launches: group counter at [0], finished workgroups at [64]; else null
    SmProb p0;
    int32_t count;
    int32_t total_tiles;
};

// LDS address of byte o of staged activation row m.  Rows are `stride` bytes
// apart: a multiple of 256 plus 56 (pn3t) or 48 (pn4t), so that the distinct
// reads of one operand load (up to 16 rows x 4 lane groups; pn3t reads 8
// bytes at 40g + 8s, pn4t 16 bytes at 32g + 16s) spread over the banks, while
// an operand's address stays a per-lane base plus a constant.  (Measured on
// the M = 16 sweep: pn3t rows 32 bytes past a multiple of 256 2.76 ms a
// token, 24, 40 or 56 bytes 2.54-2.55 ms, an XOR swizzle of 32-byte pieces
// 2.61-2.67 ms with its address arithmetic.)
template <int TYPE>
__device__ __forceinline__ uint32_t xoff(uint32_t m, uint32_t stride, uint32_t o)
{
    return m * stride + o;
}

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>());
        static_for<I + 1, N>(f);
    }
}

// LDS reads issued where they stand (inline asm, so that the compiler cannot
// sink them next to their use) and the wait that retires them, tied to the
// registers they fill: every read must be retired before its registers die.
template <int OFF>
__device__ __forceinline__ u32x2 lds_b64(uint32_t a)
{
    u32x2 r;
    asm volatile("ds_read_b64 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
    return r;
}
template <int OFF>
__device__ __forceinline__ u32x4 lds_b128(uint32_t a)
{
    u32x4 r;
    asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(r) : "v"(a), "i"(OFF));
    return r;
}
template <int OFF0, int OFF1>
__device__ __forceinline__ u32x4 lds_2b64(uint32_t a)
{
    static_assert(OFF0 % 8 == 0 && OFF1 % 8 == 0 && OFF1 / 8 < 256, "ds_read2_b64 offsets");
    u32x4 r;
    asm volatile("ds_read2_b64 %0, %1 offset0:%2 offset1:%3" : "=v"(r) : "v"(a), "i"(OFF0 / 8), "i"(OFF1 / 8));
    return r;
}
// X operands of one block as read (pn3t: 16 + 16 + 8 bytes, pn4t: 16 + 16)
struct XOp {
    u32x4 a, b;
    u32x2 c;
};
template <int N>
__device__ __forceinline__ void lgkm_wait(XOp &x)
{
    asm volatile("s_waitcnt lgkmcnt(%3)" : "+v"(x.a), "+v"(x.b), "+v"(x.c) : "i"(N) : "memory");
}

// Stage activation blocks [b0, b0 + nbc) of all M rows into LDS.  The loads
// are buffer loads like the weight loads: mixing in global (FLAT-family)
// loads makes the compiler's wait analysis drain every load in flight at the
// pipeline's loop head.  Each thread issues up to kStageBatch loads before it
// writes any of them (one memory round trip per batch, not per piece).
template <int TYPE, int NT = kSmThreads>
__device__ __forceinline__ void stage_chunk(const SmProb &p, int b0, int nbc, uint8_t *lds)
{
    constexpr int W = Fmt<TYPE>::W;
    const int per_row = nbc * (W / 8);  // 16-byte pieces per row
    const int total = p.M * per_row;
    const int row_stride = (int)(2 * p.ldx);
    const __amdgpu_buffer_rsrc_t xr =
        make_rsrc(uniform_ptr(p.X + (size_t)2 * b0 * W), (uint32_t)(row_stride * (p.M - 1) + 16 * per_row));
    constexpr int kStageBatch = 4;
    for (int i0 = 0; i0 < total; i0 += kStageBatch * NT) {
        u32x4 v[kStageBatch];
#pragma unroll
        for (int k = 0; k < kStageBatch; ++k) {
            const int i = i0 + k * NT + (int)threadIdx.x;
            const int m = i / per_row, q = i - m * per_row;
            // pieces past the end read zeros (offset past the resource) and are not written
            v[k] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, row_stride * m + 16 * q, 0, 0));
        }
#pragma unroll
        for (int k = 0; k < kStageBatch; ++k) {
            const int i = i0 + k * NT + (int)threadIdx.x;
            const int m = i / per_row, q = i - m * per_row;
            if (i < total) {
                uint8_t *d = lds + xoff<TYPE>((uint32_t)m, (uint32_t)p.stride, 16u * q);
                if constexpr (TYPE == 0) {  // pn3t rows are 8-byte aligned
                    *(u32x2 *)d = (u32x2){v[k][0], v[k][1]};
                    *(u32x2 *)(d + 8) = (u32x2){v[k][2], v[k][3]};
                } else {
                    *(u32x4 *)d = v[k];
                }
            }
        }
    }
}

// One wave's 32 rows of problem p, all blocks.  Every wave of the workgroup
// calls this with the same problem (chunk restaging uses workgroup barriers).
template <int TYPE, bool MFMA>
__device__ __forceinline__ void sm_tile(const SmProb &p, int row0, uint8_t *lds)
{
    constexpr int P = Unpack<TYPE>::kPairs;
    constexpr int U = kSmU;
    const int lane = threadIdx.x & 63;
    // Loads: lane 4j + g reads words 2g, 2g + 1 of row j, so the four lanes of
    // a quad read 32 contiguous bytes of one row.  (The vector memory pipeline
    // takes a quad whose lanes fall in different rows one lane at a time; the
    // MFMA operand layout, where consecutive lanes are consecutive rows, made
    // every quad of every load touch four rows.)
    const int j = lane >> 2, g = lane & 3;
    // MFMA operand layout: lane 16 gm + jm holds row jm, k-group gm; the words
    // move there with ds_bpermute from lane 4 jm + gm.
    const int jm = lane & 15, gm = lane >> 4;
    const int src = 4 * (4 * jm + gm);
    const int nb = uniform(p.nb), cb = uniform(p.cb), M = uniform(p.M);
    const uint32_t stride = (uint32_t)uniform(p.stride);
    const int row_bytes = 34 * nb;
    const int valid = uniform(p.N - row0 < kWaveRows ? p.N - row0 : kWaveRows);  // <= 0: no rows
    // Loads go through a buffer resource over the wave's valid rows: rows past
    // N read zeros.
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(uniform_ptr(p.W + (size_t)(valid > 0 ? row0 : 0) * row_bytes),
                  valid > 0 ? (uint32_t)valid * (uint32_t)row_bytes : 0u);
    const int vs0 = j * row_bytes, vs1 = vs0 + 16 * row_bytes;  // block scale, rows j and 16 + j
    const int vw0 = vs0 + 2 + 8 * g, vw1 = vw0 + 16 * row_bytes;  // words 2g, 2g + 1
    const uint32_t ma = jm < M ? (uint32_t)jm : 0u;  // A row (MFMA); rows >= M are discarded

    constexpr bool kGrouped = MFMA && PN_SM_GROUPED;
    constexpr int S = kGrouped ? 2 * U : U;  // load slots
    uint32_t qw[S][2][2], qs[S][2];
    float4_t accm[2];
    float accv[2][kMaxM];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
        accm[r] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int m = 0; m < kMaxM; ++m) accv[r][m] = 0.0f;
    }
    int ib = 0;                         // next block to load
    int ic = 0;                         // next block to use
    int cbase = 0;                      // first block of the staged chunk
    int cnext = cb < nb ? cb : nb + 1;  // block at which the next chunk is staged

    auto issue = [&](int slot) {
        const int soff = 34 * ib;
        const auto a = __builtin_amdgcn_raw_buffer_load_b64(rs, vw0, soff, 0);
        const auto b = __builtin_amdgcn_raw_buffer_load_b64(rs, vw1, soff, 0);
        qw[slot][0][0] = a[0];
        qw[slot][0][1] = a[1];
        qw[slot][1][0] = b[0];
        qw[slot][1][1] = b[1];
        qs[slot][0] = __builtin_amdgcn_raw_buffer_load_b16(rs, vs0, soff, 0);
        qs[slot][1] = __builtin_amdgcn_raw_buffer_load_b16(rs, vs1, soff, 0);
        ++ib;
    };
    // Chunk boundaries are multiples of U blocks: the restage is checked once
    // per group of U blocks, outside the per-block code, so that the loads in
    // flight stay in their registers across it.
    auto restage = [&]() {
        if (ic == cnext) {
            __syncthreads();
            stage_chunk<TYPE>(p, ic, nb - ic < cb ? nb - ic : cb, lds);
            __syncthreads();
            cbase = ic;
            cnext = ic + cb;
        }
    };
    auto consume = [&](int slot) {
        const uint32_t bl = (uint32_t)(ic - cbase);
        half2_t t[2][2][P];
        float d[2];
        if constexpr (MFMA) {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                const uint32_t w0 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)qw[slot][r][0]);
                const uint32_t w1 = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)qw[slot][r][1]);
                const uint32_t sc = (uint32_t)__builtin_amdgcn_ds_bpermute(src, (int)qs[slot][r]);
                Unpack<TYPE>::run(w0, t[r][0]);
                Unpack<TYPE>::run(w1, t[r][1]);
                d[r] = half_bits_to_float(sc);
            }
        } else {
#pragma unroll
            for (int r = 0; r < 2; ++r) {
                Unpack<TYPE>::run(qw[slot][r][0], t[r][0]);
                Unpack<TYPE>::run(qw[slot][r][1], t[r][1]);
                d[r] = half_bits_to_float(qs[slot][r]);
            }
        }
        if constexpr (MFMA) {
            if constexpr (TYPE == 0) {
                half4_t a[5];
#pragma unroll
                for (int s = 0; s < 5; ++s)
                    a[s] = __builtin_bit_cast(
                        half4_t, *(const u32x2 *)(lds + xoff<0>(ma, stride, 160u * bl + 40u * gm + 8u * s)));
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    // pairs 0..4 from word 2gm, 5..9 from word 2gm + 1; step s takes pairs 2s, 2s + 1
                    const half2_t *u = t[r][0];
                    const half2_t *v = t[r][1];
                    float4_t D = __builtin_amdgcn_mfma_f32_16x16x16f16(
                        a[0], __builtin_shufflevector(u[0], u[1], 0, 1, 2, 3), (float4_t){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                    D = __builtin_amdgcn_mfma_f32_16x16x16f16(a[1], __builtin_shufflevector(u[2], u[3], 0, 1, 2, 3), D, 0, 0, 0);
                    D = __builtin_amdgcn_mfma_f32_16x16x16f16(a[2], __builtin_shufflevector(u[4], v[0], 0, 1, 2, 3), D, 0, 0, 0);
                    D = __builtin_amdgcn_mfma_f32_16x16x16f16(a[3], __builtin_shufflevector(v[1], v[2], 0, 1, 2, 3), D, 0, 0, 0);
                    D = __builtin_amdgcn_mfma_f32_16x16x16f16(a[4], __builtin_shufflevector(v[3], v[4], 0, 1, 2, 3), D, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) accm[r][i] = __builtin_fmaf(D[i], d[r], accm[r][i]);
                }
            } else {
                half8_t a[2];
#pragma unroll
                for (int s = 0; s < 2; ++s)
                    a[s] = __builtin_bit_cast(
                        half8_t, *(const u32x4 *)(lds + xoff<1>(ma, stride, 128u * bl + 32u * gm + 16u * s)));
#pragma unroll
                for (int r = 0; r < 2; ++r) {
                    const half2_t *u = t[r][0];
                    const half2_t *v = t[r][1];
                    const half8_t b0 = __builtin_shufflevector(__builtin_shufflevector(u[0], u[1], 0, 1, 2, 3),
                                                               __builtin_shufflevector(u[2], u[3], 0, 1, 2, 3), 0, 1,
                                                               2, 3, 4, 5, 6, 7);
                    const half8_t b1 = __builtin_shufflevector(__builtin_shufflevector(v[0], v[1], 0, 1, 2, 3),
                                                               __builtin_shufflevector(v[2], v[3], 0, 1, 2, 3), 0, 1,
                                                               2, 3, 4, 5, 6, 7);
                    float4_t D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[0], b0, (float4_t){0.0f, 0.0f, 0.0f, 0.0f},
                                                                        0, 0, 0);
                    D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a[1], b1, D, 0, 0, 0);
#pragma unroll
                    for (int i = 0; i < 4; ++i) accm[r][i] = __builtin_fmaf(D[i], d[r], accm[r][i]);
                }
            }
        } else {
#pragma unroll
            for (int m = 0; m < kMaxM; ++m) {
                if (m < M) {
                    uint32_t xp[2 * P];
                    if constexpr (TYPE == 0) {
#pragma unroll
                        for (int s = 0; s < 5; ++s) {
                            const u32x2 v = *(const u32x2 *)(lds + xoff<0>((uint32_t)m, stride, 160u * bl + 40u * g + 8u * s));
                            xp[2 * s] = v[0];
                            xp[2 * s + 1] = v[1];
                        }
                    } else {
#pragma unroll
                        for (int s = 0; s < 2; ++s) {
                            const u32x4 v = *(const u32x4 *)(lds + xoff<1>((uint32_t)m, stride, 128u * bl + 32u * g + 16u * s));
                            xp[4 * s] = v[0];
                            xp[4 * s + 1] = v[1];
                            xp[4 * s + 2] = v[2];
                            xp[4 * s + 3] = v[3];
                        }
                    }
#pragma unroll
                    for (int r = 0; r < 2; ++r) {
                        const float part = dot_pairs(t[r][1], xp + P, dot_pairs0(t[r][0], xp));
                        accv[r][m] = __builtin_fmaf(d[r], part, accv[r][m]);
                    }
                }
            }
        }
        ++ic;
    };

    if (kGrouped && nb >= 2 * S) {
#pragma unroll
        for (int u = 0; u < S; ++u) {
            issue(u);
            __builtin_amdgcn_sched_barrier(0);
        }
        int done = 0;
        do {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                restage();
#pragma unroll
                for (int u = 0; u < U; ++u) consume(h * U + u);
                __builtin_amdgcn_sched_barrier(0);
#pragma unroll
                for (int u = 0; u < U; ++u) issue(h * U + u);
                __builtin_amdgcn_sched_barrier(0);
            }
            done += S;
        } while (done + 2 * S <= nb);
        // slots hold blocks done .. done + S - 1; fewer than S are unissued
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            restage();
#pragma unroll
            for (int u = 0; u < U; ++u) consume(h * U + u);
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (done + S + h * U + u < nb) issue(h * U + u);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            restage();
#pragma unroll
            for (int u = 0; u < U; ++u)
                if (done + S + h * U + u < nb) consume(h * U + u);
        }
    } else if (nb >= 2 * U) {
        // Slots are issued in order, so that each slot's wait covers its own
        // loads only.
#pragma unroll
        for (int u = 0; u < U; ++u) {
            issue(u);
            __builtin_amdgcn_sched_barrier(0);
        }
        int done = 0;
        do {
            restage();
#pragma unroll
            for (int u = 0; u < U; ++u) {
                consume(u);
                __builtin_amdgcn_sched_barrier(0);
                issue(u);
                __builtin_amdgcn_sched_barrier(0);
            }
            done += U;
        } while (done + 2 * U <= nb);
        restage();
#pragma unroll
        for (int u = 0; u < U; ++u) {
            consume(u);
            if (done + u + U < nb) issue(u);
        }
        restage();
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (done + U + u < nb) consume(u);
    } else {
        for (int i = 0; i < nb; ++i) {
            if (i % U == 0) restage();
            issue(0);
            consume(0);
        }
    }

    if constexpr (MFMA) {
        // lane (jm, gm) holds D[m = 4gm + i][row jm]
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int m = 4 * gm + i, row = 16 * r + jm;
                if (m < M && row < valid) p.Y[p.ldy * m + row0 + row] = accm[r][i];
            }
    } else {
        // add the four lanes (one quad) of each row; lane (j, g) stores m = g (mod 4)
#pragma unroll
        for (int r = 0; r < 2; ++r)
#pragma unroll
            for (int m = 0; m < kMaxM; ++m) {
                if (m < M) {
                    float v = accv[r][m];
                    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xb1, 0xf, 0xf, false));  // quad_perm 1032
                    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4e, 0xf, 0xf, false));  // quad_perm 2301
                    const int row = 16 * r + j;
                    if ((m & 3) == g && row < valid) p.Y[p.ldy * m + row0 + row] = v;
                }
            }
    }
    // Drain the stores before the next tile's loads (one counter covers both
    // on gfx9; a pending store would turn every wait of the next pipeline into
    // a full drain).
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
}

// The problem of `tile`: its index i, its record p and the first tile of
// the next problem (next0), wave-uniform; a plan's records and tile table are
// read with scalar loads.
__device__ __forceinline__ void sm_next_problem(const SmArgs &args, int tile, int &i, int &next0, SmProb &p)
{
    if (!args.table) {
        i = 0;
        p = args.p0;
        next0 = args.total_tiles;
        return;
    }
    i = uniform((int)args.lut[tile]);
    const PN_CONST SmProb &c = args.table[i];
    p.W = uniform_ptr(c.W);
    p.X = uniform_ptr(c.X);
    p.Y = uniform_ptr(c.Y);
    p.ldx = ((int64_t)uniform((int32_t)(c.ldx >> 32)) << 32) | (uint32_t)uniform((int32_t)c.ldx);
    p.ldy = ((int64_t)uniform((int32_t)(c.ldy >> 32)) << 32) | (uint32_t)uniform((int32_t)c.ldy);
    p.N = uniform(c.N);
    p.nb = uniform(c.nb);
    p.M = uniform(c.M);
    p.type = uniform(c.type);
    p.tile0 = uniform(c.tile0);
    p.cb = uniform(c.cb);
    p.nchunks = uniform(c.nchunks);
    p.stride = uniform(c.stride);
    next0 = i + 1 < args.count ? uniform(args.table[i + 1].tile0) : args.total_tiles;
}

// Workgroups take tiles (kSmWaves x 32 rows of one problem) in a grid
// stride.  The activation chunk is restaged when the problem changes, and at
// every chunk boundary of problems whose activations do not fit at once.
template <bool MFMA>
__global__ __launch_bounds__(kSmThreads) void gemm_stream(SmArgs args)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int wave = uniform(threadIdx.x >> 6);
    int i = 0, next0 = -1, staged = -1;
    SmProb p;
    for (int tile = blockIdx.x; tile < args.total_tiles; tile += gridDim.x) {
        if (tile >= next0) sm_next_problem(args, tile, i, next0, p);
        if (p.nchunks > 1 || staged != i) {
            const int nbc = p.nb < p.cb ? p.nb : p.cb;
            __syncthreads();
            if (p.type == 0)
                stage_chunk<0>(p, 0, nbc, lds);
            else
                stage_chunk<1>(p, 0, nbc, lds);
            __syncthreads();
        }
        staged = p.nchunks > 1 ? -1 : i;
        const int row0 = ((tile - p.tile0) * kSmWaves + wave) * kWaveRows;
        if (p.type == 0)
            sm_tile<0, MFMA>(p, row0, lds);
        else
            sm_tile<1, MFMA>(p, row0, lds);
    }
}

// ---------------------------------------------------------------------------
// gemm_rows: the MFMA product with the weights brought to LDS by DMA.
//
// gemm_stream's loads (a dwordx2 per lane, the four lanes of a quad on 32
// bytes of one row, sixteen rows per instruction) cap that kernel near 4 TB/s
// even with its arithmetic taken out: each request carries 32 bytes and
// every 128-byte line is requested four times.  Here a wave owns 16 rows (one
// MFMA column group) and streams them a stage at a time (kDmPPS periods of 8
// blocks: 272 bytes, 17 aligned 16-byte chunks of each row per period) into
// LDS by 16-byte DMA (buffer_load_dwordx4 ... lds), which reads each row's
// stage contiguously; the lanes then read their words and scales in the
// operand layout straight from the stage, so no ds_bpermute is needed, and
// the stage is refilled while they compute: with the tile's next stage, or
// at its last stage with the next tile's first, so that a wave's loads run
// on from tile to tile.  Rows must be whole periods (K a multiple of 640 for
// pn3t, 512 for pn4t) and 16-byte aligned.  The activations are staged per
// workgroup as in gemm_stream, in the LDS the ring leaves free; chunk
// boundaries fall on stages.
//
// Stage layout: row r's periods at byte 272 kDmPPS r (DMA slot 17 kDmPPS r +
// c holds its chunk c).  In each block pair (68 bytes = 17 dwords D) the
// first block's scale is the low half of D[0] and its word j is D[j..j+1]
// shifted by 16 bits; the second block's scale is the high half of D[8] and
// its word j is D[9 + j].  Lane (gm, jm) takes row jm and the block's words
// 2gm, 2gm + 1, the same k-group as gemm_stream's operand layout.
//
// Products: v_mfma_f32_16x16x32_f16, the lane's k-group holding 8 of a
// block's k: pn4t 2 steps (its 16 codes), pn3t 3 steps (its 20 codes, then 4
// zeros in both operands).  The X operands of a block are read from LDS one
// block ahead of their products.
// ---------------------------------------------------------------------------
typedef __attribute__((address_space(3))) void lds_void;

// Waves per workgroup and periods per stage (measured on the M = 8 sweep;
// one stage per wave: a wave reads its stage into registers and refills it
// at once, so that one stage is in flight while it computes).  16 waves of
// one-period stages: four waves per SIMD hide each other's latencies.  Two
// periods a stage read faster (12 waves: 1.97 ms a token with the
// arithmetic taken out, against 2.14 ms) but leave too little LDS for 16
// waves, and with three waves per SIMD the arithmetic no longer hides behind
// the loads (2.46 ms against 2.27 ms).  Earlier forms: 8 waves with two
// one-period stages each 2.66-2.68 ms; three stages left too little LDS for
// the activations (3.03 ms).
#ifndef PN_SM_DMA_WAVES
#define PN_SM_DMA_WAVES 16
#endif
// Tiles a workgroup takes per step of the grid stride: consecutive tiles
// (usually of one problem) share one activation staging.  Measured on the
// M = 8 sweep with 16 waves (256-row tiles): 1 tile 2.54 ms, 2 tiles 2.46, 4
// tiles 2.51, 8 tiles 2.63.
#ifndef PN_SM_DMA_GROUP
#define PN_SM_DMA_GROUP 2
#endif
constexpr int kDmRows = 16;                              // rows per wave
constexpr int kDmWaves = PN_SM_DMA_WAVES;                // waves per workgroup (one workgroup per CU)
constexpr int kDmThreads = 64 * kDmWaves;
constexpr int kDmTileRows = kDmWaves * kDmRows;          // rows per workgroup tile
#ifndef PN_SM_DMA_PPS
#define PN_SM_DMA_PPS 1
#endif
constexpr int kDmPPS = PN_SM_DMA_PPS;                             // periods per stage
constexpr int kDmChunks = 17 * kDmPPS;                            // 16-byte chunks per row and stage
constexpr int kDmDma = (kDmRows * kDmChunks + 63) / 64;           // DMA instructions per stage
constexpr int kDmStage = 16 * kDmRows * kDmChunks;                // LDS bytes per stage (4,352 per period)
constexpr int kDmLast = kDmRows * kDmChunks - 64 * (kDmDma - 1);  // lanes of the last DMA instruction
constexpr int kDmGroup = PN_SM_DMA_GROUP;                         // consecutive tiles per grid-stride step
constexpr int kDmRing = kDmWaves * kDmStage;                      // 68 KiB
constexpr int kDmSlots = kSmLdsMax - 256;                         // LDS: the next group's index (2 slots)
constexpr int kDmLdsX = kDmSlots - kDmRing;                       // activation chunk budget
static_assert(kDmPPS >= 1 && kDmPPS <= 2 && kDmThreads <= 1024 && kDmRing < kSmLdsMax, "ring shape");

// Where one wave's rows of a tile are: the resource covering its valid
// rows (rows past N read zeros and are not stored), the row bytes and the
// number of periods and stages.
struct DmSrc {
    __amdgpu_buffer_rsrc_t rs;
    int32_t S, nper, nst, valid;
};

__device__ __forceinline__ DmSrc dm_src(const SmProb &p, int row0)
{
    DmSrc d;
    const int nb = uniform(p.nb);
    d.S = 34 * nb;
    d.nper = nb >> 3;
    d.nst = (d.nper + kDmPPS - 1) / kDmPPS;
    d.valid = uniform(p.N - row0 < kDmRows ? p.N - row0 : kDmRows);  // <= 0: no rows
    d.rs = make_rsrc(uniform_ptr(p.W + (size_t)(d.valid > 0 ? row0 : 0) * d.S),
                     d.valid > 0 ? (uint32_t)d.valid * (uint32_t)d.S : 0u);
    return d;
}

// Stage s of a tile into `st`: periods kDmPPS s .. of the wave's rows; the
// chunks of periods past the row's end read nothing.  (rr, cc): the lane's
// row and chunk in each DMA instruction's slot.
__device__ __forceinline__ void dm_issue(const DmSrc &d, int s, uint8_t *st, const uint32_t (&rr)[kDmDma],
                                         const uint32_t (&cc)[kDmDma], int lane)
{
    const uint32_t lim = 17u * (uint32_t)(d.nper - kDmPPS * s);  // chunks left in the row
#pragma unroll
    for (int i = 0; i < kDmDma; ++i) {
        const uint32_t o = rr[i] < (uint32_t)kDmRows && (kDmPPS == 1 || cc[i] < lim)
                               ? rr[i] * (uint32_t)d.S + 16u * cc[i]
                               : 0x80000000u;
        if (i < kDmDma - 1 || lane < kDmLast)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(d.rs, (lds_void *)(st + 1024 * i), 16, (int)o, 272 * kDmPPS * s, 0,
                                                     0);
    }
}

// One tile of one wave.  Its stage 0 was issued by the caller; while its last
// stage is computed, the next tile's stage 0 (nx, when has_next) is already
// in flight.
template <int TYPE>
__device__ __forceinline__ void dm_tile(const SmProb &p, int row0, const DmSrc &d, const DmSrc &nx, bool has_next,
                                        uint8_t *lds, uint8_t *ring, const uint32_t (&rr)[kDmDma],
                                        const uint32_t (&cc)[kDmDma])
{
    constexpr int P = Unpack<TYPE>::kPairs;
    const int lane = threadIdx.x & 63;
    const int jm = lane & 15, gm = lane >> 4;  // operand layout: row jm, k-group gm
    const int nb = uniform(p.nb), cb = uniform(p.cb), M = uniform(p.M);
    const int nper = d.nper, nst = d.nst;
    const uint32_t stride = (uint32_t)uniform(p.stride);
    const uint32_t ma = jm < M ? (uint32_t)jm : 0u;  // A row; rows >= M are discarded
    float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};

    int cbase = 0;                      // first block of the staged chunk
    int cnext = cb < nb ? cb : nb + 1;  // block at which the next chunk is staged
    // a tile has at least one stage (rows are whole periods): a do-while, so
    // that every path through a tile passes its stage waits
    int s = 0;
    do {
        const int b0 = 8 * kDmPPS * s;
        const int nv = nper - kDmPPS * s < kDmPPS ? nper - kDmPPS * s : kDmPPS;  // periods in this stage
        if (b0 == cnext) {
            // every wave of the workgroup is on this problem and stage
            __syncthreads();
            stage_chunk<TYPE, kDmThreads>(p, b0, nb - b0 < cb ? nb - b0 : cb, lds);
            // (the staging loads are younger than the ring's DMA, so the ring
            // has landed too; saying so on every path keeps the compiler from
            // draining the ring at every stage for loads it thinks pending)
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            __syncthreads();
            cbase = b0;
            cnext = b0 + cb;
        }
        __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0): the stage (and the last tile's stores)
        // the lane's words and scales of each period: per block pair,
        // D[2gm .. 2gm + 2], D[9 + 2gm], D[10 + 2gm], D[0], D[8]
        const uint32_t *rw = (const uint32_t *)(ring + 272 * kDmPPS * jm);
        uint32_t wa[kDmPPS][4][3], wb[kDmPPS][4][2], sa[kDmPPS][4], sb[kDmPPS][4];
#pragma unroll
        for (int pp = 0; pp < kDmPPS; ++pp)
#pragma unroll
            for (int bp = 0; bp < 4; ++bp) {
                const int o = 68 * pp + 17 * bp;
#pragma unroll
                for (int j = 0; j < 3; ++j) wa[pp][bp][j] = rw[o + 2 * gm + j];
                wb[pp][bp][0] = rw[o + 9 + 2 * gm];
                wb[pp][bp][1] = rw[o + 10 + 2 * gm];
                sa[pp][bp] = rw[o];
                sb[pp][bp] = rw[o + 8];
            }
        // the stage is refilled once its reads have landed: with this tile's
        // next stage, or the next tile's first
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        if (s + 1 < nst)
            dm_issue(d, s + 1, ring, rr, cc, lane);
        else if (has_next)
            dm_issue(nx, 0, ring, rr, cc, lane);
        __builtin_amdgcn_sched_barrier(0);
        constexpr uint32_t kBB = TYPE == 0 ? 160u : 128u;  // X bytes per block and row
        const uint32_t xs = (uint32_t)(size_t)(lds_void *)(lds + ma * stride + (TYPE == 0 ? 40u : 32u) * (uint32_t)gm +
                                                          kBB * (uint32_t)(b0 - cbase));
        constexpr int NQ = 8 * kDmPPS;         // blocks of a stage
        constexpr int XR = TYPE == 0 ? 3 : 2;  // X read instructions per block
        // X operands of block q (the lane's 40 or 32 bytes), read one block
        // ahead straight into the registers the MFMAs take (nothing may copy
        // them before the wait that retires the reads)
        auto xread = [&](auto qc, XOp &x) {
            constexpr int q = decltype(qc)::value, o = (int)kBB * (q % 8);
            const uint32_t a = xs + 8u * kBB * (uint32_t)(q / 8);
            if constexpr (TYPE == 0) {
                x.a = lds_2b64<o, o + 8>(a);
                x.b = lds_2b64<o + 16, o + 24>(a);
                x.c = lds_b64<o + 32>(a);
            } else {
                x.a = lds_b128<o>(a);
                x.b = lds_b128<o + 16>(a);
                x.c = (u32x2){0u, 0u};
            }
        };
        XOp xa, xb;
        xread(std::integral_constant<int, 0>(), xa);
        auto block = [&](auto qc) {
            constexpr int q = decltype(qc)::value, pp = q / 8, b = q % 8, bp = b >> 1;
            XOp &xc = q % 2 == 0 ? xa : xb;
            XOp &xn = q % 2 == 0 ? xb : xa;
            if constexpr (q + 1 < NQ) {
                xread(std::integral_constant<int, q + 1>(), xn);
                lgkm_wait<XR>(xc);
            } else {
                lgkm_wait<0>(xc);
            }
            uint32_t w0, w1, sc;
            if (b & 1) {
                w0 = wb[pp][bp][0];
                w1 = wb[pp][bp][1];
                sc = sb[pp][bp] >> 16;
            } else {
                w0 = __builtin_amdgcn_alignbit(wa[pp][bp][1], wa[pp][bp][0], 16);
                w1 = __builtin_amdgcn_alignbit(wa[pp][bp][2], wa[pp][bp][1], 16);
                sc = sa[pp][bp] & 0xffffu;
            }
            half2_t u[P], v[P];
            Unpack<TYPE>::run(w0, u);
            Unpack<TYPE>::run(w1, v);
            const float d = half_bits_to_float(sc);
            float4_t D;
            const half8_t a0 = __builtin_bit_cast(half8_t, xc.a), a1 = __builtin_bit_cast(half8_t, xc.b);
            if constexpr (TYPE == 0) {
                // k-steps of 32: the lane's codes 0-7, 8-15 and 16-19 (then four zeros) of its 20
                const half8_t a2 = __builtin_bit_cast(half8_t, (u32x4){xc.c[0], xc.c[1], 0u, 0u});
                const half2_t z = {0.0f16, 0.0f16};
                const half8_t b0v = __builtin_shufflevector(__builtin_shufflevector(u[0], u[1], 0, 1, 2, 3),
                                                            __builtin_shufflevector(u[2], u[3], 0, 1, 2, 3), 0, 1, 2,
                                                            3, 4, 5, 6, 7);
                const half8_t b1v = __builtin_shufflevector(__builtin_shufflevector(u[4], v[0], 0, 1, 2, 3),
                                                            __builtin_shufflevector(v[1], v[2], 0, 1, 2, 3), 0, 1, 2,
                                                            3, 4, 5, 6, 7);
                const half8_t b2v = __builtin_shufflevector(__builtin_shufflevector(v[3], v[4], 0, 1, 2, 3),
                                                            __builtin_shufflevector(z, z, 0, 1, 2, 3), 0, 1, 2, 3, 4,
                                                            5, 6, 7);
                D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0v, (float4_t){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1v, D, 0, 0, 0);
                D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a2, b2v, D, 0, 0, 0);
            } else {
                const half8_t b0v = __builtin_shufflevector(__builtin_shufflevector(u[0], u[1], 0, 1, 2, 3),
                                                            __builtin_shufflevector(u[2], u[3], 0, 1, 2, 3), 0, 1, 2,
                                                            3, 4, 5, 6, 7);
                const half8_t b1v = __builtin_shufflevector(__builtin_shufflevector(v[0], v[1], 0, 1, 2, 3),
                                                            __builtin_shufflevector(v[2], v[3], 0, 1, 2, 3), 0, 1, 2,
                                                            3, 4, 5, 6, 7);
                D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a0, b0v, (float4_t){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
                D = __builtin_amdgcn_mfma_f32_16x16x32_f16(a1, b1v, D, 0, 0, 0);
            }
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(D[i], d, acc[i]);
        };
        // periods past the row's end (the last stage of a row may hold fewer)
        // are skipped; the X read issued ahead for the first of them is retired
        static_for<0, kDmPPS>([&](auto pc) {
            constexpr int pp = decltype(pc)::value;
            if (pp == 0 || nv > pp)
                static_for<8 * pp, 8 * pp + 8>(block);
            else if (nv == pp)
                lgkm_wait<0>(xa);
        });
    } while (++s < nst);
    // lane (jm, gm) holds D[m = 4gm + i][row jm]
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int m = 4 * gm + i;
        if (m < M && jm < d.valid) p.Y[p.ldy * m + row0 + jm] = acc[i];
    }
}

// Workgroups take groups of kDmGroup consecutive tiles (kDmWaves x 16 rows
// of one problem each; the activations staged for a problem serve every
// tile of a group).  Workgroup b's first group is group b; a single call
// then takes every gridDim-th group after it, and a plan launch takes its
// later groups from the plan's counter (one atomic per group, issued a group
// ahead by one lane and handed to the other waves through LDS), so that
// workgroups that finish early take more: a plan's problems repeat with a
// period that a grid stride can map onto the same XCDs every time (the
// 27B-shaped layer has 104 groups, so its heavy down-projection groups
// fell twice on XCDs 6 and 7 and once on the others in all 64 layers, and
// those two XCDs ended the M = 8 sweep 17 % after the rest).  The last
// workgroup to finish resets the counters for the plan's next run.  The
// ring sits above the activation chunk, and a wave's stages run on from
// one tile into the next without draining.
__global__ __launch_bounds__(kDmThreads) void gemm_rows(SmArgs args)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int wave = uniform(threadIdx.x >> 6);
    const int lane = threadIdx.x & 63;
    uint8_t *ring = lds + kDmLdsX + wave * kDmStage;
    uint32_t *slot = (uint32_t *)(lds + kDmSlots);
    uint32_t rr[kDmDma], cc[kDmDma];
#pragma unroll
    for (int i = 0; i < kDmDma; ++i) {
        const uint32_t q = 64u * i + (uint32_t)lane;
        rr[i] = q / kDmChunks;
        cc[i] = q - kDmChunks * rr[i];
    }
    const int groups = (args.total_tiles + kDmGroup - 1) / kDmGroup;
    const bool dyn = args.counters != nullptr;
    const bool grabber = dyn && wave == 0 && lane == 0;
    auto count_done = [&]() {
        if (grabber) {
            const uint32_t d = __hip_atomic_fetch_add(args.counters + 64, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (d == gridDim.x - 1) {  // every workgroup has made its last grab
                __hip_atomic_store(args.counters, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(args.counters + 64, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    };
    int gcur = (int)blockIdx.x;
    if (gcur >= groups) {
        count_done();
        return;
    }
    // The grab: an atomic add issued from inline asm, its result register
    // tied in and out, so that the compiler neither reads it at once (its own
    // atomic waited for the result right away, draining the stage in flight)
    // nor copies it before the atomic has written it.  It is read at the next
    // group, after the stage waits (vmcnt(0)) of at least one tile.
    uint32_t gr = 0;  // the grabbing lane: result of the outstanding grab
    auto grab = [&]() {
        asm volatile("global_atomic_add %0, %1, %2, off sc0" : "+v"(gr) : "v"(args.counters), "v"(1u) : "memory");
    };
    if (grabber) {
        grab();
        asm volatile("s_waitcnt vmcnt(0)" : "+v"(gr) :: "memory");  // nothing else is in flight yet
    }
    int gj = 0, gafter = 0;  // gcur's ordinal among the workgroup's groups; the group after it
    auto next_group = [&]() {  // every wave: gafter from gcur
        if (!dyn) {
            gafter = gcur + (int)gridDim.x;
            return;
        }
        if (grabber) {
            asm volatile("" : "+v"(gr) :: "memory");  // read only here, after the stage waits
            const uint32_t ga = gridDim.x + gr;
            slot[gj & 1] = ga;
            if ((int)ga < groups) grab();
        }
        // a bare barrier (__syncthreads' fence would drain the stage in
        // flight); the slot's write has left the wave before it
        __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        gafter = uniform((int)slot[gj & 1]);
    };
    auto tile_of = [&](int g, int s) {  // tile s of group g, or -1
        const int t = g * kDmGroup + s;
        return g < groups && t < args.total_tiles ? t : -1;
    };
    next_group();
    int sub = 0;
    int t = tile_of(gcur, 0);
    int i = 0, next0 = -1, staged = -1;
    SmProb p;
    sm_next_problem(args, t, i, next0, p);
    int row0 = ((t - p.tile0) * kDmWaves + wave) * kDmRows;
    DmSrc d = dm_src(p, row0);
    dm_issue(d, 0, ring, rr, cc, lane);
    // Each pass computes one tile, and a workgroup of a correct run computes
    // at most every tile of the launch (grabbed groups only grow); the cap ends
    // the loop all the same if the plan's counter was disturbed, e.g. by a
    // plan run concurrently with itself.  It is the same for every wave of the
    // workgroup, so they leave together.
    int passes = 0;
    for (;;) {
        // the next tile (of this group, or the first of the next), looked up
        // ahead so that its first stage can be issued early
        const int ts = sub + 1 < kDmGroup ? tile_of(gcur, sub + 1) : -1;
        const int tn = ts >= 0 ? ts : tile_of(gafter, 0);
        SmProb pn = p;
        int in = i, nn = next0, rn = 0;
        DmSrc dn = d;
        if (tn >= 0) {
            if (tn >= nn) sm_next_problem(args, tn, in, nn, pn);
            rn = ((tn - pn.tile0) * kDmWaves + wave) * kDmRows;
            dn = dm_src(pn, rn);
        }
        if (p.nchunks > 1 || staged != i) {
            const int nbc = p.nb < p.cb ? p.nb : p.cb;
            __syncthreads();
            if (p.type == 0)
                stage_chunk<0, kDmThreads>(p, 0, nbc, lds);
            else
                stage_chunk<1, kDmThreads>(p, 0, nbc, lds);
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0), on every path (see dm_tile)
            __syncthreads();
        }
        staged = p.nchunks > 1 ? -1 : i;
        if (p.type == 0)
            dm_tile<0>(p, row0, d, dn, tn >= 0, lds, ring, rr, cc);
        else
            dm_tile<1>(p, row0, d, dn, tn >= 0, lds, ring, rr, cc);
        if (tn < 0 || ++passes >= args.total_tiles) break;
        if (ts >= 0) {
            ++sub;
        } else {
            gcur = gafter;
            sub = 0;
            ++gj;
            next_group();
        }
        p = pn;
        i = in;
        next0 = nn;
        row0 = rn;
        d = dn;
    }
    // no DMA or store may be outstanding when the wave ends
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
    count_done();
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
// Per device: workgroups per CU by arithmetic and LDS KiB (0 = not queried
// yet; concurrent queries of one entry compute and store the same value).
struct SmDevice {
    std::atomic<signed char> occ[2][161];
};
SmDevice g_sm[kMaxDevices];

// Activation chunks above 64 KiB need the kernels' LDS limit raised (once
// per device).
bool set_smallm_attr()
{
    return hipFuncSetAttribute((const void *)gemm_stream<true>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               kSmLdsMax) == hipSuccess &&
           hipFuncSetAttribute((const void *)gemm_stream<false>, hipFuncAttributeMaxDynamicSharedMemorySize,
                               kSmLdsMax) == hipSuccess &&
           hipFuncSetAttribute((const void *)gemm_rows, hipFuncAttributeMaxDynamicSharedMemorySize, kSmLdsMax) ==
               hipSuccess;
}

int sm_wgs_per_cu(bool mfma, int lds)
{
    const int dev = current_device() < 0 ? 0 : current_device();
    SmDevice &d = g_sm[dev];
    int q = (lds + 1023) / 1024;
    q = q < 0 ? 0 : (q > 160 ? 160 : q);
    std::atomic<signed char> &slot = d.occ[mfma ? 1 : 0][q];
    signed char o = slot.load(std::memory_order_relaxed);
    if (o == 0) {
        int occ = 0;
        const hipError_t e = mfma ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_stream<true>, kSmThreads,
                                                                                  (size_t)q * 1024)
                                  : hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemm_stream<false>, kSmThreads,
                                                                                  (size_t)q * 1024);
        if (e != hipSuccess || occ <= 0) occ = 1;
        o = (signed char)(occ > 127 ? 127 : occ);
        slot.store(o, std::memory_order_relaxed);
    }
    return o;
}

// Can gemm_rows take this problem?  Rows of whole periods (K a multiple of
// 640 for pn3t, 512 for pn4t), W 16-byte aligned, 16-row offsets within the
// kernel's 32-bit arithmetic, the MFMA arithmetic, and a kernel choice that
// allows it (pn_set_gemv_kernel: anything but PN_GEMV_STREAM).
bool sm_dma_ok(int t, const void *W, int64_t K, bool mfma)
{
    if (!mfma || gemv_kernel_choice() == PN_GEMV_STREAM) return false;
    if (((uintptr_t)W & 15) != 0) return false;
    const int64_t nb = K / wpb(t);
    return nb % 8 == 0 && nb * 34 * kDmRows <= INT32_MAX;
}

// Fill an SmProb for one problem (validated) and choose its activation
// chunking: the fewest chunks of whole blocks whose M staged rows fit the LDS
// budget, equal in size up to U blocks (every boundary a multiple of U), or
// up to stages for gemm_rows (dma), whose ring takes part of the LDS.  Rows are
// padded to 56 (pn3t) or 48 (pn4t) bytes past a multiple of 256 (xoff).
pn_status sm_make(int t, const void *W, int64_t N, int64_t K, const void *X, int64_t ldx, int M, float *Y,
                  int64_t ldy, bool mfma, bool dma, SmProb &p)
{
    pn_status st = check_matrix(t, W, N, K);
    if (st) return st;
    if (!X || !Y) return PN_EINVAL;
    if (M < 1 || M > kMaxM || ldx < K || ldy < N || (ldx & 1)) return PN_ESHAPE;
    if (!aligned4(X) || !aligned4(Y)) return PN_EALIGN;
    if (2 * ldx * M > INT32_MAX) return PN_EUNSUPPORTED;  // activation offsets are 32-bit
    const int64_t nb = K / wpb(t);
    if (nb * 34 * kWaveRows > INT32_MAX) return PN_EUNSUPPORTED;  // per-wave offsets are 32-bit
    const int64_t bytes_per_block = (int64_t)wpb(t) * 2;              // staged bytes per block and row
    const int64_t unit = dma ? 8 * kDmPPS : kSmU;  // chunk boundaries at multiples of this many blocks
    const int64_t budget = dma ? kDmLdsX : mfma ? kSmLdsMax : kSmLdsValu;
    int64_t nchunks = 1, cb = nb, stride = 0;
    for (;; ++nchunks) {
        cb = (nb + nchunks - 1) / nchunks;
        if (cb < nb) cb = (cb + unit - 1) / unit * unit;
        stride = (cb * bytes_per_block + 255) / 256 * 256 + (t == 0 ? 56 : 48);
        if (stride * M <= budget) break;
        if (cb <= unit) return PN_EUNSUPPORTED;
    }
    memset(&p, 0, sizeof(p));
    p.W = (const uint8_t *)W;
    p.X = (const uint8_t *)X;
    p.Y = Y;
    p.ldx = ldx;
    p.ldy = ldy;
    p.N = (int32_t)N;
    p.nb = (int32_t)nb;
    p.M = M;
    p.type = t;
    p.cb = (int32_t)cb;
    p.nchunks = (int32_t)((nb + cb - 1) / cb);
    p.stride = (int32_t)stride;
    return PN_OK;
}

int sm_lds(const SmProb &p) { return p.M * p.stride; }

// A small-M plan's device memory: the problem table, the tile table (the
// problem of each tile), then for gemm_rows the group counter ([0]) and the
// count of finished workgroups ([64]).
constexpr size_t kSmCounterBytes = 512;
size_t sm_lut_offset(int count) { return (sizeof(SmProb) * (size_t)count + 15) & ~(size_t)15; }
size_t sm_counter_offset(int count, int tiles)
{
    return (sm_lut_offset(count) + sizeof(uint32_t) * (size_t)tiles + 255) & ~(size_t)255;
}

pn_status sm_launch(const SmArgs &a, int lds, bool mfma, bool dma, hipStream_t s, int variant)
{
    if (!once_per_device(kAttrSmallM, set_smallm_attr)) return PN_ELAUNCH;
    int grid = device_cus() * (dma ? 1 : sm_wgs_per_cu(mfma, lds));  // gemm_rows takes the whole LDS
    if (grid > a.total_tiles) grid = a.total_tiles;
    if (grid < 1) grid = 1;
    if (dma)
        hipLaunchKernelGGL(gemm_rows, dim3(grid), dim3(kDmThreads), kSmLdsMax, s, a);
    else if (mfma)
        hipLaunchKernelGGL(gemm_stream<true>, dim3(grid), dim3(kSmThreads), lds, s, a);
    else
        hipLaunchKernelGGL(gemm_stream<false>, dim3(grid), dim3(kSmThreads), lds, s, a);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    g_last_variant = variant;
    return PN_OK;
}

}  // namespace

pn_status pn::host::smallm_group_run(const pn_group *g, hipStream_t s)
{
    SmArgs a;
    memset(&a, 0, sizeof(a));
    a.table = (const PN_CONST SmProb *)g->table;
    a.lut = (const PN_CONST uint32_t *)((const uint8_t *)g->table + sm_lut_offset(g->count));
    a.count = g->count;
    a.total_tiles = g->total_tiles;
    const bool mfma = (g->flags & 0xf) == PN_SMALLM_MFMA;
    const bool dma = (g->flags & kSmFlagDma) != 0;
    if (dma) a.counters = (uint32_t *)((uint8_t *)g->table + sm_counter_offset(g->count, g->total_tiles));
    return sm_launch(a, g->lds, mfma, dma, s,
                     dma ? kVarGroupSmallMRows : mfma ? kVarGroupSmallMMfma : kVarGroupSmallMValu);
}

extern "C" {

pn_status pn_gemm_smallm(pn_type t, const void *W, int64_t N, int64_t K, const void *X, int64_t ldx, int M,
                         float *Y, int64_t ldy, void *stream)
{
    SmArgs a;
    memset(&a, 0, sizeof(a));
    const bool mfma = smallm_math_choice() == PN_SMALLM_MFMA;
    const bool dma = type_ok(t) && W && K >= wpb(t) && sm_dma_ok(t, W, K, mfma);
    pn_status st = sm_make(t, W, N, K, X, ldx, M, Y, ldy, mfma, dma, a.p0);
    if (st) return st;
    const int64_t rows = dma ? kDmTileRows : kTileRows;
    a.count = 1;
    a.total_tiles = (int32_t)((N + rows - 1) / rows);
    return sm_launch(a, sm_lds(a.p0), mfma, dma, (hipStream_t)stream,
                     dma ? kVarSmallMRows : mfma ? kVarSmallMMfma : kVarSmallMValu);
}

pn_status pn_group_create_smallm(const pn_gemm_desc *descs, int count, pn_group **out)
{
    if (!descs || !out || count < 1) return PN_EINVAL;
    *out = nullptr;
    SmProb *host = (SmProb *)calloc((size_t)count, sizeof(SmProb));
    if (!host) return PN_ENOMEM;
    int lds = 0;
    int64_t tiles = 0;
    pn_status st = PN_OK;
    const int math = smallm_math_choice();
    // gemm_rows runs the plan if it takes every problem (one launch, one kernel)
    bool dma = true;
    for (int i = 0; i < count && dma; ++i) {
        const pn_gemm_desc &e = descs[i];
        dma = type_ok(e.type) && e.W && e.K >= wpb(e.type) && sm_dma_ok(e.type, e.W, e.K, math == PN_SMALLM_MFMA);
    }
    const int64_t rows = dma ? kDmTileRows : kTileRows;
    for (int i = 0; i < count && st == PN_OK; ++i) {
        const pn_gemm_desc &e = descs[i];
        st = sm_make(e.type, e.W, e.N, e.K, e.X, e.ldx, e.M, e.Y, e.ldy, math == PN_SMALLM_MFMA, dma, host[i]);
        if (st != PN_OK) break;
        if (sm_lds(host[i]) > lds) lds = sm_lds(host[i]);
    }
    // The launch takes the problems' tiles in the table's order, longest rows
    // first (stable), so that the last tiles handed out are short ones: the
    // 27B-shaped layer's down projection (9,248-byte rows) in layer order
    // left one workgroup on a 4.7 MB group 0.25 ms after the others.
    if (st == PN_OK)
        std::stable_sort(host, host + count, [](const SmProb &x, const SmProb &y) { return x.nb > y.nb; });
    for (int i = 0; i < count && st == PN_OK; ++i) {
        host[i].tile0 = (int32_t)tiles;
        tiles += (host[i].N + rows - 1) / rows;
        if (tiles > INT32_MAX) st = PN_EUNSUPPORTED;
    }
    if (st != PN_OK) {
        free(host);
        return st;
    }
    pn_group *g = (pn_group *)calloc(1, sizeof(pn_group));
    if (!g) {
        free(host);
        return PN_ENOMEM;
    }
    if (current_device() < 0) {
        free(host);
        free(g);
        return PN_EUNSUPPORTED;
    }
    // the problem table, the tile table, then (gemm_rows) the group counter
    // and the count of finished workgroups, zero, 256 bytes apart
    const size_t lut_off = sm_lut_offset(count), coff = sm_counter_offset(count, (int)tiles);
    const size_t bytes = coff + (dma ? kSmCounterBytes : 0);
    uint8_t *blob = (uint8_t *)calloc(1, bytes);
    if (!blob) {
        free(host);
        free(g);
        return PN_ENOMEM;
    }
    memcpy(blob, host, sizeof(SmProb) * (size_t)count);
    uint32_t *lut = (uint32_t *)(blob + lut_off);
    for (int i = 0; i < count; ++i) {
        const int64_t end = i + 1 < count ? host[i + 1].tile0 : tiles;
        for (int64_t t = host[i].tile0; t < end; ++t) lut[t] = (uint32_t)i;
    }
    free(host);
    if (hipMalloc(&g->table, bytes) != hipSuccess) {
        free(blob);
        free(g);
        return PN_ENOMEM;
    }
    if (hipMemcpy(g->table, blob, bytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(g->table);
        free(blob);
        free(g);
        return PN_ELAUNCH;
    }
    free(blob);
    g->kind = kGroupSmallM;
    g->device = current_device();
    g->count = count;
    g->total_tiles = (int)tiles;
    g->lds = lds;
    g->flags = math | (dma ? kSmFlagDma : 0);
    *out = g;
    return PN_OK;
}

}  // extern "C"
