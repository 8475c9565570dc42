// pn_kernels.hip - PN decode GEMV kernels for AMD Instinct MI355X (gfx950)
// and the C ABI declared in include/pn.h.
//
// The hot path is the decode-time matrix-vector product over PN-packed rows
// (tensorless, "Why a P100-native weight format"; "Why the P100", section
// "Why memory bandwidth sets the pace": every weight is read once per token,
// so the product is bound by HBM bandwidth).
//
// Kernels
//   gemv_stream   M = 1, one launch for 1..n independent problems.  Persistent
//                 workgroups; the activation lives in LDS; each wave streams R
//                 rows at once, one code word per lane per row ("One lane, one
//                 word"), so one LDS read of x serves R rows.
//   gemv_generic  M = 1 fallback for shapes gemv_stream does not take (x too
//                 large for LDS): one wave per row, x from global memory.
//   gemm_smallm   M <= 8: x chunks for all M rows staged in LDS, each weight
//                 decoded once and used M times.
//   dequant       dense fp32 weights, bit-exact.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include "pn_device.h"
#include "../../include/pn.h"

using namespace pn;

namespace {

constexpr int kWaves = 4;               // waves per workgroup
constexpr int kThreads = 64 * kWaves;   // workgroup size
constexpr int kMaxLdsBytes = 64 * 1024; // LDS the streaming kernels may use

enum Variant {
    kVarNone = 0,
    kVarStream = 1,
    kVarGeneric = 2,
    kVarSmallM = 3,
    kVarDequant = 4,
    kVarGroupStream = 5,
};

thread_local int g_last_variant = kVarNone;

// One GEMV problem as the device sees it.
struct Prob {
    const uint8_t *W;   // packed rows
    const uint8_t *x;   // fp16 [K]
    float *y;           // fp32 [N]
    int32_t N;          // rows
    int32_t nw;         // code words per row = 8 * K / W
    int32_t type;       // 0 = pn3t, 1 = pn4t
    int32_t tile0;      // first global tile index of this problem
};

// Kernel arguments: up to two problems inline (pn_gemv, pn_gemv2), or a
// device table for larger groups.
struct StreamArgs {
    const Prob *table;
    Prob p0, p1;
    int32_t count;
    int32_t total_tiles;
};

// ---------------------------------------------------------------------------
// Activation staging into LDS.  Word f of a row multiplies x[C*f .. C*f+C-1].
// pn4t: LDS holds x as is (16 bytes per word).  pn3t: the first 8 values of
// each word go to a 16-byte array and the last 2 to a 4-byte array, so that
// every lane reads its word's activations with one ds_read_b128 and one
// ds_read_b32, both naturally aligned and conflict-free.  Words past the end
// of the row (a ragged last pass) read zeros.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void stage_x(const Prob &p, int nwp, uint8_t *lds)
{
    const int nw = p.nw;
    if (p.type == 0) {
        uint4 *a = (uint4 *)lds;
        uint32_t *b = (uint32_t *)(lds + 16 * nwp);
        for (int f = threadIdx.x; f < nwp; f += kThreads) {
            uint4 va = make_uint4(0, 0, 0, 0);
            uint32_t vb = 0;
            if (f < nw) {
                const uint8_t *src = p.x + 20 * (size_t)f;
                va = make_uint4(load_u32(src), load_u32(src + 4), load_u32(src + 8), load_u32(src + 12));
                vb = load_u32(src + 16);
            }
            a[f] = va;
            b[f] = vb;
        }
    } else {
        uint4 *a = (uint4 *)lds;
        for (int f = threadIdx.x; f < nwp; f += kThreads) {
            uint4 va = make_uint4(0, 0, 0, 0);
            if (f < nw) {
                const uint8_t *src = p.x + 16 * (size_t)f;
                va = make_uint4(load_u32(src), load_u32(src + 4), load_u32(src + 8), load_u32(src + 12));
            }
            a[f] = va;
        }
    }
}

// Byte offset of code word f inside a row, and of its block's scale.
__device__ __forceinline__ uint32_t word_off(uint32_t f) { return 34u * (f >> 3) + 2u + 4u * (f & 7u); }
__device__ __forceinline__ uint32_t scale_off(uint32_t f) { return 34u * (f >> 3); }

// One wave streams `nrows` consecutive rows of one problem (nrows <= 64),
// R rows at a time, one code word per lane per row ("One lane, one word").
// The loads form one continuous pipeline of "items" (R rows x one pass of 64
// words = 8 blocks = 272 bytes per row) with U items in flight; prefetch runs
// across row groups, so the load stream never drains until the wave's last
// row.  All loads go through one buffer resource that covers the wave's valid
// rows: rows past N read zeros (no clamping, no fault).  Finished row sums are
// parked in lane (row - row0) of one register and stored once at the end.
// Requires nw % 64 == 0 (K a multiple of 8 blocks).
template <int TYPE, int R, int U>
__device__ __forceinline__ void stream_wave(const Prob &p, int row0, int nrows, int nwp, const uint8_t *lds)
{
    constexpr int P = Unpack<TYPE>::kPairs;
    constexpr int kPassBytes = 64 / kWordsPerBlock * kBlockBytes;  // 272
    const int lane = threadIdx.x & 63;
    const int nfull = uniform(p.nw >> 6);
    const int row_bytes = uniform((p.nw >> 3) * 34);
    const int valid = uniform(p.N - row0 < nrows ? p.N - row0 : nrows);
    const int total = uniform(((nrows + R - 1) / R) * nfull);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(uniform_ptr(p.W + (size_t)row0 * row_bytes), (uint32_t)valid * (uint32_t)row_bytes);
    const int wo = (int)word_off(lane), so = (int)scale_off(lane);
    const int lds_lane = lane * 16;

    uint32_t qw[U][R], qs[U][R];
    float acc[R];
#pragma unroll
    for (int r = 0; r < R; ++r) acc[r] = 0.0f;
    float res = 0.0f;
    int ig = 0, ip = 0;  // issue cursor: row group, pass
    int cg = 0, cp = 0;  // consume cursor

    auto issue = [&](int slot) {
        const int soff = ig * R * row_bytes + ip * kPassBytes;
#pragma unroll
        for (int r = 0; r < R; ++r) {
            qw[slot][r] = __builtin_amdgcn_raw_buffer_load_b32(rs, wo, soff + r * row_bytes, 0);
            qs[slot][r] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, soff + r * row_bytes, 0);
        }
        if (++ip == nfull) { ip = 0; ++ig; }
    };
    auto consume = [&](int slot) {
        uint32_t xp[P];
        {
            const uint8_t *lx = lds + lds_lane + cp * 1024;
            const uint4 a = *(const uint4 *)lx;
            xp[0] = a.x; xp[1] = a.y; xp[2] = a.z; xp[3] = a.w;
            if (TYPE == 0) xp[4] = *(const uint32_t *)(lds + 16 * nwp + lane * 4 + cp * 256);
        }
#pragma unroll
        for (int r = 0; r < R; ++r) {
            half2_t t[P];
            Unpack<TYPE>::run(qw[slot][r], t);
            acc[r] = __builtin_fmaf(half_bits_to_float(qs[slot][r]), dot_pairs0(t, xp), acc[r]);
        }
        if (++cp == nfull) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const float v = wave_sum(acc[r]);
                res = lane == cg * R + r ? v : res;
                acc[r] = 0.0f;
            }
            cp = 0;
            ++cg;
        }
    };

    if (total >= 2 * U) {
        // The prologue is unconditional, so every path into the loop has the
        // same loads outstanding in the same order and each slot's wait
        // covers only its own loads.
#pragma unroll
        for (int u = 0; u < U; ++u) issue(u);
        int done = 0;
        do {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                consume(u);
                __builtin_amdgcn_sched_barrier(0);
                issue(u);
                __builtin_amdgcn_sched_barrier(0);
            }
            done += U;
        } while (done + 2 * U <= total);
        // slots hold items done .. done+U-1; fewer than U items are unissued
#pragma unroll
        for (int u = 0; u < U; ++u) {
            consume(u);
            if (done + u + U < total) issue(u);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (done + U + u < total) consume(u);
    } else {
        for (int i = 0; i < total; ++i) {
            issue(0);
            consume(0);
        }
    }

    if (lane < valid) p.y[row0 + lane] = res;
    // Drain the store before the next tile's loads: gfx9 counts stores and
    // loads in one counter, and a pending store would make every wait in the
    // next pipeline a full drain.
    __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
}

template <int R, int U>
__global__ __launch_bounds__(kThreads) void gemv_stream(StreamArgs args, int rows_per_wave)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int wave = uniform(threadIdx.x >> 6);
    const int tile_rows = kWaves * rows_per_wave;

    int cur = -1;
    Prob p;
    int nwp = 0;
    int tile_end = 0;
    for (int tile = blockIdx.x; tile < args.total_tiles; tile += gridDim.x) {
        if (tile >= tile_end || cur < 0) {
            // Find the problem holding this tile (tiles only move forward).
            int i = cur < 0 ? 0 : cur;
            for (;;) {
                Prob c = args.table ? args.table[i] : (i == 0 ? args.p0 : args.p1);
                int next0 = (i + 1 < args.count)
                                ? (args.table ? args.table[i + 1].tile0 : args.p1.tile0)
                                : args.total_tiles;
                if (tile < next0) {
                    p.W = uniform_ptr(c.W);
                    p.x = uniform_ptr(c.x);
                    p.y = uniform_ptr(c.y);
                    p.N = uniform(c.N);
                    p.nw = uniform(c.nw);
                    p.type = uniform(c.type);
                    p.tile0 = uniform(c.tile0);
                    tile_end = uniform(next0);
                    break;
                }
                ++i;
            }
            cur = i;
            nwp = p.nw;
            __syncthreads();
            stage_x(p, nwp, lds);
            __syncthreads();
        }
        const int row0 = (tile - p.tile0) * tile_rows + wave * rows_per_wave;
        if (row0 < p.N) {
            if (p.type == 0)
                stream_wave<0, R, U>(p, row0, rows_per_wave, nwp, lds);
            else
                stream_wave<1, R, U>(p, row0, rows_per_wave, nwp, lds);
        }
    }
}

// ---------------------------------------------------------------------------
// Generic M = 1 path: one wave per row, activations from global memory.
// ---------------------------------------------------------------------------
template <int TYPE>
__global__ __launch_bounds__(kThreads) void gemv_generic(Prob p0, Prob p1)
{
    constexpr int P = Unpack<TYPE>::kPairs;
    constexpr int C = Fmt<TYPE>::C;
    const Prob &p = blockIdx.y == 0 ? p0 : p1;
    const int lane = threadIdx.x & 63;
    const int64_t row = (int64_t)blockIdx.x * kWaves + uniform(threadIdx.x >> 6);
    if (row >= p.N) return;
    const uint8_t *rowp = uniform_ptr(p.W + row * (int64_t)(p.nw >> 3) * 34);
    float acc = 0.0f;
    for (int f = lane; f < p.nw; f += 64) {
        const uint32_t q = load_u32_a2(rowp + word_off(f));
        const uint32_t s = load_u16(rowp + scale_off(f));
        const uint8_t *xs = p.x + (size_t)f * C * 2;
        uint32_t xp[P];
#pragma unroll
        for (int i = 0; i < P; ++i) xp[i] = load_u32(xs + 4 * i);
        acc = __builtin_fmaf(half_bits_to_float(s), dot_word<TYPE>(q, xp, 0.0f), acc);
    }
    const float v = wave_sum(acc);
    if (lane == 0) p.y[row] = v;
}

// ---------------------------------------------------------------------------
// Small M (1..8).  A workgroup owns kWaves * R rows; K is walked in chunks of
// kChunkWords code words; each chunk's activations for all M rows are staged
// in LDS (same split layout as stage_x).  A lane decodes its word once per
// row and feeds M dot products.
// ---------------------------------------------------------------------------
constexpr int kChunkWords = 256;

template <int TYPE, int MMAX, int R>
__global__ __launch_bounds__(kThreads) void gemm_smallm(const uint8_t *W, int N, int nw,
                                                        const uint8_t *X, int64_t ldx_bytes, int M,
                                                        float *Y, int64_t ldy)
{
    constexpr int P = Unpack<TYPE>::kPairs;
    constexpr int C = Fmt<TYPE>::C;
    __shared__ __attribute__((aligned(16))) uint8_t lds[MMAX * kChunkWords * C * 2];
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const uint32_t row_bytes = (uint32_t)(nw >> 3) * 34u;
    const int tiles = (N + kWaves * R - 1) / (kWaves * R);

    for (int tile = blockIdx.x; tile < tiles; tile += gridDim.x) {
        const int row0 = tile * kWaves * R + wave * R;
        const uint8_t *rowp[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            int rr = row0 + r < N ? row0 + r : N - 1;
            rowp[r] = uniform_ptr(W + (size_t)rr * row_bytes);
        }
        float acc[R][MMAX];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int m = 0; m < MMAX; ++m) acc[r][m] = 0.0f;

        for (int c0 = 0; c0 < nw; c0 += kChunkWords) {
            const int cw = nw - c0 < kChunkWords ? nw - c0 : kChunkWords;
            __syncthreads();
            // stage X[:, C*c0 .. C*(c0+cw)) ; per m a region of kChunkWords*C*2 bytes
            for (int i = threadIdx.x; i < M * kChunkWords; i += kThreads) {
                const int m = i / kChunkWords, f = i % kChunkWords;
                uint8_t *base = lds + (size_t)m * kChunkWords * C * 2;
                if (TYPE == 0) {
                    uint4 va = make_uint4(0, 0, 0, 0);
                    uint32_t vb = 0;
                    if (f < cw) {
                        const uint8_t *src = X + m * ldx_bytes + (size_t)(c0 + f) * 20;
                        va = make_uint4(load_u32(src), load_u32(src + 4), load_u32(src + 8), load_u32(src + 12));
                        vb = load_u32(src + 16);
                    }
                    ((uint4 *)base)[f] = va;
                    ((uint32_t *)(base + 16 * kChunkWords))[f] = vb;
                } else {
                    uint4 va = make_uint4(0, 0, 0, 0);
                    if (f < cw) {
                        const uint8_t *src = X + m * ldx_bytes + (size_t)(c0 + f) * 16;
                        va = make_uint4(load_u32(src), load_u32(src + 4), load_u32(src + 8), load_u32(src + 12));
                    }
                    ((uint4 *)base)[f] = va;
                }
            }
            __syncthreads();
            if (row0 < N) {
                for (int fl = lane; fl < cw; fl += 64) {
                    const uint32_t f = (uint32_t)(c0 + fl);
                    half2_t t[R][P];
                    float d[R];
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        Unpack<TYPE>::run(load_u32_a2(rowp[r] + word_off(f)), t[r]);
                        d[r] = half_bits_to_float(load_u16(rowp[r] + scale_off(f)));
                    }
#pragma unroll
                    for (int m = 0; m < MMAX; ++m) {
                        if (m < M) {
                            const uint8_t *base = lds + (size_t)m * kChunkWords * C * 2;
                            uint32_t xp[P];
                            const uint4 a = ((const uint4 *)base)[fl];
                            xp[0] = a.x; xp[1] = a.y; xp[2] = a.z; xp[3] = a.w;
                            if (TYPE == 0) xp[P - 1] = ((const uint32_t *)(base + 16 * kChunkWords))[fl];
#pragma unroll
                            for (int r = 0; r < R; ++r)
                                acc[r][m] = __builtin_fmaf(d[r], dot_pairs(t[r], xp, 0.0f), acc[r][m]);
                        }
                    }
                }
            }
        }
        if (row0 < N) {
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
                for (int m = 0; m < MMAX; ++m) {
                    if (m < M) {
                        const float v = wave_sum(acc[r][m]);
                        if (lane == 0 && row0 + r < N) Y[(int64_t)m * ldy + row0 + r] = v;
                    }
                }
        }
    }
}

// ---------------------------------------------------------------------------
// Dequantization: one thread per code word, C fp32 outputs each.
// out = d * (float)(n - z): one binary32 multiply of two exact values.
// ---------------------------------------------------------------------------
template <int TYPE>
__global__ __launch_bounds__(256) void dequant(const uint8_t *W, int64_t N, int64_t nw, float *out)
{
    constexpr int C = Fmt<TYPE>::C, B = Fmt<TYPE>::B, Z = Fmt<TYPE>::Z;
    const int64_t total = N * nw;
    const int64_t row_bytes = (nw >> 3) * 34;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        const int64_t r = g / nw;
        const uint32_t f = (uint32_t)(g - r * nw);
        const uint8_t *rowp = W + r * row_bytes;
        const uint32_t q = load_u32_a2(rowp + word_off(f));
        const float d = half_bits_to_float(load_u16(rowp + scale_off(f)));
        float *o = out + r * (nw / 8) * (8 * C) + (int64_t)f * C;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int n = (int)((q >> (16 * (j & 1) + B * (j >> 1))) & ((1u << B) - 1u));
            o[j] = d * (float)(n - Z);
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int kR = 2;   // rows per group in gemv_stream
constexpr int kU = 4;   // items (passes of 8 blocks x R rows) in flight per wave

struct DeviceInfo {
    int cus = 0;
    int occ[5] = {0, 0, 0, 0, 0};  // gemv_stream workgroups per CU, by LDS quarter (16 KB steps)
};

DeviceInfo g_dev[64];

const DeviceInfo &device_info()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
    DeviceInfo &d = g_dev[dev];
    if (d.cus == 0) {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        for (int q = 0; q < 5; ++q) {
            int occ = 0;
            const size_t lds = (size_t)(q == 0 ? 1 : q * 16) * 1024;
            if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemv_stream<kR, kU>, kThreads, lds) !=
                    hipSuccess ||
                occ <= 0)
                occ = 1;
            d.occ[q] = occ;
        }
        d.cus = cus;
    }
    return d;
}

int stream_wgs_per_cu(const DeviceInfo &d, int lds)
{
    const int q = (lds + 16 * 1024 - 1) / (16 * 1024);
    return d.occ[q < 0 ? 0 : (q > 4 ? 4 : q)];
}

bool type_ok(int t) { return t == PN_PN3T || t == PN_PN4T; }
int wpb(int t) { return t == PN_PN3T ? 80 : 64; }

pn_status check_matrix(int t, const void *W, int64_t N, int64_t K)
{
    if (!type_ok(t) || !W) return PN_EINVAL;
    if (N < 1 || K < wpb(t) || K % wpb(t) != 0) return PN_ESHAPE;
    if ((uintptr_t)W & 1) return PN_EALIGN;
    if (N > INT32_MAX || K / wpb(t) * 34 > INT32_MAX) return PN_EUNSUPPORTED;
    return PN_OK;
}

bool aligned4(const void *p) { return ((uintptr_t)p & 3) == 0; }

Prob make_prob(int t, const void *W, int64_t N, int64_t K, const void *x, float *y)
{
    Prob p;
    p.W = (const uint8_t *)W;
    p.x = (const uint8_t *)x;
    p.y = y;
    p.N = (int32_t)N;
    p.nw = (int32_t)(K / wpb(t) * 8);
    p.type = t;
    p.tile0 = 0;
    return p;
}

int lds_bytes_for(const Prob &p) { return p.type == 0 ? 20 * p.nw : 16 * p.nw; }

// gemv_stream takes rows made of whole passes (8 blocks) whose activation
// fits in LDS, and rows of at most 32 MiB.
bool stream_ok(const Prob &p)
{
    return (p.nw & 63) == 0 && lds_bytes_for(p) <= kMaxLdsBytes;
}

// Rows per wave: enough waves to fill the device, at most 64 rows (one
// result lane each), a multiple of kR.
int rows_per_wave(int64_t total_rows, int lds)
{
    const DeviceInfo &d = device_info();
    const int64_t waves = (int64_t)d.cus * stream_wgs_per_cu(d, lds) * kWaves;
    int64_t rw = (total_rows + waves - 1) / waves;
    rw = (rw + kR - 1) / kR * kR;
    if (rw < kR) rw = kR;
    if (rw > 64) rw = 64;
    return (int)rw;
}

int64_t tiles_of(const Prob &p, int rw) { return ((int64_t)p.N + kWaves * rw - 1) / (kWaves * rw); }

pn_status launch_stream(StreamArgs &a, int lds, int rw, hipStream_t s, int variant)
{
    const DeviceInfo &d = device_info();
    int grid = d.cus * stream_wgs_per_cu(d, lds);
    if (grid > a.total_tiles) grid = a.total_tiles;
    if (grid < 1) grid = 1;
    hipLaunchKernelGGL((gemv_stream<kR, kU>), dim3(grid), dim3(kThreads), lds, s, a, rw);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    g_last_variant = variant;
    return PN_OK;
}

pn_status launch_generic(const Prob &p0, const Prob &p1, int nprob, hipStream_t s)
{
    const int64_t N = p0.N > p1.N ? p0.N : p1.N;
    dim3 grid((unsigned)((N + kWaves - 1) / kWaves), (unsigned)nprob);
    if (p0.type == 0)
        hipLaunchKernelGGL(gemv_generic<0>, grid, dim3(kThreads), 0, s, p0, p1);
    else
        hipLaunchKernelGGL(gemv_generic<1>, grid, dim3(kThreads), 0, s, p0, p1);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    g_last_variant = kVarGeneric;
    return PN_OK;
}

}  // namespace

// ===========================================================================
// C ABI
// ===========================================================================
extern "C" {

int pn_weights_per_block(pn_type t) { return type_ok(t) ? wpb(t) : 0; }

size_t pn_row_bytes(pn_type t, int64_t K)
{
    if (!type_ok(t) || K < wpb(t) || K % wpb(t) != 0) return 0;
    return (size_t)(K / wpb(t)) * 34u;
}

pn_status pn_gemv(pn_type t, const void *W, int64_t N, int64_t K, const void *x, float *y, void *stream)
{
    pn_status st = check_matrix(t, W, N, K);
    if (st) return st;
    if (!x || !y) return PN_EINVAL;
    if (!aligned4(x) || !aligned4(y)) return PN_EALIGN;
    Prob p = make_prob(t, W, N, K, x, y);
    hipStream_t s = (hipStream_t)stream;
    if (!stream_ok(p)) return launch_generic(p, p, 1, s);
    const int lds = lds_bytes_for(p);
    const int rw = rows_per_wave(p.N, lds);
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.p0 = p;
    a.p1 = p;
    a.count = 1;
    a.total_tiles = (int32_t)tiles_of(p, rw);
    return launch_stream(a, lds, rw, s, kVarStream);
}

pn_status pn_gemv2(pn_type t, const void *W0, const void *W1, int64_t N, int64_t K, const void *x, float *y0,
                   float *y1, void *stream)
{
    pn_status st = check_matrix(t, W0, N, K);
    if (st) return st;
    st = check_matrix(t, W1, N, K);
    if (st) return st;
    if (!x || !y0 || !y1) return PN_EINVAL;
    if (!aligned4(x) || !aligned4(y0) || !aligned4(y1)) return PN_EALIGN;
    Prob p0 = make_prob(t, W0, N, K, x, y0);
    Prob p1 = make_prob(t, W1, N, K, x, y1);
    hipStream_t s = (hipStream_t)stream;
    if (!stream_ok(p0)) return launch_generic(p0, p1, 2, s);
    const int lds = lds_bytes_for(p0);
    const int rw = rows_per_wave(2 * (int64_t)p0.N, lds);
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    p1.tile0 = (int32_t)tiles_of(p0, rw);
    a.p0 = p0;
    a.p1 = p1;
    a.count = 2;
    a.total_tiles = p1.tile0 + (int32_t)tiles_of(p1, rw);
    return launch_stream(a, lds, rw, s, kVarStream);
}

pn_status pn_gemm_smallm(pn_type t, const void *W, int64_t N, int64_t K, const void *X, int64_t ldx, int M,
                         float *Y, int64_t ldy, void *stream)
{
    pn_status st = check_matrix(t, W, N, K);
    if (st) return st;
    if (!X || !Y) return PN_EINVAL;
    if (M < 1 || M > 8 || ldx < K || ldy < N || (ldx & 1)) return PN_ESHAPE;
    if (!aligned4(X) || !aligned4(Y)) return PN_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    const int nw = (int)(K / wpb(t) * 8);
    const DeviceInfo &d = device_info();
    constexpr int R = 2;
    const int tiles = (int)((N + kWaves * R - 1) / (kWaves * R));
    int grid = d.cus * 2;
    if (grid > tiles) grid = tiles;
    if (t == PN_PN3T)
        hipLaunchKernelGGL((gemm_smallm<0, 8, R>), dim3(grid), dim3(kThreads), 0, s, (const uint8_t *)W, (int)N,
                           nw, (const uint8_t *)X, ldx * 2, M, Y, ldy);
    else
        hipLaunchKernelGGL((gemm_smallm<1, 8, R>), dim3(grid), dim3(kThreads), 0, s, (const uint8_t *)W, (int)N,
                           nw, (const uint8_t *)X, ldx * 2, M, Y, ldy);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    g_last_variant = kVarSmallM;
    return PN_OK;
}

pn_status pn_dequantize(pn_type t, const void *W, int64_t N, int64_t K, float *out, void *stream)
{
    pn_status st = check_matrix(t, W, N, K);
    if (st) return st;
    if (!out) return PN_EINVAL;
    if (!aligned4(out)) return PN_EALIGN;
    hipStream_t s = (hipStream_t)stream;
    const int64_t nw = K / wpb(t) * 8;
    int64_t blocks = (N * nw + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    if (t == PN_PN3T)
        hipLaunchKernelGGL(dequant<0>, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t *)W, N, nw, out);
    else
        hipLaunchKernelGGL(dequant<1>, dim3((unsigned)blocks), dim3(256), 0, s, (const uint8_t *)W, N, nw, out);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    g_last_variant = kVarDequant;
    return PN_OK;
}

struct pn_group {
    Prob *table;      // device
    int count;
    int total_tiles;
    int lds;
    int rows_per_wave;
};

pn_status pn_group_create(const pn_gemv_desc *descs, int count, pn_group **out)
{
    if (!descs || !out || count < 1) return PN_EINVAL;
    *out = nullptr;
    Prob *host = (Prob *)calloc((size_t)count, sizeof(Prob));
    if (!host) return PN_ENOMEM;
    int lds = 0;
    int64_t rows = 0;
    pn_status st = PN_OK;
    for (int i = 0; i < count && st == PN_OK; ++i) {
        const pn_gemv_desc &e = descs[i];
        st = check_matrix(e.type, e.W, e.N, e.K);
        if (st == PN_OK && (!e.x || !e.y)) st = PN_EINVAL;
        if (st == PN_OK && (!aligned4(e.x) || !aligned4(e.y))) st = PN_EALIGN;
        if (st == PN_OK) {
            host[i] = make_prob(e.type, e.W, e.N, e.K, e.x, e.y);
            if (!stream_ok(host[i])) st = PN_EUNSUPPORTED;
        }
        if (st == PN_OK) {
            rows += host[i].N;
            if (lds_bytes_for(host[i]) > lds) lds = lds_bytes_for(host[i]);
        }
    }
    const int rw = st == PN_OK ? rows_per_wave(rows, lds) : 0;
    int64_t tiles = 0;
    for (int i = 0; i < count && st == PN_OK; ++i) {
        host[i].tile0 = (int32_t)tiles;
        tiles += tiles_of(host[i], rw);
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
    if (hipMalloc((void **)&g->table, sizeof(Prob) * (size_t)count) != hipSuccess) {
        free(host);
        free(g);
        return PN_ENOMEM;
    }
    if (hipMemcpy(g->table, host, sizeof(Prob) * (size_t)count, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(g->table);
        free(host);
        free(g);
        return PN_ELAUNCH;
    }
    free(host);
    g->count = count;
    g->total_tiles = (int)tiles;
    g->lds = lds;
    g->rows_per_wave = rw;
    *out = g;
    return PN_OK;
}

pn_status pn_group_run(const pn_group *g, void *stream)
{
    if (!g) return PN_EINVAL;
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.table = g->table;
    a.count = g->count;
    a.total_tiles = g->total_tiles;
    return launch_stream(a, g->lds, g->rows_per_wave, (hipStream_t)stream, kVarGroupStream);
}

void pn_group_destroy(pn_group *g)
{
    if (!g) return;
    (void)hipDeviceSynchronize();
    (void)hipFree(g->table);
    free(g);
}

const char *pn_status_str(pn_status e)
{
    switch (e) {
    case PN_OK: return "ok";
    case PN_EINVAL: return "invalid argument (null pointer, unknown type or count)";
    case PN_ESHAPE: return "bad shape (N < 1, K not a positive multiple of the block size, M or ld out of range)";
    case PN_EALIGN: return "misaligned pointer (W needs 2-byte, x/X/y/Y/out 4-byte alignment)";
    case PN_EUNSUPPORTED: return "shape not supported by the kernels";
    case PN_ELAUNCH: return "HIP launch or runtime call failed";
    case PN_ENOMEM: return "device allocation failed";
    }
    return "unknown status";
}

int pn_last_variant(void) { return g_last_variant; }

const char *pn_variant_name(int v)
{
    switch (v) {
    case kVarNone: return "none";
    case kVarStream: return "gemv_stream";
    case kVarGeneric: return "gemv_generic";
    case kVarSmallM: return "gemm_smallm_valu";
    case kVarDequant: return "dequant";
    case kVarGroupStream: return "gemv_stream_group";
    }
    return "unknown";
}

}  // extern "C"
