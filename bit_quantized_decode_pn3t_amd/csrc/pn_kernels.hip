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
//   dequant       dense fp32 weights, bit-exact.
// The small-batch (M <= 8) kernels are in pn_smallm.hip.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>

#include "pn_device.h"
#include "pn_host.h"

using namespace pn;
using namespace pn::host;

thread_local int pn::host::g_last_variant = pn::host::kVarNone;

namespace {

#ifndef PN_WAVES
#define PN_WAVES 4
#endif
#ifndef PN_ROWS_PER_GROUP
#define PN_ROWS_PER_GROUP 2
#endif
#ifndef PN_ITEMS_IN_FLIGHT
#define PN_ITEMS_IN_FLIGHT 4
#endif
// Cache policy bits of the weight loads (2 = nontemporal).  Plain loads are
// the default: the scale loads touch the cache lines the word loads just
// fetched, and nontemporal word loads make those second touches miss.
#ifndef PN_WEIGHT_AUX
#define PN_WEIGHT_AUX 0
#endif
// With two words per lane, take the block scale from the words' own 12-byte
// window (one dwordx3 load per lane and row instead of a dwordx2 and a
// ushort).  Off by default: measured slower on MI355X.
#ifndef PN_SCALE_IN_WINDOW
#define PN_SCALE_IN_WINDOW 0
#endif

constexpr int kWaves = PN_WAVES;        // waves per workgroup
constexpr int kThreads = 64 * kWaves;   // workgroup size
constexpr int kMaxLdsBytes = 64 * 1024; // LDS the streaming kernels may use

// One GEMV problem as the device sees it.
struct Prob {
    const uint8_t *W;   // packed rows
    const uint8_t *x;   // fp16 [K]
    float *y;           // fp32 [N]
    int32_t N;          // rows
    int32_t nw;         // code words per row = 8 * K / W
    int32_t type;       // 0 = pn3t, 1 = pn4t
    int32_t tile0;      // first global tile index of this problem
    int32_t rpw;        // rows per wave in this problem's tiles
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
// With V words per lane, word f = V*j + v goes to slot v, entry j, so that
// the 64 lanes of a pass read 64 consecutive 16-byte entries of one slot
// (one conflict-free ds_read_b128 per word).  pn4t: entry = the word's 8
// activations (16 bytes).  pn3t: the first 8 go to a 16-byte entry, the last 2
// to a 4-byte entry in a second array (one ds_read_b128 + one ds_read_b32,
// both aligned).  LDS bytes: 16*nw (+ 4*nw for pn3t) = 2*K.
// ---------------------------------------------------------------------------
// Entry e of slot v holds word f = V * (e - v * per) + v.  The entries are
// filled by DMA (buffer_load ... lds, 16 bytes a lane, plus 4 for pn3t's
// second array): lane l of instruction i fetches entry 64 i + l, so the
// instruction writes 1 KiB (256 bytes) of LDS in order, and no register
// holds the activation on its way.  The workgroup's waves issue its
// instructions round-robin, all at once, and a wave issues its first weight
// loads right behind them; it waits for its own DMA and meets the others at
// a barrier only then, so the activation's latency hides under the
// weights'.  (Staged through registers, four entries in flight a thread,
// the staging made the kernel's register peak, and one round trip a batch
// came before the first weight load: the layer schedule 0.883 vs 0.842 ms
// per 16 layers, the per-matrix schedule 1.148 vs 1.073, the single calls
// 3-6 % slower.  Eight entries a batch took 88 VGPRs and five workgroups a
// CU.)  Needs nw % 64 == 0: whole instructions, none writing past the
// arrays.  The caller waits (vmcnt) and synchronises before any read.
typedef __attribute__((address_space(3))) void lds_void_t;
template <int TYPE, int V>
__device__ __forceinline__ void stage_x_dma(const Prob &p, uint8_t *lds, int wave, int lane)
{
    constexpr int kEntry = TYPE == 0 ? 20 : 16;  // activation bytes per word
    const int nw = p.nw;
    const int per = nw / V;  // entries per slot
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(uniform_ptr(p.x), (uint32_t)(kEntry * nw));
    for (int i = wave; i < nw / 64; i += kWaves) {
        const int e = 64 * i + lane;
        const int v = e / per;
        const int off = kEntry * (V * (e - v * per) + v);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t *)(lds + 1024 * i), 16, off, 0, 0, 0);
        if constexpr (TYPE == 0)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(xr, (lds_void_t *)(lds + 16 * nw + 256 * i), 4, off + 16, 0, 0, 0);
    }
}

// Byte offset of code word f inside a row, and of its block's scale.
__device__ __forceinline__ uint32_t word_off(uint32_t f) { return 34u * (f >> 3) + 2u + 4u * (f & 7u); }
__device__ __forceinline__ uint32_t scale_off(uint32_t f) { return 34u * (f >> 3); }

// One wave streams `nrows` consecutive rows of one problem (nrows <= 64),
// R rows at a time.  Lane l of a pass owns V consecutive code words of one
// block ("One lane, one word", widened to V words so that one unaligned
// buffer_load covers them and they share one scale).  The loads form one
// continuous pipeline of "items" (R rows x one pass of 64*V words = 8*V
// blocks) with U items in flight; prefetch runs across row groups, so the
// load stream never drains until the wave's last row.  All loads go through
// one buffer resource that covers the wave's valid rows: rows past N read
// zeros (no clamping, no fault).  Finished row sums are parked in lane
// (row - row0) of one register and stored once at the end.  With `restage`
// the workgroup's activation DMA was issued just before: the wave waits for
// it behind its first weight loads and meets the other waves at a barrier
// (a wave without rows, nrows = 0, only waits and meets them).
// Requires nw % (64 * V) == 0.
template <int TYPE, int R, int U, int V>
__device__ __forceinline__ void stream_wave(const Prob &p, int row0, int nrows, const uint8_t *lds, bool restage)
{
    constexpr int P = Unpack<TYPE>::kPairs;
    constexpr int kPassBytes = 8 * V * kBlockBytes;  // 272 * V
    const int lane = threadIdx.x & 63;
    const int nw = uniform(p.nw);
    const int npass = nw / (64 * V);
    const int row_bytes = uniform((nw >> 3) * 34);
    const int valid0 = uniform(p.N - row0 < nrows ? p.N - row0 : nrows);
    const int valid = valid0 < 0 ? 0 : valid0;
    const int total = uniform(((nrows + R - 1) / R) * npass);
    const __amdgpu_buffer_rsrc_t rs =
        make_rsrc(uniform_ptr(p.W + (size_t)row0 * row_bytes), (uint32_t)valid * (uint32_t)row_bytes);
    const int wo = (int)word_off((uint32_t)(V * lane)), so = (int)scale_off((uint32_t)(V * lane));
    const int per = nw / V;
    typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
    const u32x4 *lds_a = (const u32x4 *)lds + lane;
    const uint32_t *lds_b = (const uint32_t *)(lds + 16 * nw) + lane;
    // Scale in the words' window (V == 2): lane q = lane & 3 of a block owns
    // words 2q and 2q+1 and loads 12 bytes at block offset 8q (q < 3) or 22
    // (q = 3), always inside the block.  Its words start at window byte 2
    // (q < 3) or 4 (q = 3); v_perm_b32 picks them with a per-lane selector,
    // and lane q = 0 holds the block's scale in its first two bytes.
    constexpr bool kSiw = V == 2 && PN_SCALE_IN_WINDOW;
    const int q4 = lane & 3;
    const int wwo = so + (q4 < 3 ? 8 * q4 : 22);
    const uint32_t wsel = q4 < 3 ? 0x05040302u : 0x07060504u;

    uint32_t qw[U][R][V], qs[U][R];
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
            if constexpr (kSiw) {
                const auto w3 = __builtin_amdgcn_raw_buffer_load_b96(rs, wwo, soff + r * row_bytes, PN_WEIGHT_AUX);
                qw[slot][r][0] = w3[0];
                qw[slot][r][V - 1] = w3[1];
                qs[slot][r] = w3[2];
            } else if constexpr (V == 1) {
                qw[slot][r][0] = __builtin_amdgcn_raw_buffer_load_b32(rs, wo, soff + r * row_bytes, PN_WEIGHT_AUX);
                qs[slot][r] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, soff + r * row_bytes, PN_WEIGHT_AUX);
            } else {
                const auto v2 = __builtin_amdgcn_raw_buffer_load_b64(rs, wo, soff + r * row_bytes, PN_WEIGHT_AUX);
                qw[slot][r][0] = v2[0];
                qw[slot][r][V - 1] = v2[1];
                qs[slot][r] = __builtin_amdgcn_raw_buffer_load_b16(rs, so, soff + r * row_bytes, PN_WEIGHT_AUX);
            }
        }
        if (++ip == npass) { ip = 0; ++ig; }
    };
    auto consume = [&](int slot) {
        float part[R];
        uint32_t words[R][V], scale[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            if constexpr (kSiw) {
                const uint32_t d0 = qw[slot][r][0], d1 = qw[slot][r][V - 1], d2 = qs[slot][r];
                words[r][0] = __builtin_amdgcn_perm(d1, d0, wsel);
                words[r][V - 1] = __builtin_amdgcn_perm(d2, d1, wsel);
                scale[r] = (uint32_t)__builtin_amdgcn_mov_dpp((int)d0, 0x00, 0xf, 0xf, false);  // quad_perm [0,0,0,0]
            } else {
#pragma unroll
                for (int v = 0; v < V; ++v) words[r][v] = qw[slot][r][v];
                scale[r] = qs[slot][r];
            }
        }
#pragma unroll
        for (int v = 0; v < V; ++v) {
            uint32_t xp[P];
            const u32x4 a = lds_a[v * per + cp * 64];
            xp[0] = a[0]; xp[1] = a[1]; xp[2] = a[2]; xp[3] = a[3];
            if constexpr (TYPE == 0) xp[P - 1] = lds_b[v * per + cp * 64];
#pragma unroll
            for (int r = 0; r < R; ++r) {
                half2_t t[P];
                Unpack<TYPE>::run(words[r][v], t);
                part[r] = v == 0 ? dot_pairs0(t, xp) : dot_pairs(t, xp, part[r]);
            }
        }
#pragma unroll
        for (int r = 0; r < R; ++r) acc[r] = __builtin_fmaf(half_bits_to_float(scale[r]), part[r], acc[r]);
        if (++cp == npass) {
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
        if (restage) {
            // the activation's DMA (issued before these loads) has landed for
            // this wave; after the barrier, for every wave.  The prologue's
            // loads: one per row and item with the scale in the words'
            // window, else two (words, scale).
            constexpr int kPro = U * R * (kSiw ? 1 : 2);
            static_assert(kPro < 64, "vmcnt immediate");
            __builtin_amdgcn_s_waitcnt((((kPro >> 4) & 3) << 14) | 0x0f70 | (kPro & 15));
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
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
        if (restage) {
            __builtin_amdgcn_s_waitcnt(0x0f70);  // vmcnt(0)
            asm volatile("" ::: "memory");
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
        }
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

// Problem i of a launch (inline for one or two problems, else the table).
__device__ __forceinline__ const Prob *problem(const StreamArgs &a, int i)
{
    if (a.table) return a.table + i;
    return i == 0 ? &a.p0 : &a.p1;
}

__device__ __forceinline__ int problem_tile0(const StreamArgs &a, int i)
{
    if (i >= a.count) return a.total_tiles;
    if (a.table) return a.table[i].tile0;
    return i == 0 ? a.p0.tile0 : a.p1.tile0;
}

// Workgroups take tiles in a grid stride: at any moment the workgroups work on
// neighbouring tiles, i.e. one contiguous stretch of the weights, which the
// memory system serves better than scattered streams.  A workgroup stages
// the activation into LDS whenever its next tile belongs to another problem.
template <int R, int U, int V>
__global__ __launch_bounds__(kThreads) void gemv_stream(StreamArgs args)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int wave = uniform(threadIdx.x >> 6);
    int i = 0;
    int next0 = -1;  // first tile of problem i + 1; -1 before the first problem
    Prob p;
    bool restage = false;
    for (int tile = blockIdx.x; tile < args.total_tiles; tile += gridDim.x) {
        if (tile >= next0) {
            // advance to the problem holding this tile (tiles only move forward)
            if (next0 >= 0) ++i;
            while (problem_tile0(args, i + 1) <= tile) ++i;
            const Prob &c = *problem(args, i);
            p.W = uniform_ptr(c.W);
            p.x = uniform_ptr(c.x);
            p.y = uniform_ptr(c.y);
            p.N = uniform(c.N);
            p.nw = uniform(c.nw);
            p.type = uniform(c.type);
            p.tile0 = uniform(c.tile0);
            p.rpw = uniform(c.rpw);
            next0 = uniform(problem_tile0(args, i + 1));
            restage = true;
            // every wave is done reading the previous activation
            __syncthreads();
            if (p.type == 0)
                stage_x_dma<0, V>(p, lds, wave, (int)(threadIdx.x & 63));
            else
                stage_x_dma<1, V>(p, lds, wave, (int)(threadIdx.x & 63));
        }
        const int row0 = ((tile - p.tile0) * kWaves + wave) * p.rpw;
        // waves without rows still wait for the staging with the others
        if (row0 < p.N || restage) {
            const int nrows = row0 < p.N ? p.rpw : 0;
            if (p.type == 0)
                stream_wave<0, R, U, V>(p, row0, nrows, lds, restage);
            else
                stream_wave<1, R, U, V>(p, row0, nrows, lds, restage);
        }
        restage = false;
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

// The plan of pn_gemv_batch (callers that cannot allocate): one buffer per
// device, held until the process ends.  Host code never uses this name as an
// address: batch_buffer() gets each device's copy with hipGetSymbolAddress.
static __device__ __align__(256) uint8_t scratch[kBatchBytes];

// The register-pipeline kernel's batch plan: the problem table, copied from
// the kernel arguments into the batch buffer.
struct SBatch {
    Prob p[kBatchMaxProblems];
    int32_t count;
};
static_assert(kBatchMaxProblems * sizeof(Prob) <= kBatchTableBytes, "batch table");

__global__ __launch_bounds__(64) void stream_batch_setup(SBatch b, uint8_t *buf)
{
    Prob *table = (Prob *)(buf + kBatchTableOff);
    if ((int)threadIdx.x < b.count) table[threadIdx.x] = b.p[threadIdx.x];
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
constexpr int kR = PN_ROWS_PER_GROUP;   // rows per group in gemv_stream
constexpr int kU = PN_ITEMS_IN_FLIGHT;  // items (one pass of 8 blocks x R rows) in flight per wave

// Per device: CU count (filled once, under a once flag) and gemv_stream
// occupancy by LDS size in 1 KiB steps (0 = not queried yet; concurrent
// queries of one entry compute and store the same value).
struct DeviceInfo {
    int cus = 0;
    std::atomic<signed char> occ[65];
};

DeviceInfo g_dev[kMaxDevices];
std::once_flag g_dev_once[kMaxDevices];

const DeviceInfo &device_info()
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) dev = 0;
    DeviceInfo &d = g_dev[dev];
    std::call_once(g_dev_once[dev], [&d, dev]() {
        int cus = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
            cus = 256;
        for (auto &o : d.occ) o.store(0, std::memory_order_relaxed);
        d.cus = cus;
    });
    return d;
}

}  // namespace

int pn::host::device_cus() { return device_info().cus; }

int pn::host::current_device()
{
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return -1;
    return dev;
}

namespace {
struct AttrOnce {
    std::once_flag once;
    bool ok = false;
};
AttrOnce g_attr[kMaxDevices][kAttrCount];
thread_local int t_gemv_kernel = PN_GEMV_AUTO;
thread_local int t_smallm_math = PN_SMALLM_MFMA;
}  // namespace

bool pn::host::once_per_device(AttrFlag f, bool (*set)())
{
    const int dev = current_device();
    if (dev < 0) return false;
    AttrOnce &a = g_attr[dev][f];
    std::call_once(a.once, [&a, set]() { a.ok = set(); });
    return a.ok;
}

namespace {
struct BatchBuf {
    std::once_flag once;
    uint8_t *ptr = nullptr;
};
BatchBuf g_batch[kMaxDevices];

// The current device's copy of `scratch` (looked up once per device, with
// that device current), or null if the lookup failed.
uint8_t *batch_buffer()
{
    const int dev = current_device();
    if (dev < 0) return nullptr;
    BatchBuf &b = g_batch[dev];
    std::call_once(b.once, [&b]() {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) == hipSuccess) b.ptr = (uint8_t *)p;
    });
    return b.ptr;
}
}  // namespace

int pn::host::gemv_kernel_choice() { return t_gemv_kernel; }
int pn::host::smallm_math_choice() { return t_smallm_math; }

namespace {

int stream_wgs_per_cu(const DeviceInfo &dc, int lds)
{
    DeviceInfo &d = const_cast<DeviceInfo &>(dc);
    int q = (lds + 1023) / 1024;
    q = q < 0 ? 0 : (q > 64 ? 64 : q);
    signed char o = d.occ[q].load(std::memory_order_relaxed);
    if (o == 0) {
        int occ = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&occ, gemv_stream<kR, kU, 2>, kThreads,
                                                         (size_t)q * 1024) != hipSuccess ||
            occ <= 0)
            occ = 1;
        o = (signed char)(occ > 127 ? 127 : occ);
        d.occ[q].store(o, std::memory_order_relaxed);
    }
    return o;
}

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
    p.rpw = kR;
    return p;
}

int lds_bytes_for(const Prob &p) { return p.type == 0 ? 20 * p.nw : 16 * p.nw; }

// gemv_stream takes rows made of whole passes of 8 blocks whose activation
// fits in LDS; rows of whole 16-block passes use two words per lane.
bool stream_ok(const Prob &p)
{
    return (p.nw & 63) == 0 && lds_bytes_for(p) <= kMaxLdsBytes;
}
bool stream_v2(const Prob &p) { return (p.nw & 127) == 0; }

// Tiles: a wave-tile is `rpw` consecutive rows of one problem (at most 64:
// one result lane each; a multiple of kR), a workgroup-tile is kWaves of
// them, and workgroups take tiles in a grid stride.  Tiles are sized in
// bytes, the same target for every problem of a launch.
//   Launches of up to 256 MiB (a layer's groups, single calls): the target
//   whose tiles take the fewest rounds of the grid at the least cost,
//   rounds x (largest wave-tile + 8 KiB for a tile's pipeline fill and
//   drain).  Wave-tiles keep at least the rows for 2U pipelined items,
//   except in launches of at most 1 MiB, where the smallest tiles spread
//   the work widest.
//   Larger launches: about 1/24 of a wave's share, 16-96 KiB.
// Measured on one box (ms for a 16-layer sweep, graphs): the layer schedule
// 0.974 -> 0.937 and the per-matrix one 1.278 -> 1.235 against the earlier
// rule (1/24 of a share, at least 16 KiB); the 256-row pn3t GEMV 6.9 us
// with 2-row tiles against 9.9 with 16 KiB ones and 7.8 with 4 rows; the
// 47-76 MB single calls unchanged.
#ifndef PN_TILES_PER_WAVE
#define PN_TILES_PER_WAVE 24
#endif
#ifndef PN_MAX_WAVE_TILE_KB
#define PN_MAX_WAVE_TILE_KB 96
#endif
constexpr int64_t kTilesPerWave = PN_TILES_PER_WAVE;
#ifndef PN_MIN_WAVE_TILE_KB
#define PN_MIN_WAVE_TILE_KB 16
#endif
constexpr int64_t kMinWaveTileBytes = PN_MIN_WAVE_TILE_KB * 1024;
constexpr int64_t kMaxWaveTileBytes = PN_MAX_WAVE_TILE_KB * 1024;
constexpr int64_t kBalancedMaxBytes = (int64_t)256 << 20;
constexpr int64_t kTinyLaunchBytes = (int64_t)1 << 20;
constexpr int64_t kTileFillBytes = 8 * 1024;

int64_t row_bytes_of(const Prob &p) { return (int64_t)(p.nw >> 3) * 34; }

// Rows of a wave-tile of about `target` bytes: a multiple of kR, at most 64,
// and (pipelined) at least enough for 2U items of kR rows x one pass.
int64_t tile_rows(int64_t target, const Prob &p, bool pipelined)
{
    int64_t lo = kR;
    if (pipelined) {
        const int64_t npass = p.nw / ((p.nw & 127) == 0 ? 128 : 64);
        lo = (2 * kU * kR + npass - 1) / npass;
        lo = (lo + kR - 1) / kR * kR;
        if (lo < kR) lo = kR;
        if (lo > 64) lo = 64;
    }
    int64_t rpw = (target / row_bytes_of(p) + kR / 2) / kR * kR;
    if (rpw < lo) rpw = lo;
    if (rpw > 64) rpw = 64;
    return rpw;
}

// Set rpw and tile0 of every problem; returns the number of tiles, or -1.
int64_t plan_tiles(Prob *probs, int count, int lds)
{
    const DeviceInfo &d = device_info();
    const int64_t wgs = (int64_t)d.cus * stream_wgs_per_cu(d, lds);
    const int64_t waves = wgs * kWaves;
    int64_t bytes = 0;
    for (int i = 0; i < count; ++i) bytes += (int64_t)probs[i].N * row_bytes_of(probs[i]);
    const bool balanced = bytes <= kBalancedMaxBytes;
    const bool pipelined = balanced && bytes > kTinyLaunchBytes;
    int64_t target;
    if (balanced) {
        int64_t best_cost = INT64_MAX;
        target = 2048;
        for (int64_t t = 2048; t <= kMaxWaveTileBytes; t += 1024) {
            int64_t n = 0, largest = 0;
            for (int i = 0; i < count; ++i) {
                const int64_t rpw = tile_rows(t, probs[i], pipelined);
                n += ((int64_t)probs[i].N + kWaves * rpw - 1) / (kWaves * rpw);
                if (rpw * row_bytes_of(probs[i]) > largest) largest = rpw * row_bytes_of(probs[i]);
            }
            const int64_t cost = (n + wgs - 1) / wgs * (largest + kTileFillBytes);
            if (cost < best_cost) {
                best_cost = cost;
                target = t;
            }
        }
    } else {
        target = bytes / (waves * kTilesPerWave);
        if (target < kMinWaveTileBytes) target = kMinWaveTileBytes;
        if (target > kMaxWaveTileBytes) target = kMaxWaveTileBytes;
    }
    int64_t tiles = 0;
    for (int i = 0; i < count; ++i) {
        Prob &p = probs[i];
        const int64_t rpw = tile_rows(target, p, pipelined);
        p.rpw = (int32_t)rpw;
        p.tile0 = (int32_t)tiles;
        tiles += ((int64_t)p.N + kWaves * rpw - 1) / (kWaves * rpw);
        if (tiles > INT32_MAX) return -1;
    }
    return tiles;
}

pn_status launch_stream(StreamArgs &a, int lds, bool v2, hipStream_t s, int variant)
{
    const DeviceInfo &d = device_info();
    int grid = d.cus * stream_wgs_per_cu(d, lds);
    if (grid > a.total_tiles) grid = a.total_tiles;
    if (grid < 1) grid = 1;
    if (v2)
        hipLaunchKernelGGL((gemv_stream<kR, kU, 2>), dim3(grid), dim3(kThreads), lds, s, a);
    else
        hipLaunchKernelGGL((gemv_stream<kR, kU, 1>), dim3(grid), dim3(kThreads), lds, s, a);
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
    hipStream_t s = (hipStream_t)stream;
    if (rows_ok(t, W, K, x) && rows_pays(rows_tiles(N))) return rows_launch(t, W, nullptr, N, K, x, y, nullptr, s);
    Prob p = make_prob(t, W, N, K, x, y);
    if (!stream_ok(p)) return launch_generic(p, p, 1, s);
    const int lds = lds_bytes_for(p);
    const int64_t tiles = plan_tiles(&p, 1, lds);
    if (tiles < 0) return PN_EUNSUPPORTED;
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.p0 = p;
    a.p1 = p;
    a.count = 1;
    a.total_tiles = (int32_t)tiles;
    return launch_stream(a, lds, stream_v2(p), s, kVarStream);
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
    hipStream_t s = (hipStream_t)stream;
    if (rows_ok(t, W0, K, x) && rows_ok(t, W1, K, x) && rows_pays(2 * rows_tiles(N)))
        return rows_launch(t, W0, W1, N, K, x, y0, y1, s);
    Prob p0 = make_prob(t, W0, N, K, x, y0);
    Prob p1 = make_prob(t, W1, N, K, x, y1);
    if (!stream_ok(p0)) return launch_generic(p0, p1, 2, s);
    const int lds = lds_bytes_for(p0);
    Prob pp[2] = {p0, p1};
    const int64_t tiles = plan_tiles(pp, 2, lds);
    if (tiles < 0) return PN_EUNSUPPORTED;
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.p0 = pp[0];
    a.p1 = pp[1];
    a.count = 2;
    a.total_tiles = (int32_t)tiles;
    return launch_stream(a, lds, stream_v2(p0), s, kVarStream);
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

namespace {

// The plan for problems whose x is used as given.
pn_status group_create_plain(const pn_gemv_desc *descs, int count, pn_group **out)
{
    Prob *host = (Prob *)calloc((size_t)count, sizeof(Prob));
    if (!host) return PN_ENOMEM;
    int lds = 0;
    bool v2 = true;
    pn_status st = PN_OK;
    bool all_rows = true;
    int64_t rows_total = 0;
    for (int i = 0; i < count && st == PN_OK; ++i) {
        const pn_gemv_desc &e = descs[i];
        st = check_matrix(e.type, e.W, e.N, e.K);
        if (st == PN_OK && (!e.x || !e.y)) st = PN_EINVAL;
        if (st == PN_OK && (!aligned4(e.x) || !aligned4(e.y))) st = PN_EALIGN;
        if (st == PN_OK) {
            all_rows = all_rows && rows_ok(e.type, e.W, e.K, e.x);
            rows_total += rows_tiles(e.N);
        }
    }
    // the row-tile kernel takes the group if it takes every problem and the
    // launch is large enough
    if (st == PN_OK && all_rows && rows_pays(rows_total)) {
        free(host);
        return rows_group_create(descs, count, out);
    }
    for (int i = 0; i < count && st == PN_OK; ++i) {
        const pn_gemv_desc &e = descs[i];
        host[i] = make_prob(e.type, e.W, e.N, e.K, e.x, e.y);
        if (!stream_ok(host[i])) st = PN_EUNSUPPORTED;
        if (st == PN_OK) {
            v2 = v2 && stream_v2(host[i]);
            if (lds_bytes_for(host[i]) > lds) lds = lds_bytes_for(host[i]);
        }
    }
    const int64_t tiles = st == PN_OK ? plan_tiles(host, count, lds) : 0;
    if (tiles < 0) st = PN_EUNSUPPORTED;
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
    if (hipMalloc(&g->table, sizeof(Prob) * (size_t)count) != hipSuccess) {
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
    g->kind = kGroupGemv;
    g->device = current_device();
    g->count = count;
    g->total_tiles = (int)tiles;
    g->lds = lds;
    g->flags = v2 ? 1 : 0;
    *out = g;
    return PN_OK;
}

}  // namespace

// Problems flagged PN_DESC_ROTATE get a plan-owned copy of x, rotated at the
// start of every run (one launch over all their 1024-element blocks); the
// GEMV plan is built on descriptors that point at the copies.
pn_status pn_group_create(const pn_gemv_desc *descs, int count, pn_group **out)
{
    if (!descs || !out || count < 1) return PN_EINVAL;
    *out = nullptr;
    int64_t rot_elems = 0, rot_jobs = 0;
    for (int i = 0; i < count; ++i) {
        const pn_gemv_desc &e = descs[i];
        if (e.flags & ~PN_DESC_ROTATE) return PN_EINVAL;
        if (!(e.flags & PN_DESC_ROTATE)) continue;
        if (!e.x) return PN_EINVAL;
        if (e.K < PN_ROTATE_BLOCK || e.K % PN_ROTATE_BLOCK != 0) return PN_ESHAPE;
        if (!aligned4(e.x)) return PN_EALIGN;
        rot_elems += e.K;
        rot_jobs += e.K / PN_ROTATE_BLOCK;
    }
    if (rot_jobs == 0) return group_create_plain(descs, count, out);
    if (rot_jobs > INT32_MAX / 2) return PN_EUNSUPPORTED;
    const size_t jbytes = ((size_t)rot_jobs * sizeof(RotJob) + 4095) & ~(size_t)4095;
    void *dev = nullptr;
    if (hipMalloc(&dev, jbytes + (size_t)rot_elems * sizeof(uint16_t)) != hipSuccess) return PN_ENOMEM;
    pn_gemv_desc *d2 = (pn_gemv_desc *)malloc(sizeof(pn_gemv_desc) * (size_t)count);
    RotJob *jobs = (RotJob *)malloc(sizeof(RotJob) * (size_t)rot_jobs);
    if (!d2 || !jobs) {
        free(d2);
        free(jobs);
        (void)hipFree(dev);
        return PN_ENOMEM;
    }
    uint16_t *copies = (uint16_t *)((uint8_t *)dev + jbytes);  // 4 KiB aligned, 2 KiB per block
    int64_t off = 0, j = 0;
    for (int i = 0; i < count; ++i) {
        d2[i] = descs[i];
        d2[i].flags = 0;
        if (!(descs[i].flags & PN_DESC_ROTATE)) continue;
        const uint16_t *src = (const uint16_t *)descs[i].x;
        for (int64_t b = 0; b < descs[i].K / PN_ROTATE_BLOCK; ++b, ++j) {
            jobs[j].src = src + b * PN_ROTATE_BLOCK;
            jobs[j].dst = copies + off + b * PN_ROTATE_BLOCK;
        }
        d2[i].x = copies + off;
        off += descs[i].K;
    }
    pn_status st = hipMemcpy(dev, jobs, sizeof(RotJob) * (size_t)rot_jobs, hipMemcpyHostToDevice) == hipSuccess
                       ? PN_OK
                       : PN_ELAUNCH;
    if (st == PN_OK) st = group_create_plain(d2, count, out);
    free(d2);
    free(jobs);
    if (st != PN_OK) {
        (void)hipFree(dev);
        return st;
    }
    (*out)->rot = dev;
    (*out)->rot_jobs = (int)rot_jobs;
    return PN_OK;
}

pn_status pn_group_run(const pn_group *g, void *stream)
{
    if (!g) return PN_EINVAL;
    if (current_device() != g->device) return PN_EUNSUPPORTED;  // the plan's tables live on its device
    if (g->rot_jobs > 0) {
        const pn_status st = rotate_jobs_launch((const RotJob *)g->rot, g->rot_jobs, (hipStream_t)stream);
        if (st != PN_OK) return st;
    }
    if (g->kind == kGroupSmallM) return smallm_group_run(g, (hipStream_t)stream);
    if (g->kind == kGroupGemvRows) return rows_group_run(g, (hipStream_t)stream);
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.table = (const Prob *)g->table;
    a.count = g->count;
    a.total_tiles = g->total_tiles;
    return launch_stream(a, g->lds, g->flags != 0, (hipStream_t)stream, kVarGroupStream);
}

void pn_group_destroy(pn_group *g)
{
    if (!g) return;
    (void)hipDeviceSynchronize();
    (void)hipFree(g->table);
    if (g->rot) (void)hipFree(g->rot);
    free(g);
}

pn_status pn_gemv_batch(const pn_gemv_desc *descs, int count, void *stream)
{
    if (!descs || count < 1) return PN_EINVAL;
    if (count > kBatchMaxProblems) return PN_EUNSUPPORTED;
    bool all_rows = true;
    int64_t rows_total = 0;
    for (int i = 0; i < count; ++i) {
        const pn_gemv_desc &e = descs[i];
        if (e.flags & ~PN_DESC_ROTATE) return PN_EINVAL;
        if (e.flags & PN_DESC_ROTATE) return PN_EUNSUPPORTED;  // a rotated copy would need a buffer
        const pn_status st = check_matrix(e.type, e.W, e.N, e.K);
        if (st != PN_OK) return st;
        if (!e.x || !e.y) return PN_EINVAL;
        if (!aligned4(e.x) || !aligned4(e.y)) return PN_EALIGN;
        all_rows = all_rows && rows_ok(e.type, e.W, e.K, e.x);
        rows_total += rows_tiles(e.N);
    }
    const bool rows = all_rows && rows_pays(rows_total);
    if (rows && rows_total > kBatchMaxTiles) return PN_EUNSUPPORTED;
    SBatch b;
    int lds = 0;
    bool v2 = true;
    int64_t tiles = 0;
    if (!rows) {
        memset(&b, 0, sizeof(b));
        for (int i = 0; i < count; ++i) {
            const pn_gemv_desc &e = descs[i];
            b.p[i] = make_prob(e.type, e.W, e.N, e.K, e.x, e.y);
            if (!stream_ok(b.p[i])) return PN_EUNSUPPORTED;
            v2 = v2 && stream_v2(b.p[i]);
            if (lds_bytes_for(b.p[i]) > lds) lds = lds_bytes_for(b.p[i]);
        }
        tiles = plan_tiles(b.p, count, lds);
        if (tiles < 0) return PN_EUNSUPPORTED;
        b.count = count;
    }
    uint8_t *buf = batch_buffer();
    if (!buf) return PN_ELAUNCH;
    const hipStream_t s = (hipStream_t)stream;
    if (rows) return rows_batch_launch(descs, count, buf, s);
    hipLaunchKernelGGL(stream_batch_setup, dim3(1), dim3(64), 0, s, b, buf);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    StreamArgs a;
    memset(&a, 0, sizeof(a));
    a.table = (const Prob *)(buf + kBatchTableOff);
    a.count = count;
    a.total_tiles = (int32_t)tiles;
    return launch_stream(a, lds, v2, s, kVarBatchStream);
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

pn_status pn_set_gemv_kernel(pn_gemv_kernel k)
{
    if (k != PN_GEMV_AUTO && k != PN_GEMV_STREAM && k != PN_GEMV_ROWS) return PN_EINVAL;
    t_gemv_kernel = (int)k;
    return PN_OK;
}

pn_gemv_kernel pn_get_gemv_kernel(void) { return (pn_gemv_kernel)t_gemv_kernel; }

pn_status pn_set_smallm_math(pn_smallm_math m)
{
    if (m != PN_SMALLM_MFMA && m != PN_SMALLM_VALU) return PN_EINVAL;
    t_smallm_math = (int)m;
    return PN_OK;
}

pn_smallm_math pn_get_smallm_math(void) { return (pn_smallm_math)t_smallm_math; }

const char *pn_variant_name(int v)
{
    switch (v) {
    case kVarNone: return "none";
    case kVarStream: return "gemv_stream";
    case kVarGeneric: return "gemv_generic";
    case kVarSmallMValu: return "gemm_stream_valu";
    case kVarSmallMMfma: return "gemm_stream_mfma";
    case kVarGroupSmallMValu: return "gemm_stream_valu_group";
    case kVarGroupSmallMMfma: return "gemm_stream_mfma_group";
    case kVarSmallMRows: return "gemm_rows_mfma";
    case kVarGroupSmallMRows: return "gemm_rows_mfma_group";
    case kVarRows: return "gemv_rows";
    case kVarGroupRows: return "gemv_rows_group";
    case kVarRotate: return "hadamard_rotate";
    case kVarPrefill: return "gemm_prefill";
    case kVarPrefillGroup: return "gemm_prefill_group";
    case kVarDequant: return "dequant";
    case kVarGroupStream: return "gemv_stream_group";
    case kVarBatchRows: return "gemv_rows_batch";
    case kVarBatchStream: return "gemv_stream_batch";
    }
    return "unknown";
}

}  // extern "C"
