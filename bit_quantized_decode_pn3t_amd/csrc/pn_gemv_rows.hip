// pn_gemv_rows.hip - M = 1 PN GEMV over 16-row tiles staged through LDS,
// for AMD Instinct MI355X (gfx950).
//
// The product is the same as gemv_stream's (pn_kernels.hip): y = W x with
// w = d * (n - z) decoded exactly ("Exact decode in fp32") and fp32 sums.
// What differs is how the bytes reach the lanes and how x meets them.
//
// Periods.  Eight 34-byte blocks ("Every block is 34 bytes") are 272 bytes,
// 17 aligned 16-byte chunks.  This kernel takes rows whose length is whole
// periods (K a multiple of 640 for pn3t, 512 for pn4t), so every period
// starts 16-byte aligned and has the same layout: four block pairs of 17
// dwords; in each pair the first block's words sit two bytes off the dword
// grid and are rebuilt with one v_alignbit each, the second block's words
// are whole dwords, and the two scales are the low half of the pair's dword
// 0 and the high half of its dword 8.
//
// Lanes.  Lane (g, r) = (lane / 16, lane % 16) owns row r of the wave's
// 16-row tile and, in each stage, period 4w + g of that row (w the tile
// window).  The 16 lanes of a DPP row (one g) thus read the same columns of
// 16 rows, so every activation pair they need is the same: it is loaded once
// per DPP row (lane r holds pairs 4r..4r+3 of each 64) and reaches all 16
// lanes as the broadcast source operand of v_dot2c_f32_f16 (DPP
// row_newbcast).  A lane accumulates its row over the whole tile; the four
// DPP rows' partial sums are added with two permlane swaps once per tile.
// There is no per-row wave reduction and no activation traffic through LDS.
//
// Loads.  A stage is one window of the tile: 16 rows x 1088 bytes, brought
// to LDS by 17 aligned 16-byte DMA instructions (buffer_load_dwordx4 ... lds)
// that each cover 1024 contiguous bytes of the matrix.  Each wave has a ring
// of two stages and keeps one stage in flight while it computes the other;
// x for a stage comes from global memory (L2) into registers, five dwordx4
// per lane, issued with the stage's DMA.
//
// Grid.  One workgroup of four waves per CU (the rings take 136 KiB of LDS).
// Waves work independently on contiguous ranges of tiles, balanced by
// windows; a launch with few tiles per wave balances badly, and the host
// gives such launches to gemv_stream.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#include <type_traits>

#include "pn_device.h"
#include "pn_host.h"

using namespace pn;
using namespace pn::host;

namespace {

constexpr int kRWaves = 4;                    // waves per workgroup, one per SIMD
constexpr int kRThreads = 64 * kRWaves;
constexpr int kTileRows = 16;                 // rows per tile: the lanes of a DPP row
constexpr int kPeriod = 272;                  // 8 blocks
constexpr int kWindow = 4 * kPeriod;          // tile-row bytes per stage
constexpr int kStage = kTileRows * kWindow;   // 17,408
constexpr int kDma = kStage / 1024;           // 17 DMA instructions per stage
constexpr int kXLoads = 5;                    // x loads per lane per stage
constexpr int kLater = kDma + kXLoads;        // VMEM instructions of one stage
constexpr int kRing = kRWaves * 2 * kStage;   // 139,264 bytes of LDS
constexpr int kMinTilesPerWave = 8;           // below this "auto" uses gemv_stream

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;
#define PN_CONST __attribute__((address_space(4)))

// One problem as the device sees it.
struct RProb {
    const uint8_t *W;  // packed rows, 16-byte aligned
    const uint8_t *x;  // fp16 [K], 16-byte aligned
    float *y;          // fp32 [N]
    int32_t N;         // rows
    int32_t S;         // row bytes = 272 * P
    int32_t P;         // periods per row
    int32_t nwin;      // windows per tile = ceil(P / 4)
    int32_t tiles;     // ceil(N / 16)
    int32_t type;      // 0 = pn3t, 1 = pn4t
};

// A wave's share of a group launch: its first tile and how many.
struct RStart {
    int32_t prob;
    int32_t tile;
    int32_t ntiles;
    int32_t nitems;  // windows of those tiles
};

struct RArgs {
    const PN_CONST RProb *table;   // group plan, or null for the inline problems
    const PN_CONST RStart *start;  // per wave (with the table)
    RProb p0, p1;                  // inline problems (pn_gemv, pn_gemv2)
    int32_t count;                 // problems
    int32_t total_tiles;           // inline problems: tiles of both
};

template <int I, int N, typename F>
__device__ __forceinline__ void static_for(F &&f)
{
    if constexpr (I < N) {
        f(std::integral_constant<int, I>());
        static_for<I + 1, N>(f);
    }
}

// acc += w.lo * x_L.lo + w.hi * x_L.hi, x_L = x in lane L of this lane's
// 16-lane DPP row.  x comes from a load, never from a VALU write, so the DPP
// read has no wait-state hazard.  A chain of these accumulating into acc
// needs no wait states either (the accumulator is forwarded to the next dot
// product), but any other instruction that reads or writes acc must come at
// least three wait states after the last one: the compiler does not know
// this instruction, so dot_done() says so.

template <int L>
__device__ __forceinline__ void dot2c_bcast(float &acc, uint32_t x, half2_t w)
{
    asm("v_dot2c_f32_f16_dpp %0, %1, %2 row_newbcast:%3 row_mask:0xf bank_mask:0xf"
        : "+v"(acc)
        : "v"(x), "v"(w), "i"(L));
}

// Three wait states between the last dot product into v and the next
// instruction that touches v (gfx950 requires them after a dot instruction's
// write before another VALU reads or writes the same register).
__device__ __forceinline__ void dot_done(float &v) { asm volatile("s_nop 2" : "+v"(v)); }

// One code word: its pairs meet activation pairs P0 .. P0 + kPairs - 1 of the
// period (pair p = x[2p], x[2p+1]), held as described in the header.
template <int TYPE, int P0>
__device__ __forceinline__ void word_dot(float &bs, uint32_t w, const u32x4 (&xs)[kXLoads])
{
    half2_t u[Unpack<TYPE>::kPairs];
    Unpack<TYPE>::run(w, u);
    static_for<0, Unpack<TYPE>::kPairs>([&](auto q) {
        constexpr int P = P0 + decltype(q)::value;
        dot2c_bcast<((P & 63) >> 2)>(bs, xs[P >> 6][P & 3], u[decltype(q)::value]);
    });
}

// Sum over one period of a row: sum over its 8 blocks of d * sum (n - z) x.
template <int TYPE>
__device__ __forceinline__ float period_dot(const uint8_t *src, const u32x4 (&xs)[kXLoads])
{
    constexpr int PB = TYPE == 0 ? 40 : 32;  // activation pairs per block
    constexpr int PW = TYPE == 0 ? 5 : 4;    // per word
    uint32_t D[68];
#pragma unroll
    for (int t = 0; t < 17; ++t) {
        const u32x4 v = *(const u32x4 *)(src + 16 * t);
        D[4 * t] = v[0];
        D[4 * t + 1] = v[1];
        D[4 * t + 2] = v[2];
        D[4 * t + 3] = v[3];
    }
    float it = 0.0f;
    static_for<0, 4>([&](auto bpc) {
        constexpr int bp = decltype(bpc)::value;
        constexpr int o = 17 * bp;
        float bs = 0.0f;
        static_for<0, 8>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            word_dot<TYPE, PB * (2 * bp) + PW * j>(bs, __builtin_amdgcn_alignbit(D[o + j + 1], D[o + j], 16), xs);
        });
        dot_done(bs);
        it = __builtin_fmaf(half_bits_to_float(D[o] & 0xffffu), bs, it);
        bs = 0.0f;
        static_for<0, 8>([&](auto jc) {
            constexpr int j = decltype(jc)::value;
            word_dot<TYPE, PB * (2 * bp + 1) + PW * j>(bs, D[o + 9 + j], xs);
        });
        dot_done(bs);
        it = __builtin_fmaf(half_bits_to_float(D[o + 8] >> 16), bs, it);
    });
    return it;
}

// Where a wave's issue side is in its work: problem, tile, window, tiles
// left, and the problem's fields.  The cursor is advanced without nested
// branches and the problem is reloaded (scalar loads) at every step, so that
// every field is defined on every path and stays in scalar registers.
struct Cursor {
    int32_t pi, tile, win, left;
    const uint8_t *W, *x;
    float *y;
    int32_t N, S, P, nwin, tiles, type;
};

// Group launches read the problem from the plan's table (scalar loads);
// inline launches have one or two problems of one shape, which differ only
// in W and y.
template <bool TABLE>
__device__ __forceinline__ void load_prob(Cursor &c, const RArgs &a)
{
    if constexpr (TABLE) {
        const int32_t i = c.pi < a.count ? c.pi : a.count - 1;
        const PN_CONST RProb &p = a.table[i];
        c.W = p.W;
        c.x = p.x;
        c.y = p.y;
        c.N = p.N;
        c.S = p.S;
        c.P = p.P;
        c.nwin = p.nwin;
        c.tiles = p.tiles;
        c.type = p.type;
    } else {
        const bool one = c.pi != 0;
        c.W = one ? a.p1.W : a.p0.W;
        c.y = one ? a.p1.y : a.p0.y;
        c.x = a.p0.x;
        c.N = a.p0.N;
        c.S = a.p0.S;
        c.P = a.p0.P;
        c.nwin = a.p0.nwin;
        c.tiles = a.p0.tiles;
        c.type = a.p0.type;
    }
}

template <bool TABLE>
__device__ __forceinline__ void advance(Cursor &c, const RArgs &a)
{
    const int32_t win1 = c.win + 1;
    const int32_t wrap_w = win1 >= c.nwin ? 1 : 0;
    c.win = wrap_w ? 0 : win1;
    c.left -= wrap_w;
    const int32_t tile1 = c.tile + wrap_w;
    const int32_t wrap_t = tile1 >= c.tiles ? 1 : 0;
    c.tile = wrap_t ? 0 : tile1;
    c.pi += wrap_t;
    load_prob<TABLE>(c, a);
}

// What the compute side needs of a stage, recorded when the stage is issued.
struct Slot {
    float *y;
    int32_t live, type, P, win, last, row0, N;
};

// Per-lane DMA offsets of the 17 instructions for row stride S: slot
// q = 64 i + lane holds chunk q % 68 of tile row q / 68.
__device__ __forceinline__ void dma_offsets(uint32_t (&vo)[kDma], int32_t S, int lane)
{
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        const uint32_t q = 64u * i + (uint32_t)lane;
        const uint32_t row = q / 68u;
        vo[i] = row * (uint32_t)S + 16u * (q - 68u * row);
    }
}

// Issue the cursor's stage: the window's DMA into the ring stage and the x
// loads into xs.  A cursor past its last tile issues the same instructions
// on empty buffer ranges (they read nothing and return zeros), so every
// stage is exactly kLater VMEM instructions.
__device__ __forceinline__ void issue(const Cursor &c, uint8_t *stage, const uint32_t (&vo)[kDma], uint32_t xlane,
                                      u32x4 (&xs)[kXLoads], Slot &sl)
{
    const bool live = c.left > 0;
    const int32_t rows_left = c.N - kTileRows * c.tile;
    const uint32_t rows = !live ? 0u : rows_left < kTileRows ? (uint32_t)rows_left : (uint32_t)kTileRows;
    // (readfirstlane: the resource must be in scalar registers, and the
    // compiler cannot always tell that these values are wave-uniform)
    const uint8_t *wbase = uniform_ptr(c.W + (size_t)(kTileRows * c.tile) * (size_t)c.S);
    const __amdgpu_buffer_rsrc_t wr = make_rsrc(wbase, (uint32_t)uniform((int32_t)(rows * (uint32_t)c.S)));
    const uint32_t soff = (uint32_t)(c.win * kWindow);
#pragma unroll
    for (int i = 0; i < kDma; ++i)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void *)(stage + 1024 * i), 16, (int)vo[i], (int)soff, 0,
                                                 2 /* nontemporal */);
    const uint32_t px = c.type == 0 ? 1280u : 1024u;  // x bytes per period
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(uniform_ptr(c.x), (uint32_t)uniform((int32_t)(live ? (uint32_t)c.P * px : 0u)));
    const uint32_t xsoff = 4u * (uint32_t)c.win * px;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i)
        xs[i] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(xlane + 256u * i), (int)xsoff, 0));
    sl.y = c.y;
    sl.live = live ? 1 : 0;
    sl.type = c.type;
    sl.P = c.P;
    sl.win = c.win;
    sl.last = live && c.win == c.nwin - 1 ? 1 : 0;
    sl.row0 = kTileRows * c.tile;
    sl.N = c.N;
}

// Wait until at most kLater VMEM instructions are outstanding: the stage
// issued last may still be in flight, everything before it has landed.
// Loads (DMA included) return in issue order; stores only add to the count.
// The empty asm keeps LDS reads of the stage below the wait.
__device__ __forceinline__ void wait_stage()
{
    __builtin_amdgcn_s_waitcnt((((kLater >> 4) & 3) << 14) | 0x0f70 | (kLater & 15));
    asm volatile("" ::: "memory");
}

__device__ __forceinline__ void wait_lds_reads()
{
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
    asm volatile("" ::: "memory");
}

template <bool TABLE>
__global__ __launch_bounds__(kRThreads) void gemv_rows(RArgs a)
{
    extern __shared__ __attribute__((aligned(16))) uint8_t lds[];
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int gw = blockIdx.x * kRWaves + wave;
    const int g = lane >> 4, r = lane & 15;
    uint8_t *ring = lds + wave * 2 * kStage;

    // this wave's tiles and windows
    Cursor ci;
    int32_t nitems;
    if constexpr (TABLE) {
        const PN_CONST RStart &st = a.start[gw];
        ci.pi = st.prob;
        ci.tile = st.tile;
        ci.left = st.ntiles;
        nitems = st.nitems;
    } else {
        const int nw = gridDim.x * kRWaves;
        const int t0 = (int)((int64_t)a.total_tiles * gw / nw);
        const int t1 = (int)((int64_t)a.total_tiles * (gw + 1) / nw);
        ci.pi = t0 >= a.p0.tiles ? 1 : 0;
        ci.tile = t0 - (ci.pi ? a.p0.tiles : 0);
        ci.left = t1 - t0;
        nitems = ci.left * a.p0.nwin;
    }
    ci.win = 0;
    if (nitems <= 0) return;
    load_prob<TABLE>(ci, a);

    uint32_t vo[kDma];
    int32_t vo_s = ci.S;
    dma_offsets(vo, vo_s, lane);
    const uint32_t xl3 = (uint32_t)(16 * r + 1280 * g), xl4 = (uint32_t)(16 * r + 1024 * g);

    u32x4 xs0[kXLoads], xs1[kXLoads];
    Slot sl0, sl1;
    issue(ci, ring, vo, ci.type == 0 ? xl3 : xl4, xs0, sl0);
    advance<TABLE>(ci, a);
    asm volatile("" ::: "memory");  // keep the two stages' loads in issue order
    issue(ci, ring + kStage, vo, ci.type == 0 ? xl3 : xl4, xs1, sl1);
    advance<TABLE>(ci, a);
    float acc = 0.0f;

    // One step: compute the stage in ring slot `stage`, then refill that slot
    // with the issue cursor's stage.  A step past the wave's last window
    // computes zeros and stores nothing.
    auto step = [&](uint8_t *stage, u32x4 (&xs)[kXLoads], Slot &sl) {
        wait_stage();
        const uint8_t *src = stage + r * kWindow + g * kPeriod;
        float it;
        if (sl.type == 0)
            it = period_dot<0>(src, xs);
        else
            it = period_dot<1>(src, xs);
        acc += 4 * sl.win + g < sl.P ? it : 0.0f;
        if (sl.last) {
            // the tile is done: add the four DPP rows' sums of each row
            auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
            float v = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
            auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
            v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
            const int row = sl.row0 + r;
            if (g == 0 && row < sl.N) sl.y[row] = v;
            acc = 0.0f;
        }
        wait_lds_reads();
        if (ci.S != vo_s) {
            vo_s = ci.S;
            dma_offsets(vo, vo_s, lane);
        }
        issue(ci, stage, vo, ci.type == 0 ? xl3 : xl4, xs, sl);
        advance<TABLE>(ci, a);
    };
    for (int k = 0; k < nitems; k += 2) {
        step(ring, xs0, sl0);
        step(ring + kStage, xs1, sl1);
    }
    // no DMA may still be writing this wave's LDS when the workgroup ends
    __builtin_amdgcn_s_waitcnt(0x0f70);
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
int g_kernel = PN_GEMV_AUTO;

void rfill(RProb &p, int t, const void *W, int64_t N, int64_t K, const void *x, float *y)
{
    memset(&p, 0, sizeof(p));
    p.W = (const uint8_t *)W;
    p.x = (const uint8_t *)x;
    p.y = y;
    p.N = (int32_t)N;
    p.P = (int32_t)(K / wpb(t) / 8);
    p.S = kPeriod * p.P;
    p.nwin = (p.P + 3) / 4;
    p.tiles = (int32_t)((N + kTileRows - 1) / kTileRows);
    p.type = t;
}

int rows_waves() { return device_cus() * kRWaves; }

bool set_rows_attr()
{
    static int done = 0;  // per process; the attribute is per function
    if (!done) {
        if (hipFuncSetAttribute((const void *)gemv_rows<true>, hipFuncAttributeMaxDynamicSharedMemorySize, kRing) !=
                hipSuccess ||
            hipFuncSetAttribute((const void *)gemv_rows<false>, hipFuncAttributeMaxDynamicSharedMemorySize, kRing) !=
                hipSuccess)
            return false;
        done = 1;
    }
    return true;
}

pn_status rlaunch(const RArgs &a, hipStream_t s, int variant)
{
    if (!set_rows_attr()) return PN_ELAUNCH;
    if (a.table)
        hipLaunchKernelGGL(gemv_rows<true>, dim3((unsigned)device_cus()), dim3(kRThreads), kRing, s, a);
    else
        hipLaunchKernelGGL(gemv_rows<false>, dim3((unsigned)device_cus()), dim3(kRThreads), kRing, s, a);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    g_last_variant = variant;
    return PN_OK;
}

}  // namespace

// Can gemv_rows take this problem?  Rows of whole periods (K a multiple of
// 640 for pn3t, 512 for pn4t), 16-byte aligned W and x, and sizes whose byte
// offsets fit the kernel's 32-bit arithmetic.
bool pn::host::rows_ok(int t, const void *W, int64_t K, const void *x)
{
    if (pn_get_gemv_kernel() == PN_GEMV_STREAM) return false;
    if (((uintptr_t)W & 15) != 0 || ((uintptr_t)x & 15) != 0) return false;
    const int64_t nb = K / wpb(t);
    if (nb % 8 != 0) return false;
    return nb * 34 <= ((int64_t)1 << 24);  // row bytes: 16 rows x row bytes < 2^28
}

// Is a launch of `tiles` 16-row tiles large enough for gemv_rows?
bool pn::host::rows_pays(int64_t tiles)
{
    if (pn_get_gemv_kernel() == PN_GEMV_ROWS) return true;
    return tiles >= (int64_t)kMinTilesPerWave * rows_waves();
}

int64_t pn::host::rows_tiles(int64_t N) { return (N + kTileRows - 1) / kTileRows; }

pn_status pn::host::rows_launch(int t, const void *W0, const void *W1, int64_t N, int64_t K, const void *x,
                                float *y0, float *y1, hipStream_t s)
{
    RArgs a;
    memset(&a, 0, sizeof(a));
    rfill(a.p0, t, W0, N, K, x, y0);
    a.count = 1;
    a.total_tiles = a.p0.tiles;
    if (W1) {
        rfill(a.p1, t, W1, N, K, x, y1);
        a.count = 2;
        a.total_tiles += a.p1.tiles;
    }
    return rlaunch(a, s, kVarRows);
}

pn_status pn::host::rows_group_create(const pn_gemv_desc *descs, int count, pn_group **out)
{
    *out = nullptr;
    const int nw = rows_waves();
    const size_t tbytes = sizeof(RProb) * (size_t)count;
    const size_t sbytes = sizeof(RStart) * (size_t)nw;
    uint8_t *blob = (uint8_t *)calloc(1, tbytes + sbytes);
    pn_group *g = (pn_group *)calloc(1, sizeof(pn_group));
    if (!g || !blob) {
        free(blob);
        free(g);
        return PN_ENOMEM;
    }
    RProb *host = (RProb *)blob;
    int64_t windows = 0;  // the launch's stages: the unit of balance
    for (int i = 0; i < count; ++i) {
        const pn_gemv_desc &e = descs[i];
        rfill(host[i], e.type, e.W, e.N, e.K, e.x, e.y);
        windows += (int64_t)host[i].tiles * host[i].nwin;
    }
    // Wave w takes the tiles whose first window falls in its equal share
    // [windows * w / nw, windows * (w + 1) / nw) of the launch's windows.
    RStart *st = (RStart *)(blob + tbytes);
    int pi = 0, tile = 0;
    int64_t pos = 0;  // first window of (pi, tile)
    for (int w = 0; w < nw; ++w) {
        const int64_t lo = windows * w / nw, hi = windows * (w + 1) / nw;
        while (pi < count && pos < lo) {  // skip tiles that start before the share
            pos += host[pi].nwin;
            if (++tile == host[pi].tiles) {
                tile = 0;
                ++pi;
            }
        }
        st[w].prob = pi;
        st[w].tile = tile;
        int n = 0, items = 0;
        while (pi < count && pos < hi) {
            pos += host[pi].nwin;
            items += host[pi].nwin;
            ++n;
            if (++tile == host[pi].tiles) {
                tile = 0;
                ++pi;
            }
        }
        st[w].ntiles = n;
        st[w].nitems = items;
    }
    if (hipMalloc(&g->table, tbytes + sbytes) != hipSuccess) {
        free(blob);
        free(g);
        return PN_ENOMEM;
    }
    if (hipMemcpy(g->table, blob, tbytes + sbytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(g->table);
        free(blob);
        free(g);
        return PN_ELAUNCH;
    }
    free(blob);
    g->kind = kGroupGemvRows;
    g->count = count;
    g->total_tiles = nw;
    g->lds = kRing;
    g->flags = 0;
    *out = g;
    return PN_OK;
}

pn_status pn::host::rows_group_run(const pn_group *g, hipStream_t s)
{
    if (g->total_tiles != rows_waves()) return PN_EUNSUPPORTED;  // made for another device
    RArgs a;
    memset(&a, 0, sizeof(a));
    a.table = (const PN_CONST RProb *)g->table;
    a.start = (const PN_CONST RStart *)((const uint8_t *)g->table + sizeof(RProb) * (size_t)g->count);
    a.count = g->count;
    return rlaunch(a, s, kVarGroupRows);
}

extern "C" {

pn_status pn_set_gemv_kernel(pn_gemv_kernel k)
{
    if (k != PN_GEMV_AUTO && k != PN_GEMV_STREAM && k != PN_GEMV_ROWS) return PN_EINVAL;
    __atomic_store_n(&g_kernel, (int)k, __ATOMIC_RELAXED);
    return PN_OK;
}

pn_gemv_kernel pn_get_gemv_kernel(void) { return (pn_gemv_kernel)__atomic_load_n(&g_kernel, __ATOMIC_RELAXED); }

}  // extern "C"
