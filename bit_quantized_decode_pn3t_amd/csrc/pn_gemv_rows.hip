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
// to LDS by 16-byte DMA instructions (buffer_load_dwordx4 ... lds), rows
// 976 bytes apart in LDS so that the lanes' period reads do not collide in
// banks; the last 8 chunks of each row go to a separate region with the
// normal cache policy (the 128-byte line they share with the next window
// then is often still cached when that window is fetched).  Each wave has one stage: once its lanes have read their periods
// into registers, the stage is refilled with the wave's next window, in two
// pieces between the block pairs' products, so that the next window is in
// flight while this one is computed.  x for a stage comes from global
// memory (L2) into registers, five dwordx4 per lane.
//
// Grid.  One workgroup of eight waves per CU (two per SIMD: one computes
// while the other waits; the stages take 152 KiB of LDS).  Inline launches
// (one matrix, or the fused pair) split their tiles evenly over the waves;
// group launches (many matrices, one launch) hand tiles out from pools of
// per-pool atomic counters, longest tiles first.  A launch with few tiles
// per wave balances badly, and the host gives such launches to gemv_stream.
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

// Design choices, measured on the 64-layer sweep:
//   PN_ROWS_PAD    rows of a stage 1104 bytes apart in LDS (conflict-free
//                  period reads, 18 DMA instructions a stage) or 1088 (17,
//                  four-way bank conflicts);
//   PN_ROWS_SPLIT  refill the ring slot after the first block pair's
//                  products (the period reads have landed by then) rather
//                  than waiting for the reads before any products;
//   PN_ROWS_ILP    independent accumulation chains per block (1 or 2);
//   PN_ROWS_STAGES ring stages per wave: 2 (4 waves per CU, one per SIMD,
//                  two windows in flight per wave) or 1 (8 waves per CU,
//                  two per SIMD: one computes while the other waits);
//   PN_ROWS_BND    each row's last 8 chunks of a window (where a 128-byte
//                  line shared with the next window lies) in an LDS region
//                  of their own, filled by 3 DMA instructions with the
//                  normal cache policy, the rest nontemporal: fetched bytes
//                  1.073 -> 1.051 of the algorithmic ones, ~1 % faster;
//   PN_ROWS_SPREAD pieces a stage's DMA is issued in, between the block
//                  pairs' products (1: all at once, which stalls the wave
//                  while the eight waves' bursts queue up; 2 or 3).
#ifndef PN_ROWS_PAD
#define PN_ROWS_PAD 1
#endif
#ifndef PN_ROWS_SPLIT
#define PN_ROWS_SPLIT 1
#endif
#ifndef PN_ROWS_ILP
#define PN_ROWS_ILP 2
#endif
#ifndef PN_ROWS_STAGES
#define PN_ROWS_STAGES 1
#endif
#ifndef PN_ROWS_BND
#define PN_ROWS_BND 1
#endif
#ifndef PN_ROWS_SPREAD
#define PN_ROWS_SPREAD 2
#endif

constexpr int kNS = PN_ROWS_STAGES;           // ring stages per wave
constexpr int kRWaves = kNS == 2 ? 4 : 8;      // waves per workgroup (one workgroup per CU)
constexpr int kRThreads = 64 * kRWaves;
constexpr int kTileRows = 16;                 // rows per tile: the lanes of a DPP row
constexpr int kPeriod = 272;                  // 8 blocks
constexpr int kWindow = 4 * kPeriod;          // tile-row bytes per stage
constexpr int kRowLds = PN_ROWS_PAD ? kWindow + 16 : kWindow;  // LDS bytes per tile row
constexpr int kRowSlots = kRowLds / 16;      // 16-byte DMA slots per tile row
// PN_ROWS_BND: the last 8 chunks of each row's window (where a line shared
// with the next window lies) go to a region of their own, filled with the
// normal cache policy so that the next window finds the line cached.
constexpr int kMainCk = PN_ROWS_BND ? 60 : 68;  // chunks per row in the main region
constexpr int kMainSlots = PN_ROWS_BND ? 61 : kRowSlots;
constexpr int kMainDma = (kTileRows * kMainSlots + 63) / 64;
constexpr int kBndSlots = 9;                    // boundary region: 8 chunks + pad per row
constexpr int kBndDma = PN_ROWS_BND ? (kTileRows * kBndSlots + 63) / 64 : 0;
constexpr int kDma = kMainDma + kBndDma;        // DMA instructions per stage
constexpr int kStage = 1024 * kDma;          // LDS bytes per stage
constexpr int kXLoads = 5;                    // x loads per lane per stage
constexpr int kLater = (kNS - 1) * (kDma + kXLoads);  // VMEM instructions issued after a stage
// With one stage per wave every wait is for all loads in flight, so a stage
// without work issues no loads at all (with two, every stage issues the same
// instructions so that the counted waits stay exact).  Issuing a stage's 23
// instructions is not free: a wave with nothing else in flight on its CU
// takes about a microsecond to push them.
constexpr bool kSkipIdle = kNS == 1;
constexpr int kRing = kRWaves * kNS * kStage;  // 155,648 bytes of LDS (147,456 without the boundary region)
constexpr int kMinTilesPerCu = 32;            // below this "auto" uses gemv_stream
constexpr int kPools = 16;                    // tile pools of a group launch
constexpr uint32_t kPoolChunk = 64;           // consecutive tiles a pool is dealt at a time
constexpr int kCounterStride = 1024;          // uint32s between pool counters (4 KiB)
static_assert(kPools <= 32 && (kPools & (kPools - 1)) == 0, "pools: a power of two, one lane each");

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

struct RArgs {
    const PN_CONST RProb *table;   // group plan, or null for the inline problems
    const PN_CONST uint32_t *lut;  // group plan: tile k of the launch = problem
                                   // lut[k] >> 20, tile lut[k] & 0xfffff
    uint32_t *counters;            // group plan: pool p's counter at
                                   // [kCounterStride * p], waves done after them
    RProb p0, p1;                  // inline problems (pn_gemv, pn_gemv2)
    int32_t count;                 // problems
    int32_t total_tiles;           // tiles of the launch
    int32_t step_cap;              // steps no wave of a correct run reaches
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

// The lane's period of the stage: 17 chunks from LDS.
__device__ __forceinline__ void load_period(const uint8_t *src, uint32_t (&D)[68])
{
#pragma unroll
    for (int t = 0; t < 17; ++t) {
        const u32x4 v = *(const u32x4 *)(src + 16 * t);
        D[4 * t] = v[0];
        D[4 * t + 1] = v[1];
        D[4 * t + 2] = v[2];
        D[4 * t + 3] = v[3];
    }
}

// The same, with chunks 9..16 from a second base (the boundary region).
__device__ __forceinline__ void load_period2(const uint8_t *lo, const uint8_t *hi, uint32_t (&D)[68])
{
#pragma unroll
    for (int t = 0; t < 17; ++t) {
        const u32x4 v = *(const u32x4 *)((t < 9 ? lo : hi) + 16 * t);
        D[4 * t] = v[0];
        D[4 * t + 1] = v[1];
        D[4 * t + 2] = v[2];
        D[4 * t + 3] = v[3];
    }
}

// Block pairs [BP0, BP1) of a period of a row: it += d * sum (n - z) x over
// their blocks.
template <int TYPE, int BP0, int BP1>
__device__ __forceinline__ void period_dot(const uint32_t (&D)[68], const u32x4 (&xs)[kXLoads], float &it)
{
    constexpr int PB = TYPE == 0 ? 40 : 32;  // activation pairs per block
    constexpr int PW = TYPE == 0 ? 5 : 4;    // per word
    static_for<BP0, BP1>([&](auto bpc) {
        constexpr int bp = decltype(bpc)::value;
        constexpr int o = 17 * bp;
        static_for<0, 2>([&](auto hc) {  // block 2 bp + h of the period
            constexpr int h = decltype(hc)::value;
            float bs[PN_ROWS_ILP];
#pragma unroll
            for (int c = 0; c < PN_ROWS_ILP; ++c) bs[c] = 0.0f;
            static_for<0, 8>([&](auto jc) {
                constexpr int j = decltype(jc)::value;
                // first block: words straddle the dword grid; second: whole dwords
                const uint32_t w = h == 0 ? __builtin_amdgcn_alignbit(D[o + j + 1], D[o + j], 16) : D[o + 9 + j];
                word_dot<TYPE, PB * (2 * bp + h) + PW * j>(bs[j % PN_ROWS_ILP], w, xs);
            });
#pragma unroll
            for (int c = 0; c < PN_ROWS_ILP; ++c) dot_done(bs[c]);
            float b = bs[0];
#pragma unroll
            for (int c = 1; c < PN_ROWS_ILP; ++c) b += bs[c];
            const uint32_t dh = h == 0 ? D[o] & 0xffffu : D[o + 8] >> 16;
            it = __builtin_fmaf(half_bits_to_float(dh), b, it);
        });
    });
}

// Where a wave's issue side is in its work: problem, tile, window, state,
// and the problem's fields.  The cursor is advanced without nested branches
// where possible and the problem is reloaded (scalar loads) at every step,
// so that every field is defined on every path and stays in scalar
// registers.
//
// Inline launches (one or two problems) split the tiles statically: wave w
// takes tiles [T w / n, T (w + 1) / n).  Group launches hand out tiles
// dynamically: the XCDs of an MI355X stream at measurably different rates
// (up to 15 % apart on the sweep), so a static split leaves the fast ones
// idle at the end.  One counter for the whole device would serialize the
// grabs (device-scope atomics on one address, tens of ns each), so the
// launch's tiles are dealt into kPools pools, one per half XCD, each with its
// own counter: chunks of kPoolChunk consecutive tiles in turn, so that a
// wave's next tiles are usually its last one's neighbours in memory (one
// tile at a time, 16 tiles apart, ran the sweep 1 % slower; chunks of 1,024
// and more leave long tiles to the end).  A wave takes tiles from its home
// pool and, once that is empty, reads all the counters at once (one atomic
// add of zero per lane) and moves to a pool with tiles left, or ends when
// none has any.  (Trying the pools one by one cost a step per empty pool at the end
// of every launch.)  The grab for a wave's next tile is issued at the start
// of the step after it moved to a new tile, and read when it moves again,
// at least one step later; so is the counter read.
enum { kLive = 0, kIdle = 1, kDone = 2, kScan = 3 };

struct Cursor {
    int32_t pi, tile, win, state;
    int32_t pool, rot;  // group: pool of the outstanding grab, where the wave starts looking
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

// The pool counters.  Lanes with `on` add `v` to pool p's counter and get
// its old value in k; lane 0 adding 1 to its pool's counter takes that
// pool's next tile (a grab), lanes 0 .. kPools - 1 adding 0 to every counter
// read them all (a scan).  Inline asm keeps the compiler's atomic optimizer
// from broadcasting the result right away, which would wait for every load
// in flight; the instruction returns in issue order with the stage's loads,
// and the kernel reads k only after a wait that covers it (see the step).
// There is one such instruction in the loop and k is both its input and
// output, so that the compiler has no reason to copy the result register
// before that wait (a copy there reads it before the atomic has written
// it).  Not visible to the compiler's wait analysis, the instruction makes
// that analysis more cautious, never less.
__device__ __forceinline__ void counter_op(uint32_t *counters, bool on, int p, uint32_t v, uint32_t &k)
{
    if (on)
        asm volatile("global_atomic_add %0, %1, %2, off sc0"
                     : "+v"(k)
                     : "v"(counters + kCounterStride * p), "v"(v)
                     : "memory");
}

// Wait until at most kLater VMEM instructions are outstanding (every stage
// before the ones issued after the one to compute is complete), and only
// then let k be read.
__device__ __forceinline__ void wait_stage_and(uint32_t &k)
{
    // (the builtin, so that the compiler's own wait analysis knows of it)
    __builtin_amdgcn_s_waitcnt((((kLater >> 4) & 3) << 14) | 0x0f70 | (kLater & 15));
    asm volatile("" : "+v"(k) :: "memory");
}

// Group launches: take the result of the outstanding grab or counter read
// (readable: the caller has waited).  Index k of pool p is tile
// pool_tile(p, k) of the launch, and pool p has tiles left while that is
// below the launch's tile count (pool_tile grows with k).  A
// grab that found its pool empty reads every counter; the read picks the
// first pool with tiles left at or after the wave's own starting point (so
// that the waves of an emptied pool spread over the others) and grabs from
// it, or ends the wave.  Every grab and read moves the wave on: a pool's
// counter only grows, so the wave ends after finitely many.
// Index k of pool p: tile (k / C) kPools C + p C + k % C of the launch, C =
// kPoolChunk.
__device__ __forceinline__ uint32_t pool_tile(uint32_t p, uint32_t k)
{
    return (k / kPoolChunk) * (kPools * kPoolChunk) + p * kPoolChunk + k % kPoolChunk;
}

__device__ __forceinline__ void next_tile(Cursor &c, const RArgs &a, int lane, uint32_t &gv)
{
    if (c.state == kScan) {
        const bool open = lane < kPools && pool_tile((uint32_t)lane, gv) < (uint32_t)a.total_tiles;
        const uint32_t m = (uint32_t)__builtin_amdgcn_ballot_w64(open) & ((1u << kPools) - 1u);
        const uint32_t s = (uint32_t)c.rot;
        const uint32_t rm = ((m >> s) | (m << (kPools - s))) & ((1u << kPools) - 1u);  // pool s at bit 0
        c.pool = m != 0 ? (int32_t)(((uint32_t)__builtin_ctz(rm | (1u << kPools)) + s) & (uint32_t)(kPools - 1)) : c.pool;
        c.state = m != 0 ? kIdle : kDone;
    } else {
        const uint32_t t = pool_tile((uint32_t)c.pool, (uint32_t)uniform((int32_t)gv));
        if (t < (uint32_t)a.total_tiles) {
            const uint32_t e = a.lut[t];
            c.pi = (int32_t)(e >> 20);
            c.tile = (int32_t)(e & 0xfffffu);
            c.win = 0;
            c.state = kLive;
            load_prob<true>(c, a);
        } else {
            c.state = kScan;
        }
    }
    const bool scan = c.state == kScan;
    counter_op(a.counters, scan ? lane < kPools : c.state != kDone && lane == 0, scan ? lane : c.pool,
               scan ? 0u : 1u, gv);
}

// Inline launches: next window, next tile, next problem.
__device__ __forceinline__ void advance_inline(Cursor &c, const RArgs &a, int32_t &left)
{
    const int32_t win1 = c.win + 1;
    const int32_t wrap = win1 >= c.nwin ? 1 : 0;
    c.win = wrap ? 0 : win1;
    left -= wrap;
    const int32_t tile1 = c.tile + wrap;
    const int32_t wrap_t = tile1 >= c.tiles ? 1 : 0;
    c.tile = wrap_t ? 0 : tile1;
    c.pi += wrap_t;
    c.state = left > 0 ? kLive : kDone;
    load_prob<false>(c, a);
}

// What the compute side needs of a stage, recorded when the stage is issued.
struct Slot {
    float *y;       // the tile's first output row
    int32_t live;   // the stage holds work
    int32_t done;   // no stage after this one holds work
    int32_t type;
    int32_t pv;     // periods of the window in the row (lane rows g < pv count)
    int32_t last;   // the tile's last window
    int32_t nrows;  // rows of the tile that exist
};

// The chunk (0..67) of a tile row that slot 64 i + lane of a stage holds,
// or 68 for a pad slot or one past the last row.
__device__ __forceinline__ uint32_t slot_chunk(int i, int lane, uint32_t &row)
{
    if (i < kMainDma) {
        const uint32_t q = 64u * i + (uint32_t)lane;
        row = q / (uint32_t)kMainSlots;
        const uint32_t ck = q - (uint32_t)kMainSlots * row;
        return row < (uint32_t)kTileRows && ck < (uint32_t)kMainCk ? ck : 68u;
    }
    const uint32_t q = 64u * (i - kMainDma) + (uint32_t)lane;
    row = q / (uint32_t)kBndSlots;
    const uint32_t cc = q - (uint32_t)kBndSlots * row;
    return row < (uint32_t)kTileRows && cc < 8u ? (uint32_t)kMainCk + cc : 68u;
}

// Per-lane DMA offsets for row stride S (see slot_chunk); pad slots and
// slots past the last row get an out-of-range offset (they read nothing).
__device__ __forceinline__ void dma_offsets(uint32_t (&vo)[kDma], int32_t S, int lane)
{
#pragma unroll
    for (int i = 0; i < kDma; ++i) {
        uint32_t row;
        const uint32_t ck = slot_chunk(i, lane, row);
        vo[i] = ck < 68u ? row * (uint32_t)S + 16u * ck : 0x80000000u;
    }
}

// The cursor's window into a ring stage: kDma DMA instructions.  A cursor
// without a tile issues none with one stage per wave (kSkipIdle), and with
// two issues them on an empty buffer range (they read nothing and write
// zeros), so that every stage is exactly kDma + kXLoads VMEM instructions
// (issue_x below).  Chunks past the end of a row in a partial last window
// are given an out-of-range offset, so that nothing is read twice.  The
// instructions are issued in pieces (dma_part), set up once (dma_setup).
struct Dma {
    __amdgpu_buffer_rsrc_t wr;
    uint32_t soff;  // the window's byte offset in the tile's rows
    uint32_t nck;   // valid chunks per row
    bool on;        // the instructions are issued
};

__device__ __forceinline__ Dma dma_setup(const Cursor &c)
{
    // (readfirstlane: the resource must be in scalar registers, and the
    // compiler cannot always tell that these values are wave-uniform)
    const bool live = c.state == kLive;
    const int32_t rows_left = c.N - kTileRows * c.tile;
    const uint32_t rows = !live ? 0u : rows_left < kTileRows ? (uint32_t)rows_left : (uint32_t)kTileRows;
    const uint8_t *wbase = uniform_ptr(c.W + (size_t)(kTileRows * c.tile) * (size_t)c.S);
    Dma d;
    d.wr = make_rsrc(wbase, (uint32_t)uniform((int32_t)(rows * (uint32_t)c.S)));
    d.soff = (uint32_t)(c.win * kWindow);
    const int32_t pv = c.P - 4 * c.win;  // periods of this window in the row
    d.nck = pv >= 4 ? 68u : 17u * (uint32_t)pv;
    d.on = live || !kSkipIdle;
    return d;
}

template <int I0, int I1>
__device__ __forceinline__ void dma_part(const Dma &d, uint8_t *stage, const uint32_t (&vo)[kDma], int lane)
{
    if (!d.on) return;
#pragma unroll
    for (int i = I0; i < (I1 < kMainDma ? I1 : kMainDma); ++i) {
        uint32_t row;
        const uint32_t ck = slot_chunk(i, lane, row);
        const uint32_t off = ck < d.nck ? vo[i] : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.wr, (lds_void *)(stage + 1024 * i), 16, (int)off, (int)d.soff, 0,
                                                 2 /* nontemporal */);
    }
#pragma unroll
    for (int i = (I0 > kMainDma ? I0 : kMainDma); i < I1; ++i) {
        uint32_t row;
        const uint32_t ck = slot_chunk(i, lane, row);
        const uint32_t off = ck < d.nck ? vo[i] : 0x80000000u;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(d.wr, (lds_void *)(stage + 1024 * i), 16, (int)off, (int)d.soff, 0,
                                                 0 /* normal: kept for the next window */);
    }
}

__device__ __forceinline__ void issue_dma(const Cursor &c, uint8_t *stage, const uint32_t (&vo)[kDma], int lane)
{
    dma_part<0, kDma>(dma_setup(c), stage, vo, lane);
}

// The cursor's x for its window (lane (g, r): pairs 4r..4r+3 of each 64 of
// period 4w + g), and what the compute side needs to know of the stage.
__device__ __forceinline__ void issue_x(const Cursor &c, uint32_t xlane, u32x4 (&xs)[kXLoads], Slot &sl)
{
    const bool live = c.state == kLive;
    const uint32_t px = c.type == 0 ? 1280u : 1024u;  // x bytes per period
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(uniform_ptr(c.x), (uint32_t)uniform((int32_t)(live ? (uint32_t)c.P * px : 0u)));
    const uint32_t xsoff = 4u * (uint32_t)c.win * px;
    if (live || !kSkipIdle) {
#pragma unroll
        for (int i = 0; i < kXLoads; ++i)
            xs[i] = __builtin_bit_cast(u32x4,
                                       __builtin_amdgcn_raw_buffer_load_b128(xr, (int)(xlane + 256u * i), (int)xsoff, 0));
    }
    sl.y = c.y + kTileRows * c.tile;
    sl.live = live ? 1 : 0;
    sl.done = c.state == kDone ? 1 : 0;
    sl.type = c.type;
    sl.pv = live ? c.P - 4 * c.win : 0;
    sl.last = live && c.win == c.nwin - 1 ? 1 : 0;
    sl.nrows = c.N - kTileRows * c.tile;
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
    __shared__ uint32_t wg_done;  // group launches: waves of this workgroup that have finished
    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int gw = blockIdx.x * kRWaves + wave;
    const int g = lane >> 4, r = lane & 15;
    if constexpr (TABLE) {
        if (threadIdx.x == 0) wg_done = 0;
        __syncthreads();
    }
    uint8_t *ring = lds + wave * kNS * kStage;

    Cursor ci;
    ci.win = 0;
    ci.state = kIdle;
    ci.rot = gw & (kPools - 1);
    int32_t left = 0;  // inline launches: tiles left
    uint32_t gv = 0;   // lane 0: result of the outstanding grab
    if constexpr (TABLE) {
        // home pool: workgroups go to the XCDs in turn (blockIdx % 8), and a
        // pool serves half of an XCD's CUs
        ci.pool = (int)((blockIdx.x & 7) * 2 + ((blockIdx.x >> 3) & 1)) % kPools;
        counter_op(a.counters, lane == 0, ci.pool, 1u, gv);
        asm volatile("s_waitcnt vmcnt(0)" : "+v"(gv) :: "memory");
        next_tile(ci, a, lane, gv);
    } else {
        const int nw = gridDim.x * kRWaves;
        const int t0 = (int)((int64_t)a.total_tiles * gw / nw);
        const int t1 = (int)((int64_t)a.total_tiles * (gw + 1) / nw);
        ci.pi = t0 >= a.p0.tiles ? 1 : 0;
        ci.tile = t0 - (ci.pi ? a.p0.tiles : 0);
        left = t1 - t0;
        ci.state = left > 0 ? kLive : kDone;
        load_prob<false>(ci, a);
    }
    // Next window.  A group cursor leaving its tile, or without one, takes
    // the grabbed tile (gv must be readable: the caller has waited).
    auto advance = [&]() {
        if constexpr (TABLE) {
            if (ci.state == kIdle || ci.state == kScan || (ci.state == kLive && ++ci.win >= ci.nwin))
                next_tile(ci, a, lane, gv);
        } else {
            advance_inline(ci, a, left);
        }
    };

    if (ci.state != kDone) {
        uint32_t vo[kDma];
        int32_t vo_s = ci.S;
        dma_offsets(vo, vo_s, lane);
        const uint32_t xl3 = (uint32_t)(16 * r + 1280 * g), xl4 = (uint32_t)(16 * r + 1024 * g);

        u32x4 xs0[kXLoads], xs1[kXLoads];
        Slot sl0, sl1;
        issue_dma(ci, ring, vo, lane);
        issue_x(ci, ci.type == 0 ? xl3 : xl4, xs0, sl0);
        if constexpr (kNS == 2) {
            // the second stage (each step starts by moving the cursor on)
            if constexpr (TABLE) wait_stage_and(gv);  // the grab is older than stage 0
            advance();
            asm volatile("" ::: "memory");  // keep the two stages' loads in issue order
            if (ci.S != vo_s) {
                vo_s = ci.S;
                dma_offsets(vo, vo_s, lane);
            }
            issue_dma(ci, ring + kStage, vo, lane);
            issue_x(ci, ci.type == 0 ? xl3 : xl4, xs1, sl1);
        }
        float acc = 0.0f;
        // A finished tile's sums are stored at the start of the next step,
        // ahead of that step's loads, so that the wait for those loads does
        // not also wait for the store to be acknowledged.
        // (per lane, in VGPRs: scalar registers are all taken)
        float pend_v = 0.0f;
        float *pend_a = nullptr;  // this lane's output, if it stores one
        int32_t pend = 0;

        // One step.  The stage in ring slot `stage` has landed (and so has any
        // grab issued before the later stages): move the issue cursor on, read
        // the lane's period into registers, and as soon as the reads are done
        // refill the slot with the issue cursor's window, so that windows are
        // in flight while this one is computed.  With two stages per wave the
        // cursor's x goes into xs once this stage's x is no longer needed;
        // with one, into the other register set (xn, sn) right away.  A stage
        // without work computes zeros and stores nothing.
        auto step = [&](uint8_t *stage, u32x4 (&xs)[kXLoads], Slot &sl, u32x4 (&xn)[kXLoads], Slot &sn) {
            wait_stage_and(gv);
            advance();
            // The cursor's scalar loads land before the period reads are
            // issued: scalar loads return out of order and share lgkmcnt
            // with LDS reads, so one still in flight would make the first
            // use of D wait for all 17 reads.
            wait_lds_reads();
            uint32_t D[68];
            if constexpr (PN_ROWS_BND) {
                const uint8_t *lo = stage + 16 * (kMainSlots * r + 17 * g);
                const uint8_t *hi = g == 3 ? stage + 1024 * kMainDma + 16 * (kBndSlots * r - 9) : lo;
                load_period2(lo, hi, D);
            } else {
                load_period(stage + r * kRowLds + g * kPeriod, D);
            }
            if (pend) *pend_a = pend_v;
            pend = 0;
            float it = 0.0f;
            if (PN_ROWS_SPLIT && sl.live) {
                // the first block pair's products while the other reads land
                if (sl.type == 0)
                    period_dot<0, 0, 1>(D, xs, it);
                else
                    period_dot<1, 0, 1>(D, xs, it);
            }
            wait_lds_reads();
            if (ci.S != vo_s) {
                vo_s = ci.S;
                dma_offsets(vo, vo_s, lane);
            }
            // The refill, in PN_ROWS_SPREAD pieces between the remaining
            // block pairs (sched_barrier keeps the compiler from gathering
            // them again); a stage without work computes nothing.
            const Dma dm = dma_setup(ci);
            constexpr int kPiece = (kDma + PN_ROWS_SPREAD - 1) / PN_ROWS_SPREAD;
            dma_part<0, kPiece>(dm, stage, vo, lane);
            if constexpr (kNS == 1) issue_x(ci, ci.type == 0 ? xl3 : xl4, xn, sn);
            __builtin_amdgcn_sched_barrier(0);
            static_for<PN_ROWS_SPLIT, 4>([&](auto bpc) {
                constexpr int bp = decltype(bpc)::value;
                if (sl.live) {
                    if (sl.type == 0)
                        period_dot<0, bp, bp + 1>(D, xs, it);
                    else
                        period_dot<1, bp, bp + 1>(D, xs, it);
                }
                constexpr int k = bp - PN_ROWS_SPLIT + 1;  // pieces issued after this block pair
                if constexpr (k < PN_ROWS_SPREAD) {
                    __builtin_amdgcn_sched_barrier(0);
                    dma_part<(k * kPiece < kDma ? k * kPiece : kDma), ((k + 1) * kPiece < kDma ? (k + 1) * kPiece : kDma)>(
                        dm, stage, vo, lane);
                    __builtin_amdgcn_sched_barrier(0);
                }
            });
            acc += g < sl.pv ? it : 0.0f;
            if (sl.last) {
                // the tile is done: add the four DPP rows' sums of each row
                auto s32 = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc), __float_as_uint(acc), false, false);
                float v = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
                auto s16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
                v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
                pend_v = v;
                pend_a = sl.y + r;
                pend = g == 0 && r < sl.nrows;
                acc = 0.0f;
            }
            if constexpr (kNS == 2) {
                asm volatile("" ::: "memory");  // this stage's x loads after its DMA, in issue order
                issue_x(ci, ci.type == 0 ? xl3 : xl4, xs, sl);
            }
        };
        // A wave's steps are its windows, grabs and scans, all bounded in a
        // correct run (pool counters only grow); the cap ends the loop all the
        // same if the counters were disturbed, e.g. by a plan run concurrently
        // with itself, so that the launch ends with wrong sums instead of
        // never ending.
        int32_t steps = 0;
        for (;;) {
            if (sl0.done || (steps += 2) > a.step_cap) break;
            step(ring, xs0, sl0, xs1, sl1);
            if (sl1.done) break;
            step(ring + (kNS - 1) * kStage, xs1, sl1, xs0, sl0);
        }
        if (pend) *pend_a = pend_v;
    }
    // no DMA (or grab) may still be in flight when the wave ends
    asm volatile("s_waitcnt vmcnt(0)" : "+v"(gv) :: "memory");
    if constexpr (TABLE) {
        // The last wave to finish resets the plan's counters for its next run.
        // The waves of a workgroup count themselves in LDS, and the last of
        // them counts the workgroup in the plan's device counter: 256 device
        // atomics on that address per launch instead of 2,048.  Relaxed
        // ordering is enough: every wave has waited for its own counter
        // atomics (vmcnt(0) above) before it counts itself done, each count
        // depends on the one before it, the reset depends on the count the
        // last atomic returns, and the kernel's end publishes the reset to the
        // next launch.  (Acquire-release ordering at agent scope made every
        // wave write back and invalidate its L2 as it finished: about 100 us
        // per launch of a small plan, 2,048 L2 flushes under the waves still
        // streaming.)
        if (lane == 0 &&
            __hip_atomic_fetch_add(&wg_done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) == kRWaves - 1) {
            uint32_t *done = a.counters + kCounterStride * kPools;
            if (__hip_atomic_fetch_add(done, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == gridDim.x - 1) {
                for (int p = 0; p < kPools; ++p)
                    __hip_atomic_store(a.counters + kCounterStride * p, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(done, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Host side
// ---------------------------------------------------------------------------
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
    return hipFuncSetAttribute((const void *)gemv_rows<true>, hipFuncAttributeMaxDynamicSharedMemorySize, kRing) ==
               hipSuccess &&
           hipFuncSetAttribute((const void *)gemv_rows<false>, hipFuncAttributeMaxDynamicSharedMemorySize, kRing) ==
               hipSuccess;
}

// A batch plan written by a kernel (pn_gemv_batch): the problems travel in
// the kernel arguments, sorted longest rows first, with the first tile of
// each in the hand-out order; the kernel writes the problem table, the tile
// order (as rows_group_create lays it out) and zeroed pool counters into
// the batch buffer.
struct RBatch {
    RProb p[kBatchMaxProblems];
    int32_t first[kBatchMaxProblems + 1];
    int32_t count;
    int32_t total;
};
static_assert((kPools + 1) * kCounterStride * sizeof(uint32_t) <= kBatchCounterBytes, "batch counters");
static_assert(kBatchMaxProblems * sizeof(RProb) <= kBatchTableBytes, "batch table");
static_assert(sizeof(RBatch) <= 2048, "batch kernel arguments");

__global__ __launch_bounds__(256) void rows_batch_setup(RBatch b, uint8_t *buf)
{
    const int tid = blockIdx.x * 256 + threadIdx.x;
    const int stride = gridDim.x * 256;
    RProb *table = (RProb *)(buf + kBatchTableOff);
    if (tid < b.count) table[tid] = b.p[tid];
    uint32_t *lut = (uint32_t *)(buf + kBatchLutOff);
    for (int t = tid; t < b.total; t += stride) {
        int i = 0;
        while (i + 1 < b.count && b.first[i + 1] <= t) ++i;
        lut[t] = ((uint32_t)i << 20) | (uint32_t)(t - b.first[i]);
    }
    uint32_t *counters = (uint32_t *)buf;
    for (int j = tid; j < (int)(kBatchCounterBytes / 4); j += stride) counters[j] = 0u;
}

// More steps than any wave of a correct launch takes: every window of the
// launch, a grab or scan per tile and per pool, and the pipeline's ends.
int32_t step_cap(int64_t total_tiles, int maxwin)
{
    const int64_t c = total_tiles * (int64_t)(maxwin + 2) + 2 * kPools + 8;
    return c < INT32_MAX ? (int32_t)c : INT32_MAX;
}

pn_status rlaunch(const RArgs &a, hipStream_t s, int variant)
{
    if (!once_per_device(kAttrRows, set_rows_attr)) return PN_ELAUNCH;
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
    if (gemv_kernel_choice() == PN_GEMV_STREAM) return false;
    if (((uintptr_t)W & 15) != 0 || ((uintptr_t)x & 15) != 0) return false;
    const int64_t nb = K / wpb(t);
    if (nb % 8 != 0) return false;
    return nb * 34 <= ((int64_t)1 << 24);  // row bytes: 16 rows x row bytes < 2^28
}

// Is a launch of `tiles` 16-row tiles large enough for gemv_rows?
bool pn::host::rows_pays(int64_t tiles)
{
    if (gemv_kernel_choice() == PN_GEMV_ROWS) return true;
    return tiles >= (int64_t)kMinTilesPerCu * device_cus();
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
    a.step_cap = step_cap(a.total_tiles, a.p0.nwin);
    return rlaunch(a, s, kVarRows);
}

pn_status pn::host::rows_group_create(const pn_gemv_desc *descs, int count, pn_group **out)
{
    *out = nullptr;
    if (count > 4096) return PN_EUNSUPPORTED;  // the tile table packs 12 bits of problem
    RProb *host = (RProb *)calloc((size_t)count, sizeof(RProb));
    if (!host) return PN_ENOMEM;
    int64_t total = 0;
    int maxwin = 0;
    for (int i = 0; i < count; ++i) {
        const pn_gemv_desc &e = descs[i];
        rfill(host[i], e.type, e.W, e.N, e.K, e.x, e.y);
        if (host[i].tiles > (1 << 20)) {  // and 20 bits of tile
            free(host);
            return PN_EUNSUPPORTED;
        }
        total += host[i].tiles;
        if (host[i].nwin > maxwin) maxwin = host[i].nwin;
    }
    if (total >= INT32_MAX) {
        free(host);
        return PN_EUNSUPPORTED;
    }
    // The plan: problems, the launch's tiles in the order they are handed out
    // (longest first, so that the last tiles of a run are short ones; pool p
    // takes chunks p, p + kPools, ... of kPoolChunk of them), and the pools'
    // counters and the count of finished waves, 4 KiB apart.
    const size_t tbytes = sizeof(RProb) * (size_t)count;
    const size_t lbytes = sizeof(uint32_t) * (size_t)total;
    const size_t cbytes = sizeof(uint32_t) * kCounterStride * (kPools + 1);
    const size_t loff = tbytes, coff = (tbytes + lbytes + 4095) & ~(size_t)4095;
    uint8_t *blob = (uint8_t *)calloc(1, coff + cbytes);
    pn_group *g = (pn_group *)calloc(1, sizeof(pn_group));
    if (!g || !blob) {
        free(host);
        free(blob);
        free(g);
        return PN_ENOMEM;
    }
    memcpy(blob, host, tbytes);
    uint32_t *lut = (uint32_t *)(blob + loff);
    size_t k = 0;
    for (int w = maxwin; w >= 1; --w)
        for (int i = 0; i < count; ++i)
            if (host[i].nwin == w)
                for (int t = 0; t < host[i].tiles; ++t) lut[k++] = ((uint32_t)i << 20) | (uint32_t)t;
    free(host);
    if (current_device() < 0) {
        free(blob);
        free(g);
        return PN_EUNSUPPORTED;
    }
    if (hipMalloc(&g->table, coff + cbytes) != hipSuccess) {
        free(blob);
        free(g);
        return PN_ENOMEM;
    }
    if (hipMemcpy(g->table, blob, coff + cbytes, hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(g->table);
        free(blob);
        free(g);
        return PN_ELAUNCH;
    }
    free(blob);
    g->kind = kGroupGemvRows;
    g->device = current_device();
    g->count = count;
    g->total_tiles = (int)total;
    g->max_win = maxwin;
    g->lds = kRing;
    g->flags = (int)coff;  // byte offset of the counters
    *out = g;
    return PN_OK;
}

pn_status pn::host::rows_group_run(const pn_group *g, hipStream_t s)
{
    RArgs a;
    memset(&a, 0, sizeof(a));
    a.table = (const PN_CONST RProb *)g->table;
    a.lut = (const PN_CONST uint32_t *)((const uint8_t *)g->table + sizeof(RProb) * (size_t)g->count);
    a.counters = (uint32_t *)((uint8_t *)g->table + g->flags);
    a.count = g->count;
    a.total_tiles = g->total_tiles;
    a.step_cap = step_cap(g->total_tiles, g->max_win);
    return rlaunch(a, s, kVarGroupRows);
}

pn_status pn::host::rows_batch_launch(const pn_gemv_desc *descs, int count, uint8_t *buf, hipStream_t s)
{
    if (count < 1 || count > kBatchMaxProblems) return PN_EUNSUPPORTED;
    RBatch b;
    memset(&b, 0, sizeof(b));
    int order[kBatchMaxProblems];
    int maxwin = 0;
    RProb p[kBatchMaxProblems];
    for (int i = 0; i < count; ++i) {
        const pn_gemv_desc &e = descs[i];
        rfill(p[i], e.type, e.W, e.N, e.K, e.x, e.y);
        if (p[i].nwin > maxwin) maxwin = p[i].nwin;
    }
    // longest rows first, as rows_group_create orders the tiles
    int n = 0;
    for (int w = maxwin; w >= 1; --w)
        for (int i = 0; i < count; ++i)
            if (p[i].nwin == w) order[n++] = i;
    int64_t total = 0;
    for (int j = 0; j < count; ++j) {
        b.p[j] = p[order[j]];
        b.first[j] = (int32_t)total;
        total += b.p[j].tiles;
    }
    if (total > kBatchMaxTiles) return PN_EUNSUPPORTED;
    b.first[count] = (int32_t)total;
    b.count = count;
    b.total = (int32_t)total;
    const int grid = (int)((total + 255) / 256) < 64 ? (int)((total + 255) / 256) : 64;
    hipLaunchKernelGGL(rows_batch_setup, dim3((unsigned)(grid > 0 ? grid : 1)), dim3(256), 0, s, b, buf);
    if (hipGetLastError() != hipSuccess) return PN_ELAUNCH;
    RArgs a;
    memset(&a, 0, sizeof(a));
    a.table = (const PN_CONST RProb *)(buf + kBatchTableOff);
    a.lut = (const PN_CONST uint32_t *)(buf + kBatchLutOff);
    a.counters = (uint32_t *)buf;
    a.count = count;
    a.total_tiles = (int32_t)total;
    a.step_cap = step_cap(total, maxwin);
    return rlaunch(a, s, kVarBatchRows);
}
